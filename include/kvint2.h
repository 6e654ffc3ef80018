/*
 * kvint2 -- 2-bit KV cache for MI355X (gfx950): quantize-append into a
 * packed INT2 cache, and attention read directly from the packed cache.
 *
 * C ABI.  Every pointer argument named *_dev is device memory on the
 * current HIP device; `stream` is a hipStream_t passed as void* (NULL = the
 * default stream).  All calls only enqueue work on `stream` and return; a
 * return of KVQ_OK means "enqueued", not "finished".  The library allocates
 * nothing and keeps no state between calls (apart from the fixed scratch
 * buffer of attn_int2_decode_noalloc), and is safe to call from several
 * host threads.  Every argument is checked on the host before anything is
 * launched: on any status other than KVQ_OK and KVQ_EHIP nothing was
 * launched and no output was touched.
 *
 * Methods (web pages, cited by title and section):
 *  [QWM]  "QuantWM: Training-Free 2-bit KV Cache Quantization for Stable
 *         Video World Models" -- "QuantWM Framework": 1. QSAC (centroid +
 *         INT2 residual keys, sensitivity-aware centroid choice), 2. PSAC
 *         (low-rank compensation of the key error along principal query
 *         directions); "System Implementation" (compressed cache).
 *  [OKV]  "OmniKVQuant: KV Cache Quantization for Omni-LLMs" -- English
 *         abstract: key ranges per short window of the stream, rotated
 *         values, a decode kernel that unpacks the 2-bit cache inside
 *         attention without building a dense cache.
 *  [WUSH] "WUSH-KV Applies Data-Adaptive Transforms to KV Cache
 *         Quantization" -- affine low-bit quantizer.
 *
 * Number formats and rounding (the pages fix none of them):
 *  - INT2 group quantizer over a group x_0..x_{n-1} (32 channels of one
 *    token, or 64 tokens of one channel): inputs canonicalised x + 0.0f,
 *    s = fp16((max - min) / 3) and z = fp16(min) with fp32 subtraction and
 *    correctly rounded fp32 division, fp16 round-to-nearest-even; with
 *    s, z the stored values widened to fp32, code = [x >= fma(.5,s,z)] +
 *    [x >= fma(1.5,s,z)] + [x >= fma(2.5,s,z)] (round half up to the
 *    nearest stored level), or 0 for every element when s == 0.
 *    Dequantised value: code * s + z.
 *  - Packing: 4 codes per byte, 2 bits each, lowest position in the lowest
 *    bits (codes 0,1,2,3 pack to 0xE4): key codes by token row (channel 4j+t
 *    in byte j), value codes by channel within 64-token tiles (see v_codes).
 *  - A parameter word is 32 bits: fp16 scale in the low half, fp16 zero in
 *    the high half.
 */
#ifndef KVINT2_H
#define KVINT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status */
enum {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,       /* null pointer, bad enum, bad size or alignment */
  KVQ_EUNSUPPORTED = -2, /* valid but not built (e.g. head_dim 96)        */
  KVQ_ECAPACITY = -3,    /* tokens beyond the cache capacity              */
  KVQ_EWORKSPACE = -4,   /* workspace missing or too small                */
  KVQ_EHIP = -5,         /* the HIP runtime reported an error at launch   */
  KVQ_ESCRATCH = -6      /* needs more than the fixed scratch buffer of
                            attn_int2_decode_noalloc                      */
};

/* ------------------------------------------------------------ modes */
enum {
  /* [OKV]: per (64-token window, channel) min/max over a window aligned to
   * absolute stream position; tokens of the unfinished last window are kept
   * verbatim in a bf16 tail until the window completes. */
  KVQ_KEY_WINDOW = 0,
  /* [QWM] 1 (the centroid + residual scheme it starts from): key k goes to
   * its nearest fp32 centroid j (fp32 squared distance accumulated in
   * channel order with fma, ties to the lowest index) and the residual
   * k - C_j is INT2-quantised per token in groups of 32 channels. */
  KVQ_KEY_CENTROID = 1,
  /* [QWM] 1, QSAC: the qsac_topk nearest centroids under the weighted
   * distance sum_d fma(w_d t_d, t_d) are candidates; each candidate's
   * residual is INT2-quantised and the one with the smallest weighted
   * squared residual error sum_d fma(w_d e_d, e_d) is kept (ties: lowest
   * index).  w are the query-sensitivity weights (sens_w). */
  KVQ_KEY_CENTROID_QSAC = 2
};

enum {
  KVQ_VAL_GROUP = 0,    /* values INT2 per token in groups of 32 channels */
  /* [OKV] rotated values: the orthonormal Walsh-Hadamard transform of size
   * head_dim (Sylvester order, stages 1,2,4,.. in fp32, then times
   * fp32(1/sqrt(head_dim))) is applied before quantisation; attention
   * outputs are rotated back. */
  KVQ_VAL_HADAMARD = 1,
  /* [OKV] values rotated separately per modality: token t of modality
   * m = v_modality[b][t] is rotated by R_m = diag(sigma_m) H, H the
   * Walsh-Hadamard transform above and sigma_m in {+1,-1}^head_dim the
   * sign vector of (kv head, modality m) in v_signs; i.e. the rotated row
   * of the KVQ_VAL_HADAMARD mode with the channels whose sign is -1
   * negated.  Attention rotates back with R_m^T = H diag(sigma_m).  With
   * every sign +1 this is KVQ_VAL_HADAMARD. */
  KVQ_VAL_HADAMARD_MODAL = 2
};

/* QSAC perturbation estimate (kvq_layout.qsac_score) */
enum {
  /* the candidate's actual weighted INT2 residual error, as above */
  KVQ_QSAC_EXACT = 0,
  /* [QWM] 1 reads as an estimate from the residual groups' dynamic range
   * and the query sensitivity: E = sum over groups g, in order, of
   * fma(s_g * s_g, W_g, E), s_g the fp16 step the quantizer would store for
   * the candidate's residual group ((max - min) / 3 rounded to fp16), W_g
   * the fp32 sum of w over the group's channels in channel order (INT2
   * rounding noise has variance s^2/12 per element; the common 1/12 is
   * left out).  No residual codes are needed to rank candidates. */
  KVQ_QSAC_RANGE = 1
};

/* PSAC coefficient storage (kvq_layout.psac_format) */
enum {
  KVQ_PSAC_F16 = 0,   /* a_m as fp16 */
  /* [QWM] 2 stores the coefficients as INT8: per token one fp16 scale
   * sc = fp16(max_m |a_m| / 127) and q_m = a_m / sc rounded to nearest
   * (ties to even), clamped to [-127, 127] (all 0 when sc is 0); the
   * coefficient used is q_m * sc.  10 bytes per token-head instead of 16. */
  KVQ_PSAC_INT8 = 1
};

enum { KVQ_F32 = 0, KVQ_BF16 = 1 };

#define KVQ_GROUP 32  /* channels per value / residual parameter group */
#define KVQ_WINDOW 64 /* tokens per key-range window                   */

/* ------------------------------------------------------------ layout */
typedef struct kvq_layout {
  int32_t batch;       /* sequences B                                  */
  int32_t kv_heads;    /* KV heads H                                   */
  int32_t head_dim;    /* D: 64 or 128                                 */
  int32_t capacity;    /* Tcap tokens per sequence, a multiple of 64,
                          at most 2^24                                 */
  int32_t key_mode;    /* KVQ_KEY_*                                    */
  int32_t value_mode;  /* KVQ_VAL_*                                    */
  int32_t n_centroids; /* C, 1..256 (centroid modes; else ignored)     */
  int32_t qsac_topk;   /* QSAC candidates, 1..8 and <= C (QSAC only)   */
  int32_t psac_rank;   /* R: 0 (off) or 8 -- [QWM] 2 uses 8 directions;
                          centroid modes only                          */
  int32_t qsac_score;  /* KVQ_QSAC_* (QSAC only; else ignored)         */
  int32_t psac_format; /* KVQ_PSAC_* (psac_rank > 0; else ignored)     */
  int32_t centroid_key_split; /* 0 or 1, accepted and ignored: chunk
                         attention enters every centroid key as fp16
                         hi + lo (kept for layout compatibility)       */
  int32_t n_modalities; /* M, 1..3 (KVQ_VAL_HADAMARD_MODAL; else ignored) */
} kvq_layout;

/* Device buffers of one layer's packed cache.  Shapes are C order.
 *   k_codes    u8  [B][H][Tcap][D/4]   packed key codes (window keys, or
 *                                      centroid residuals)
 *   k_params   u32 window:   [B][H][Tcap/64][D]  per (window, channel)
 *                  centroid: [B][H][Tcap][D/32]  per (token, group)
 *   k_tail     u16 [B][H][64][D]       bf16 keys of the unfinished window
 *                                      at slot position % 64 (window mode)
 *   k_idx      u8  [B][H][Tcap]        centroid index (centroid modes)
 *   centroids  f32 [B][H][C][D]        caller-filled calibration input
 *   sens_w     f32 [B][H][D]           caller-filled (QSAC)
 *   psac_basis f32 [B][H][D][R]        caller-filled (PSAC): orthonormal
 *                                      principal query directions
 *   k_psac     u16 [B][H][Tcap][R]     fp16 PSAC coefficients
 *                                      a_m = fp16(sum_d fma(U_dm, e_d)),
 *                                      e = residual - dequantised residual;
 *              with KVQ_PSAC_INT8:     i8 [B][H][Tcap][R] codes q_m, then
 *                                      u16 [B][H][Tcap] fp16 scales
 *                                      (B*H*Tcap*(R+2) bytes in all)
 *   v_codes    u8  [B][H][Tcap/64][D][16]  value codes per 64-token tile,
 *                                      channel-major: token t of the tile,
 *                                      channel c in byte 16c + t/4, bits
 *                                      [2(t%4), 2(t%4)+1] -- a channel's 64
 *                                      codes are contiguous, as the
 *                                      token-axis reduction of P.V reads them
 *   v_params   u32 [B][H][Tcap][D/32]
 *   v_signs    u32 [H][M][D/32]        caller-filled (KVQ_VAL_HADAMARD_MODAL):
 *                                      sigma of (head h, modality m), bit
 *                                      c % 32 of word c / 32 set = -1
 *   v_modality u8  [B][Tcap]           caller-filled (KVQ_VAL_HADAMARD_MODAL):
 *                                      modality (0..M-1) of each token, written
 *                                      before the token is appended and kept
 *                                      (an id >= M is read as M - 1)
 * Buffers a mode does not use may be NULL.  Rows of tokens in an
 * unfinished window and tail slots at or beyond (length % 64) hold
 * unspecified bytes (for values: the bits of tokens at or beyond the length in
 * its 64-token tile).  All buffers must be 16-byte aligned. */
typedef struct kvq_cache {
  kvq_layout layout;
  void* k_codes;
  void* k_params;
  void* k_tail;
  void* k_idx;
  const void* centroids;
  const void* sens_w;
  const void* psac_basis;
  void* k_psac;
  void* v_codes;
  void* v_params;
  const void* v_signs;
  const void* v_modality;
} kvq_cache;

enum {
  KVQ_BUF_K_CODES = 0,
  KVQ_BUF_K_PARAMS,
  KVQ_BUF_K_TAIL,
  KVQ_BUF_K_IDX,
  KVQ_BUF_CENTROIDS,
  KVQ_BUF_SENS_W,
  KVQ_BUF_PSAC_BASIS,
  KVQ_BUF_K_PSAC,
  KVQ_BUF_V_CODES,
  KVQ_BUF_V_PARAMS,
  KVQ_BUF_V_SIGNS,
  KVQ_BUF_V_MODALITY,
  KVQ_BUF_COUNT
};

/* Bytes buffer `which` (KVQ_BUF_*) needs under layout L; 0 when the mode
 * does not use it or L is invalid.  Host only, no device access. */
size_t kvq_buffer_bytes(const kvq_layout* L, int32_t which);

/* Checks a layout; returns KVQ_OK, KVQ_EINVAL or KVQ_EUNSUPPORTED
 * (head_dim, centroid count or PSAC rank not built; batch or kv_heads above
 * 65535 or capacity above 2^24, the limits of the launch grids and of the
 * 32-bit row offsets inside one (sequence, head)). */
int kvq_layout_check(const kvq_layout* L);

/* ------------------------------------------------------------ append */
/* Quantise tokens [cur_len, cur_len + n_new) of every sequence into the
 * cache ([QWM] 1 and 2, [OKV] windows and rotated values).
 * k_bf16_dev, v_bf16_dev: bf16 [B][n_new][H][D] (the new tokens).
 * Keys and values must be finite: a NaN or an infinity gives unspecified
 * codes and parameters for its group.
 * Window keys: every window completed by this append is quantised per
 * channel from the tail and the new tokens; the tokens of the window left
 * unfinished are written to the tail.  The cache bytes depend on the token
 * sequence only, not on how it was split into appends.
 * The library keeps no length: the caller passes it.  With window keys,
 * cur_len must be the number of tokens appended so far, or a multiple of
 * 64 below it (a rewind to a window boundary, after which the later tokens
 * are overwritten): the append completes the unfinished window from the
 * tail, which holds the tokens of the last window only.
 * Errors: KVQ_EINVAL (null buffer a mode needs, cur_len < 0, n_new < 0),
 * KVQ_ECAPACITY (cur_len + n_new > capacity). n_new == 0 is a no-op. */
int kv_quantize_append(const kvq_cache* cache, const void* k_bf16_dev,
                       const void* v_bf16_dev, int32_t cur_len, int32_t n_new,
                       void* stream);

/* ------------------------------------------------------------ assign */
/* Centroid index of each key ([QWM] 1): key i is the bf16 vector at
 * keys_bf16_dev + i * key_stride elements (head_dim contiguous elements).
 * centroids_dev f32 [n_centroids][head_dim].  sens_w_dev NULL: nearest
 * centroid (the KVQ_KEY_CENTROID rule); non-NULL f32 [head_dim]: QSAC
 * with `topk` candidates (the KVQ_KEY_CENTROID_QSAC rule).
 * idx_out_dev i32 [n].  Errors: KVQ_EINVAL (n < 0, nulls, key_stride <
 * head_dim, topk outside 1..8 with weights), KVQ_EUNSUPPORTED (head_dim
 * not 64/128, n_centroids outside 1..256). */
int kv_cluster_assign(const void* keys_bf16_dev, int64_t n, int32_t head_dim,
                      int64_t key_stride, const float* centroids_dev,
                      int32_t n_centroids, const float* sens_w_dev,
                      int32_t topk, int32_t* idx_out_dev, void* stream);

/* ------------------------------------------------------------ k-means */
/* Lloyd k-means of the keys of each (sequence, head) ([QWM] 1: the cluster
 * centres come from clustering keys; a calibration step before the hot
 * path), giving the per-(sequence, kv head) centroid tables of a
 * centroid-key cache.  Each of `iters` rounds assigns every key with the
 * KVQ_KEY_CENTROID rule of kv_cluster_assign and then sets each centroid to
 * the f32 value of the fp64 mean of its members, summed in key order; a
 * centroid without members keeps its value.  Key i of head h of sequence b
 * is the bf16 vector (head_dim contiguous elements) at keys_bf16_dev +
 * b * batch_stride + i * key_stride + h * head_stride elements (the
 * append input [B][n][H][D] has key_stride H*D, head_stride D, batch_stride
 * n*H*D).  centroids_dev f32 [batch][heads][n_centroids][head_dim]: read as
 * the starting tables, overwritten with the result.  assign_out_dev i32
 * [batch][heads][n] (nullable): the last round's assignment (with iters ==
 * 0, the assignment to the starting tables).  ws_dev: at least
 * kv_kmeans_workspace(batch, heads, n) bytes of device memory, 256-byte
 * aligned, in use until the stream passes the call (it holds the
 * assignment and the member lists of the rounds).  All work is enqueued on `stream`.  Errors:
 * KVQ_EINVAL (negative sizes or strides, iters < 0, nulls, misaligned
 * pointers, key_stride < head_dim), KVQ_EUNSUPPORTED (head_dim not 64/128,
 * n_centroids outside 1..256, batch or heads above 65535), KVQ_EWORKSPACE
 * (missing or short ws). */
size_t kv_kmeans_workspace(int32_t batch, int32_t heads, int64_t n);
int kv_kmeans(const void* keys_bf16_dev, int32_t batch, int64_t n, int32_t heads,
              int32_t head_dim, int64_t key_stride, int64_t head_stride, int64_t batch_stride,
              float* centroids_dev, int32_t n_centroids, int32_t iters,
              int32_t* assign_out_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ decode */
/* Workspace bytes attn_int2_decode needs for these sizes. */
size_t attn_int2_decode_workspace(const kvq_layout* L, int32_t q_heads,
                                  int32_t n_tokens);

/* One query token per sequence against the first n_tokens cached tokens,
 * read straight from the packed cache ([OKV]: the 2-bit cache is unpacked
 * inside attention; no dense cache is built).  q_dev [B][q_heads][D] in
 * q_dtype (KVQ_F32 or KVQ_BF16); query head h reads kv head
 * h / (q_heads / H).  out_dev [B][q_heads][D] in out_dtype, rotated back
 * to the input basis for the rotated value modes; lse_dev (nullable) f32
 * [B][q_heads] = log sum_t exp(scale * logit_t).  Logits include the PSAC
 * term (U^T q) . a_t when psac_rank > 0.  No mask.  ws_dev: scratch of
 * attn_int2_decode_workspace() bytes.
 * With window keys the tokens of an unfinished window are read from the
 * tail, which holds the last window of the appended sequence only: n_tokens
 * must be the number of tokens appended so far, or a multiple of 64 not
 * above it (a prefix of whole windows).
 * Errors: KVQ_EINVAL (nulls, q_heads not a multiple of H, n_tokens < 1),
 * KVQ_EUNSUPPORTED (q_heads / H not in {1,2,4,8}, q_heads above 65535),
 * KVQ_ECAPACITY (n_tokens > capacity), KVQ_EWORKSPACE. */
int attn_int2_decode(const kvq_cache* cache, int32_t n_tokens,
                     const void* q_dev, int32_t q_dtype, int32_t q_heads,
                     float scale, void* out_dev, int32_t out_dtype,
                     float* lse_dev, void* ws_dev, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------ no-alloc */
/* attn_int2_decode for callers that cannot allocate device memory or pass
 * a workspace: code under stream capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, kernels, results and errors as
 * attn_int2_decode without ws_dev/ws_bytes: the split partials go to a
 * fixed scratch buffer of KVQ_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each device it runs on until the process ends (its address is
 * looked up on the first call on a device).  Calls whose partials need
 * more (attn_int2_decode_workspace() > KVQ_NOALLOC_SCRATCH_BYTES) return
 * KVQ_ESCRATCH and launch nothing.  Every call on one device shares that
 * buffer: calls that overlap on one device (on different streams, or from
 * several host threads) race and give unspecified results; calls ordered
 * on one stream are safe.  Nothing is allocated or freed. */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_int2_decode_noalloc(const kvq_cache* cache, int32_t n_tokens,
                             const void* q_dev, int32_t q_dtype, int32_t q_heads,
                             float scale, void* out_dev, int32_t out_dtype,
                             float* lse_dev, void* stream);

/* ------------------------------------------------------------ chunk */
/* Workspace bytes attn_int2_chunk needs for these sizes. */
size_t attn_int2_chunk_workspace(const kvq_layout* L, int32_t q_len,
                                 int32_t q_heads, int32_t n_tokens);

/* A chunk of q_len query tokens per sequence (e.g. the frames being
 * generated) against the first n_tokens cached tokens, read from the packed
 * cache.  q_bf16_dev bf16 [B][q_len][q_heads][D]; out_dev
 * [B][q_len][q_heads][D] in out_dtype; lse_dev (nullable) f32
 * [B][q_heads][q_len].  Every query row sees every cached token (no mask);
 * the chunk's own keys/values are not included -- merge them with lse.
 * Precision: fp16 MFMA operands with fp32 accumulation.  A window key
 * enters as (code - 1) s, exact in fp16, with its channels' z + s added to
 * each row as a bias; a centroid key (centroid + residual, fp32) as fp16
 * hi + lo, the PSAC term as hi/lo parts too; a value as (code - 1) s, exact
 * in fp16, with z + s of its group summed exactly by one more MFMA;
 * probabilities are fp16 (their rounding multiplies v - o).  Within 2e-3
 * of the exact attention for keys with per-channel scales to 5 and values
 * with peaks near 12 (the tests).  Same window-key contract on n_tokens
 * and same errors as attn_int2_decode. */
int attn_int2_chunk(const kvq_cache* cache, int32_t n_tokens,
                    const void* q_bf16_dev, int32_t q_len, int32_t q_heads,
                    float scale, void* out_dev, int32_t out_dtype,
                    float* lse_dev, void* ws_dev, size_t ws_bytes,
                    void* stream);

/* ------------------------------------------------------------ diagnostic */
/* The attention-shift diagnostic of [QWM] (Figure 2 and "Experimental
 * Validation", Table 1: how often key quantization moves a query's
 * highest-scoring history token): for every query row, the cached token
 * t < n_tokens with the largest logit q . khat_t (+ (U^T q) . a_t with
 * PSAC), the logit attention uses before its scale; the first token on
 * ties.  Logits in fp32: channel-order fma chains over keys dequantised per
 * element (window: fma(code, s, z); tail: bf16; centroid: C_j + fma(code,
 * s, z)), then the PSAC terms in order.  q_bf16_dev bf16
 * [B][q_len][q_heads][D]; idx_out_dev i32 [B][q_heads][q_len];
 * logit_out_dev (nullable) f32 [B][q_heads][q_len].  Not a hot path (fp32
 * VALU, every row against every token).  Errors as attn_int2_chunk (no
 * workspace), and KVQ_EUNSUPPORTED for batch or q_heads above 65535. */
int attn_int2_top1(const kvq_cache* cache, int32_t n_tokens, const void* q_bf16_dev,
                   int32_t q_len, int32_t q_heads, int32_t* idx_out_dev,
                   float* logit_out_dev, void* stream);

/* Static text for a status code. */
const char* kvq_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* KVINT2_H */
