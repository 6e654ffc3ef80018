// Chunk attention: a block of query rows (e.g. the frames being generated)
// against the packed INT2 cache, on the MFMA units.
//
// Block = 8 waves x 32 query rows (256 rows) of one (sequence, query head)
// and one range of cached tokens, which stream through in 64-token tiles.
// Each thread dequantises 16 keys and 16 values of a tile straight from its
// registers into fp16 LDS tiles.  A code dword pairs codes i and i + 8 of a
// packed word (code_operand.h: base + code, exact in fp16), so key channels
// and value tokens are stored in that pairing: key operand position
// 16 w + 2 p + e holds channel 16 w + p + 8 e (the queries are loaded in the
// same order), and the score tiles and the PV k order pair tokens u, u + 8
// (slab_token, pv_pos).
//   S^T = Khat Q^T    A = key tile from LDS, B = the wave's queries (kept in
//                     registers for the whole loop);
//   O^T += Vc^T P^T   A = the value tile, B = P straight from the score
//                     registers (every lane already holds the eight P values
//                     it supplies);
//   L   += M^T P^T    A = a 16-row tile of row sums: row 0 all ones (the
//                     softmax denominator), the next rows each value
//                     group's level-1 point mu = z + s per (token, group)
//                     as fp16 hi and lo parts (per modality for
//                     per-modality rotations), so sum_t p_t mu_t comes out
//                     exact to fp32.
// Precision.  A value enters as (code - 1) s in {-s, 0, s, 2s}: one packed
// fp16 add and one packed multiply per two values, both exact, with z + s
// from the row sums above, so the values carry no rounding.  Window keys
// are (code - 1) s as well (exact, one MFMA pass) and the channels' level-1
// points z + s enter each row as a bias: a 16-row A tile holding their hi
// and lo parts gives sum_c q_c (z_c + s_c) from 8 small MFMAs per tile.
// Centroid keys (centroid + residual, fp32) enter as fp16 hi + lo (two
// passes), the lo part one v_fma_mixlo/mixhi per half.  The PSAC term uses
// k 0..23 of one more k-step as a_hi q'_hi + a_hi q'_lo + a_lo q'_hi.
// Probabilities are fp16 (their rounding multiplies v - o, not v).
// Softmax is base 2 with a lazy reference maximum: a row's m moves only
// when a score passes it by more than 2^8; each lane tests its own scores,
// and the cross-lane row maximum and the rescale run in a wave-uniform
// branch that is rarely taken.
// PSAC ([QWM] 2) adds (U^T q) . a as that extra MFMA k-step.
// Rotated values ([OKV]) are rotated back in registers at the end; with
// per-modality rotations each value takes its modality's signs first.
//
// Schedule: the two waves of each SIMD (w and w + 4) alternate a matrix
// phase (QK of tile k, PV of tile k - 1) and a vector phase (softmax of tile
// k, a share of a later tile's dequantisation, the next loads), one group
// a phase behind the other, with a barrier per phase; the matrix phase's
// LDS reads are ordered ahead of their MFMAs.  A ragged last tile runs
// unpipelined after the others.  When the row blocks alone would not fill
// the device, the cached tokens are split over blocks and a merge kernel
// combines the partial (o, m, l).
#include <type_traits>

#include "code_operand.h"
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Fourth word of a raw buffer resource (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kWaves = 8;
constexpr int kNT = 2;                       // 16-row query tiles per wave
constexpr int kBM = kWaves * kNT * 16;      // query rows per block
constexpr int kThreads = kWaves * kWave;
// a row's reference maximum may trail its true maximum by this much (log2)
constexpr float kLazyLog2 = 8.0f;

struct ChunkArgs {
  const uint8_t* kcodes;
  const uint32_t* kparams;
  const uint16_t* ktail;
  const uint8_t* kidx;
  const float* cent;
  const float* basis;
  const uint16_t* kpsac;      // fp16 coefficients, or INT8 codes (psac_int8)
  const uint16_t* kpsac_sc;   // INT8: per-token fp16 scales
  const uint8_t* vcodes;
  const uint32_t* vparams;
  const uint32_t* vsigns;     // per-modality rotations: [H][M][D/32] sign bits
  const uint8_t* vmodal;      // per-modality rotations: [B][Tcap] modality ids
  const uint16_t* q;
  void* out;
  float* lse;
  float* ws;          // split partials [S][B][Lq][Hq][D + 2] when S > 1
  int H, Hq, Tcap, C, n_tokens, Lq, out_bf16, S, tiles_per_split, n_rb, psac_int8, M;
  float scale_log2;
};

// Two fp32 values rounded to nearest fp16 and packed (one v_cvt_pk_f16_f32).
KVQ_DEV uint32_t pk_rne(float a, float b) {
  const h2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// (base + code) * s + zc, the operand half selected by hi: the half
// converts exactly, so this is one fma in fp32.
KVQ_DEV float fma_code(uint32_t word, bool hi, float s, float zc) {
  const _Float16 c = __builtin_bit_cast(h2, word)[hi ? 1 : 0];
  return __builtin_fmaf((float)c, s, zc);
}

// fp16(x0 - lo half of hi), fp16(x1 - high half of hi): the lo parts of an
// fp16 hi + lo split, each one fused multiply-add (exact in fp32) rounded
// once to nearest, written straight into the two halves of the result.
KVQ_DEV uint32_t lo_pair(uint32_t hi, float x0, float x1) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(r)
      : "v"(hi), "v"(x0), "v"(x1));
  return r;
}

// (code - 1) s for the two codes of an operand dword (base + code in each
// half) and the two scales of s2; nb holds -(base + 1) in both halves.  The
// sum leaves the small integers code - 1, the product -s, 0, s or 2s: both
// exact in fp16, one packed instruction each.
KVQ_DEV uint32_t code_scale(uint32_t cw, uint32_t nb, uint32_t s2) {
  const h2 c = __builtin_bit_cast(h2, cw) + __builtin_bit_cast(h2, nb);
  return __builtin_bit_cast(uint32_t, c * __builtin_bit_cast(h2, s2));
}

// Token order of the score tiles.  An operand dword holds codes i and i + 8
// of a word, so a thread's values pair tokens u and u + 8 of its 16, and
// the PV k order follows: position 8 g' + 2 m + e of a k-step (lane group
// g' supplies eight) holds token 16 (g' >> 1) + 4 (g' & 1) + m + 8 e.  QK
// produces those scores in the lanes that supply them when row r of score
// slab t is token slab_token(t, r).
KVQ_DEV int slab_token(int t, int r) { return 32 * (t >> 1) + 8 * (t & 1) + (r & 7) + 16 * (r >> 3); }
KVQ_DEV int pv_pos(int t) {
  const int u = t & 15, p = u & 7;
  return (t & 32) + 8 * (2 * ((t >> 4) & 1) + (p >> 2)) + 2 * (p & 3) + (u >> 3);
}

// Orders a scheduling region of NR operand reads from LDS, each feeding two
// MFMAs: DEPTH reads go first, then every read is issued two MFMAs ahead of
// its turn, so the reads' latency hides under the matrix pipe.
template <int NR, int DEPTH>
KVQ_DEV void mfma_read_order() {
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
#pragma unroll
  for (int i = 0; i < NR - DEPTH; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * DEPTH, 0);
}

template <int D, int VM>
struct Shape {
  static constexpr int NG = D / kGroup;                 // parameter groups per row
  static constexpr int M = VM == 2 ? 3 : 1;             // modality rows reserved
  static constexpr int MU_ROWS = 1 + 2 * M * NG;        // ones + mu hi/lo rows
  static constexpr int NMU = (MU_ROWS + 15) / 16;       // 16-row row-sum tiles
};

template <int D, int KM, int VM, int R>
__global__ __launch_bounds__(kThreads) void chunk_kernel(const ChunkArgs a) {
  constexpr int NKS = D / 32;        // QK k-steps
  constexpr int NDT = D / 16;        // PV output dim tiles
  // Tile pitches of 2 (mod 4) 16-byte units let the sixteen rows one operand
  // read touches fall on distinct banks; odd key rows and every other pair
  // of value rows swap neighbouring 16-byte units, which spreads the tile
  // stores over all banks as well.
  constexpr int KP = D + 16;         // key tile pitch (halfs)
  constexpr int VP = 64 + 16;        // value tile pitch (halfs)
  constexpr int NG = Shape<D, VM>::NG;
  constexpr int NMU = Shape<D, VM>::NMU;
  constexpr int KW = D / 16;         // key code words (16 channels) per token
  constexpr int NKT = 64 * KW;       // key words per tile
  constexpr int NVT = D * 4;         // value words per tile (16 tokens each)
  constexpr bool HAD = VM != 0;
  // window keys: rows 64 and 65 of a key buffer hold the channels'
  // level-1 points (hi, lo), row 66 zeros
  constexpr int KBUF = (KM == 0 ? 67 : 64) * KP;
  constexpr int LBUF = 64 * KP;
  constexpr int VBUF = D * VP;
  constexpr int MBUF = NMU * 16 * VP;
  __shared__ __align__(16) _Float16 khi[2 * KBUF];
  __shared__ __align__(16) _Float16 klo[2 * LBUF];
  __shared__ __align__(16) _Float16 vt[3 * VBUF];
  __shared__ __align__(16) _Float16 mut[3 * MBUF];
  // PSAC operand rows, 32 halves per token: a_hi, a_hi, a_lo, 0 (8 each);
  // 16-byte units swizzled by bits 2-3 of the token so the 16 rows an
  // operand read touches spread over the banks
  __shared__ __align__(16) _Float16 coef[R > 0 ? 2 * 64 * 32 : 8];
  // PSAC: each wave's q'_hi (halves 0..7) and q'_lo (8..15) per query row,
  // the B operand of the PSAC k-step, kept here rather than in registers
  // where the LDS has room for it
  constexpr int kLdsBytes = 2 * (2 * KBUF + 2 * LBUF + 3 * VBUF + 3 * MBUF + (R > 0 ? 2 * 64 * 32 : 8)) +
                            4 * (2 * (KM == 0 ? D : 64 * NG) + 2 * NG * 64 + 2 * (VM == 2 ? 16 : 1));
  constexpr bool QPL = R > 0 && kLdsBytes + 2 * kWaves * kNT * 16 * 16 <= 160 * 1024;
  __shared__ __align__(16) _Float16 qpl[QPL ? kWaves * kNT * 16 * 16 : 8];
  // parameters, two sets: tile t's in set t & 1, stored two tiles ahead.
  // Window keys: per channel, as fp16 pairs in key-operand order, the s
  // pairs in words 0 .. D/2 - 1, the z pairs after them; centroid keys:
  // (s, z) per (token, group).  Values: per group, the s of tokens u and
  // u + 8 of each 16 paired in words 0..31, the z pairs in words 32..63.
  __shared__ __align__(16) uint32_t kpar[2][KM == 0 ? D : 64 * NG];
  __shared__ __align__(16) uint32_t vpar[2][NG][64];
  __shared__ __align__(16) uint32_t vmod[2][VM == 2 ? 16 : 1];         // modality bytes of the tile

  const int rb = blockIdx.x % a.n_rb, split = blockIdx.x / a.n_rb;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.H, h = hq / G;
  const int64_t bh = (int64_t)b * a.H + h;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int row0 = rb * kBM + wave * kNT * 16;
  const bool live = row0 < a.Lq;   // wave-uniform
  const bool flip = (wave >> 2) & 1;  // the second wave of each SIMD
  const int n = a.n_tokens;
  const int n_tiles = (n + 63) / 64, n_full = n / 64;
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, n_tiles);
  const bool has_ragged = (n & 63) != 0 && tile_end == n_tiles && tile_begin < tile_end;
  const int full_end = has_ragged ? tile_end - 1 : tile_end;   // tiles [tile_begin, full_end) are full
  const int M = a.M;

  CodeOr kor = {0x54005400u, 0x4C004C00u, 0x44004400u};
  asm volatile("" : "+v"(kor.b64), "+v"(kor.b16), "+v"(kor.b4));
  // -(base + 1) in both halves for the three operand bases (64, 16, 4)
  uint32_t nb65 = 0xD410D410u, nb17 = 0xCC40CC40u, nb5 = 0xC500C500u;
  asm volatile("" : "+v"(nb65), "+v"(nb17), "+v"(nb5));
  auto nbase = [&](int p) { return (p == 2 || p == 5) ? nb65 : ((p == 1 || p == 4 || p == 7) ? nb5 : nb17); };

  // ---- LDS set-up: value and row-sum buffers zero (the first PV step
  // multiplies a zero P by buffer 2), row 0 of every row-sum tile all ones
  {
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (int e = tid; e < 3 * VBUF / 8; e += kThreads) reinterpret_cast<uint4*>(vt)[e] = z4;
    for (int e = tid; e < 3 * MBUF / 8; e += kThreads) reinterpret_cast<uint4*>(mut)[e] = z4;
    if (KM == 0 && tid < 2 * D / 8)   // the zero row of both key buffers
      reinterpret_cast<uint4*>(khi + (tid / (D / 8)) * KBUF + 66 * KP)[tid % (D / 8)] = z4;
    __syncthreads();
    if (tid < 3 * NMU * 64) {
      const int buf = tid / (NMU * 64), rest = tid % (NMU * 64), tile16 = rest / 64, t = rest % 64;
      if (tile16 == 0) mut[buf * MBUF + pv_pos(t)] = (_Float16)1.0f;   // row 0 swizzle: none
    }
  }

  // ---- queries (B operand), fp16 (exact from bf16), resident for the whole
  // loop, in key-operand channel order: operand position 16 w + 2 p + e
  // holds channel 16 w + p + 8 e (the two channels of one code dword), so
  // lane group g of k-step ks takes channels c0 + {0, 8, 1, 9, 2, 10, 3, 11}
  h8 qreg[kNT][NKS];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int row = row0 + nt * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      h8 v;
      if (row < a.Lq) {
        const uint16_t* qr = a.q + (((int64_t)b * a.Lq + row) * a.Hq + hq) * D + ks * 32 + 16 * (g >> 1) + 4 * (g & 1);
        const uint2 u0 = *reinterpret_cast<const uint2*>(qr), u1 = *reinterpret_cast<const uint2*>(qr + 8);
        float x[8];
        bf16x8_to_f32(make_uint4(u0.x, u1.x, u0.y, u1.y), x);   // channels c0, c0+1, c0+8, c0+9, ...
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = (_Float16)x[(j >> 1) * 4 + (j & 1)];
          v[2 * j + 1] = (_Float16)x[(j >> 1) * 4 + 2 + (j & 1)];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (_Float16)0.0f;
      }
      qreg[nt][ks] = v;
    }
  }
  // ---- PSAC: q' = U^T q, the B operand of one more 16x16x32 k-step: lanes
  // g = 0, 1, 2 supply q'_hi, q'_lo, q'_hi of their row (k 0..23); g = 3
  // supplies q'_hi again, against the coefficient tile's zeros (k 24..31)
  static_assert(R == 0 || R == 8, "PSAC rank 8 fills k 0..23 of one k-step");
  h8 qpr[kNT];   // (without room in the LDS)
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    if (R > 0 && (g < 2 || !QPL)) {
      h8 qv;
#pragma unroll
      for (int j = 0; j < 8; ++j) qv[j] = (_Float16)0.0f;
      const int row = row0 + nt * 16 + c16;
      if (row < a.Lq) {
        const uint16_t* qr = a.q + (((int64_t)b * a.Lq + row) * a.Hq + hq) * D;
        const float* U = a.basis + bh * D * (R > 0 ? R : 1);
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        for (int d = 0; d < D; ++d) {
          const float qd = bf16_to_f32(qr[d]);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(U[d * R + j], qd, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const _Float16 hi = (_Float16)opaque(acc[j]);
          qv[j] = (g == 1) ? (_Float16)(acc[j] - (float)hi) : hi;
        }
      }
      if (QPL) *reinterpret_cast<h8*>(&qpl[((wave * kNT + nt) * 16 + c16) * 16 + 8 * g]) = qv;
      else qpr[nt] = qv;
    }
  }

  // m_run: reference maximum (log2 units); thr: the raw score above which it
  // moves, (m_run + kLazyLog2) / scale_log2
  float m_run[kNT], thr[kNT];
  const float inv_scale_log2 = 1.0f / a.scale_log2;
  f4 o[kNT][NDT], ol[kNT][NMU];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    m_run[nt] = -__builtin_inff();
    thr[nt] = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < NMU; ++u) ol[nt][u] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[nt][dt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // ---- per-thread share of a tile: key word = token tk, channels
  // 16 kw .. 16 kw + 15 (each group of eight lanes holds two tokens);
  // value word = channel vc, tokens 16 vq .. 16 vq + 15; row sums: token
  // tm, group gm
  const int tk = KW == 8 ? 2 * (tid >> 4) + ((tid >> 2) & 1) : tid / KW;
  const int kw = KW == 8 ? (tid & 3) + 4 * ((tid >> 3) & 1) : tid % KW;
  const int vc = tid >> 2, vq = tid & 3;
  // (the conditions fold to true where a tile has a word for every thread;
  // threads beyond the 64 NG (token, group) pairs repeat the first ones)
  const int tm = (tid % (64 * NG)) / NG, gm = tid % NG;
  const bool has_k = NKT >= kThreads || tid < NKT, has_v = NVT >= kThreads || tid < NVT;
  // per-modality rotations: bit m of vsgn = sign of channel vc in modality m
  uint32_t vsgn = 0u;
  if (VM == 2 && has_v) {
    for (int m = 0; m < M; ++m)
      vsgn |= ((a.vsigns[((int64_t)h * M + m) * (D / 32) + vc / 32] >> (vc & 31)) & 1u) << m;
  }

  struct Pre {
    uint32_t kcw, vcw, cf, cs;   // cf/cs: PSAC words (INT8: two codes, scale)
    int ix;            // centroid index of token tk
    float cv[16];      // centroid channels 16 kw .. 16 kw + 15 of token tk
  };
  struct Par {
    uint32_t kp, vp, md;
  };
  // this thread's packed words of a tile: codes, centroid index, PSAC
  // coefficients.  RAG (the ragged last tile): rows past the length read as
  // 0, so they dequantise to finite values; full tiles load unconditionally.
  // Buffer views of this (sequence, kv head)'s rows: per-thread offsets
  // stay fixed, a tile's offset goes in the scalar offset, and no 64-bit
  // address arithmetic is left in the loop (reads past a view return 0).
  const auto rkc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.kcodes + bh * a.Tcap * (D / 4)), (short)0,
                                                     a.Tcap * (D / 4), kRsrcWord3);
  const auto rki = __builtin_amdgcn_make_buffer_rsrc((void*)(a.kidx + (KM != 0 ? bh * a.Tcap : 0)), (short)0,
                                                     KM != 0 ? a.Tcap : 0, kRsrcWord3);
  const auto rvc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.vcodes + bh * (a.Tcap / 64) * (int64_t)D * 16), (short)0, (a.Tcap / 64) * D * 16, kRsrcWord3);
  const auto rvp = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vparams + bh * a.Tcap * NG), (short)0,
                                                     a.Tcap * NG * 4, kRsrcWord3);
  const auto rkp = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.kparams + (KM == 0 ? bh * (a.Tcap / 64) * D : bh * a.Tcap * NG)), (short)0,
      (KM == 0 ? (a.Tcap / 64) * D : a.Tcap * NG) * 4, kRsrcWord3);
  const auto rmd = __builtin_amdgcn_make_buffer_rsrc((void*)(VM == 2 ? a.vmodal + (int64_t)b * a.Tcap : a.vmodal),
                                                     (short)0, VM == 2 ? a.Tcap : 0, kRsrcWord3);
  const auto rce = __builtin_amdgcn_make_buffer_rsrc((void*)(KM != 0 ? a.cent + bh * a.C * D : a.cent), (short)0,
                                                     KM != 0 ? a.C * D * 4 : 0, kRsrcWord3);
  const int pi = tid % (64 * NG);   // (token, group) parameter word of this thread
  // this thread's packed words of a tile: codes, centroid index, PSAC
  // coefficients.  RAG (the ragged last tile): rows past the length read as
  // 0, so they dequantise to finite values; full tiles load unconditionally.
  auto load_codes = [&](int tile, Pre& f, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const int t0 = tile * 64;
    const int64_t rowbase = bh * a.Tcap + t0;
    f.kcw = has_k ? __builtin_amdgcn_raw_buffer_load_b32(rkc, (tk * KW + kw) * 4, t0 * (D / 4), 0) : 0u;
    f.vcw = has_v ? __builtin_amdgcn_raw_buffer_load_b32(rvc, tid * 4, tile * D * 16, 0) : 0u;
    if (KM != 0) {
      f.ix = has_k ? (int)__builtin_amdgcn_raw_buffer_load_b8(rki, tk, t0, 0) : 0;
      if (RAG && t0 + tk >= n) f.ix = 0;
    }
    f.cf = 0u;
    f.cs = 0u;
    if (R > 0 && (64 * 8 >= kThreads || tid < 64 * 8)) {   // PSAC coefficients: two per thread
      const int t = tid >> 3, m2 = (tid & 7) * 2;
      const bool mine = m2 < R && (!RAG || t0 + t < n);
      if (a.psac_int8) {
        f.cf = reinterpret_cast<const uint16_t*>(
            reinterpret_cast<const uint8_t*>(a.kpsac) + (rowbase + t) * R)[(m2 & (R - 1)) / 2];
        f.cs = a.kpsac_sc[rowbase + t];
      } else {
        f.cf = reinterpret_cast<const uint32_t*>(a.kpsac + (rowbase + t) * R)[(m2 & (R - 1)) / 2];
      }
      if (!mine) {
        f.cf = 0u;
        f.cs = 0u;
      }
    }
  };
  // the tile's parameter words (value and key (z, s), modality bytes):
  // threads 0 .. 255 cover every word and stage them in LDS
  auto load_params = [&](int tile, Par& f, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const int t0 = tile * 64;
    f.vp = __builtin_amdgcn_raw_buffer_load_b32(rvp, pi * 4, t0 * NG * 4, 0);
    if (RAG && t0 + pi / NG >= n) f.vp = 0u;
    if (KM == 0) {
      f.kp = (RAG && tile >= n_full) ? 0u : __builtin_amdgcn_raw_buffer_load_b32(rkp, (tid % D) * 4, tile * D * 4, 0);
    } else {
      f.kp = __builtin_amdgcn_raw_buffer_load_b32(rkp, pi * 4, t0 * NG * 4, 0);
      if (RAG && t0 + pi / NG >= n) f.kp = 0u;
    }
    f.md = 0u;
    if (VM == 2 && tid < 16) f.md = __builtin_amdgcn_raw_buffer_load_b32(rmd, tid * 4, t0, 0);
  };
  // centroid rows need the index, so they are requested one step later
  auto prefetch_cent = [&](Pre& f) {
    if (KM != 0 && has_k) {
      const int co = (f.ix * D + 16 * kw) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // bit-cast the whole vector: this compiler reads element 0 for a
        // bit_cast of one subscripted vector element
        const float4 c4 = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rce, co + 16 * j, 0, 0));
        f.cv[4 * j] = c4.x; f.cv[4 * j + 1] = c4.y; f.cv[4 * j + 2] = c4.z; f.cv[4 * j + 3] = c4.w;
      }
    }
  };
  // (threads 0..255; beyond the words of a tile they repeat earlier ones)
  auto store_params = [&](int tile, const Par& f) {
    const int ps = tile & 1;
    {
      // token tm = 16 vq + 8 e + p: half e of pair word 8 vq + p
      uint16_t* vw = reinterpret_cast<uint16_t*>(&vpar[ps][gm][0]);
      const int hx = 2 * (8 * (tm >> 4) + (tm & 7)) + ((tm >> 3) & 1);
      vw[hx] = (uint16_t)f.vp;
      vw[64 + hx] = (uint16_t)(f.vp >> 16);
    }
    if (KM == 0) {
      if (tid < D) {   // channel tid = 16 w + 8 e + p: operand position 16 w + 2 p + e
        uint16_t* kw16 = reinterpret_cast<uint16_t*>(&kpar[ps][0]);
        const int hx = 16 * (tid >> 4) + 2 * (tid & 7) + ((tid >> 3) & 1);
        kw16[hx] = (uint16_t)f.kp;
        kw16[D + hx] = (uint16_t)(f.kp >> 16);
      }
    } else {
      kpar[ps][tid % (64 * NG)] = f.kp;
    }
    if (VM == 2 && tid < 16) vmod[ps][tid] = f.md;
  };

  // ---- dequantise tile `tile` into key buffer kb, value / row-sum buffer
  // vbuf, coefficient buffer kb.  RAG: the ragged last tile (window keys of
  // the unfinished window come from the tail; keys past the length are 0).
  auto dequant_v = [&](int tile, const Pre& c, int kb, int vbuf, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const int ps = tile & 1;
    const int t0 = tile * 64;
    if (R > 0 && (64 * 8 >= kThreads || tid < 64 * 8)) {
      // coefficient pair j = tid & 7 (< 4) of token t: hi in u32 words j and
      // 4 + j, lo in 8 + j; threads j >= 4 clear words 8 + j
      const int t = tid >> 3, j = tid & 7;
      uint32_t hw = c.cf, lw = 0u;
      if (a.psac_int8) {   // two INT8 codes times the token's scale (exact in fp32)
        const float sc = f16_bits_to_f32(c.cs);
        const float a0 = (float)(int8_t)(c.cf & 0xFFu) * sc, a1 = (float)(int8_t)(c.cf >> 8) * sc;
        hw = pk_rne(opaque(a0), opaque(a1));
        const h2 hh = __builtin_bit_cast(h2, hw);
        lw = pk_rne(a0 - (float)hh[0], a1 - (float)hh[1]);
      }
      uint32_t* cr = reinterpret_cast<uint32_t*>(coef + kb * 64 * 32) + t * 16;
      const int sw = (t >> 2) & 3;
      auto at = [&](int w) { return cr + ((((w >> 2) ^ sw) << 2) | (w & 3)); };
      if (j < 4) {
        *at(j) = hw;
        *at(4 + j) = hw;
        *at(8 + j) = lw;
      } else {
        *at(8 + j) = 0u;
      }
    }
    // values: channel vc, tokens 16 vq + p and 16 vq + 8 + p in dword p,
    // (code - 1) s (exact); with the PV token order the eight dwords are the
    // two 16-byte units 2 (vq & 1) and 2 (vq & 1) + 1 of k-step vq / 2
    // (swapped in pairs of rows)
    if (has_v) {
      uint32_t cw[8];
      code_word(c.vcw, kor, cw);
      const uint4* sp4 = reinterpret_cast<const uint4*>(&vpar[ps][vc / kGroup][8 * vq]);
      const uint4 s0 = sp4[0], s1 = sp4[1];
      const uint32_t sp[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      uint32_t pk[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) pk[p] = code_scale(cw[p], nbase(p), sp[p]);
      if (VM == 2) {
        // sign of (token, channel vc): bit m(t) of vsgn; negate those halves
        const uint32_t* mw = &vmod[ps][4 * vq];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const uint32_t mb = mw[w4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int u = 4 * w4 + k;   // token 16 vq + u
            const uint32_t m = min((mb >> (8 * k)) & 0xFFu, (uint32_t)(M - 1));
            pk[u & 7] ^= ((vsgn >> m) & 1u) << (15 + 16 * (u >> 3));
          }
        }
      }
      _Float16* dst = &vt[vbuf * VBUF + vc * VP + 32 * (vq >> 1)];
      const int vs = (vc >> 1) & 1, u0 = 2 * (vq & 1);
      *reinterpret_cast<uint4*>(dst + 8 * (u0 ^ vs)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4*>(dst + 8 * ((u0 + 1) ^ vs)) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
    // row sums: level 1, z + s, of (token tm, group gm) as fp16 hi and lo,
    // in the rows of the token's modality (zero in the others)
    {
      const uint16_t* vw = reinterpret_cast<const uint16_t*>(&vpar[ps][gm][0]);
      const int hx = 2 * (8 * (tm >> 4) + (tm & 7)) + ((tm >> 3) & 1);
      const float mu = f16_bits_to_f32(vw[64 + hx]) + f16_bits_to_f32(vw[hx]);
      const _Float16 mh = (_Float16)opaque(mu);
      const _Float16 ml = (_Float16)(mu - (float)mh);
      int mt = 0;
      if (VM == 2) mt = min((int)((vmod[ps][tm >> 2] >> (8 * (tm & 3))) & 0xFFu), M - 1);
      const int pos = pv_pos(tm);
      constexpr int MM = Shape<D, VM>::M;
      for (int m = 0; m < (VM == 2 ? M : 1); ++m) {
        const int rh = 1 + m * NG + gm;
        const int rl = 1 + MM * NG + m * NG + gm;
        const bool mine = (m == mt);
        const int ph = (pos & ~24) | ((((pos >> 3) & 3) ^ ((rh >> 1) & 1)) << 3);
        const int pl = (pos & ~24) | ((((pos >> 3) & 3) ^ ((rl >> 1) & 1)) << 3);
        mut[vbuf * MBUF + rh * VP + ph] = mine ? mh : (_Float16)0.0f;
        mut[vbuf * MBUF + rl * VP + pl] = mine ? ml : (_Float16)0.0f;
      }
    }
  };
  auto dequant_k = [&](int tile, const Pre& c, int kb, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const int ps = tile & 1;
    const int t0 = tile * 64;
    // keys: token tk, channels 16 kw + p and 16 kw + 8 + p in dword p
    if (has_k) {
      uint32_t hw[8], lw[8];
      const bool tail = RAG && KM == 0;   // the unfinished window
      if (KM == 0 && !tail) {
        // window keys: (code - 1) s, exact, one MFMA pass; the level-1 point
        // z + s of each channel enters as a per-row bias
        uint32_t cw[8];
        code_word(c.kcw, kor, cw);
        const uint4* sp4 = reinterpret_cast<const uint4*>(&kpar[ps][8 * kw]);
        const uint4 s0 = sp4[0], s1 = sp4[1];
        const uint32_t sp[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int p = 0; p < 8; ++p) hw[p] = code_scale(cw[p], nbase(p), sp[p]);
      } else {
        float kv[16];
        if (!tail) {
          uint32_t cw[8];
          code_word(c.kcw, kor, cw);
          const uint32_t pw = kpar[ps][tk * NG + kw / 2];
          const float s = f16_bits_to_f32(pw), z = f16_bits_to_f32(pw >> 16);
          const float z16 = __builtin_fmaf(-16.0f, s, z), z4 = __builtin_fmaf(-4.0f, s, z),
                      z64 = __builtin_fmaf(-64.0f, s, z);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int p = i & 7;
            const float zb = (p == 2 || p == 5) ? z64 : ((p == 1 || p == 4 || p == 7) ? z4 : z16);
            // centroid + residual (the residual rounded to fp32 first)
            kv[i] = c.cv[i] + fma_code(cw[p], i >= 8, s, zb);
          }
        } else {
          const uint16_t* kt = a.ktail + (bh * 64 + tk) * D + 16 * kw;
          bf16x8_to_f32(*reinterpret_cast<const uint4*>(kt), kv);
          bf16x8_to_f32(*reinterpret_cast<const uint4*>(kt + 8), kv + 8);
        }
        if (RAG && t0 + tk >= n) {
#pragma unroll
          for (int i = 0; i < 16; ++i) kv[i] = 0.0f;
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          hw[p] = pk_rne(kv[p], kv[p + 8]);
          lw[p] = lo_pair(hw[p], kv[p], kv[p + 8]);
        }
      }
      // 16-byte units 2 kw, 2 kw + 1 of row tk, swapped in odd rows
      const int o0 = tk * KP + 8 * ((2 * kw) ^ (tk & 1));
      const int o1 = tk * KP + 8 * ((2 * kw + 1) ^ (tk & 1));
      *reinterpret_cast<uint4*>(&khi[kb * KBUF + o0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&khi[kb * KBUF + o1]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      if (KM != 0 || tail) {
        *reinterpret_cast<uint4*>(&klo[kb * LBUF + o0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint4*>(&klo[kb * LBUF + o1]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      }
    }
    // window keys: each channel's level-1 point z + s as fp16 hi (row 64)
    // and lo (row 65) of the key buffer, at the channel's operand position
    if (KM == 0 && !RAG && tid < D) {
      const uint16_t* kw16 = reinterpret_cast<const uint16_t*>(&kpar[ps][0]);
      const int hx = 16 * (tid >> 4) + 2 * (tid & 7) + ((tid >> 3) & 1);
      const float mu = f16_bits_to_f32(kw16[D + hx]) + f16_bits_to_f32(kw16[hx]);
      const _Float16 mh = (_Float16)opaque(mu);
      khi[kb * KBUF + 64 * KP + hx] = mh;
      khi[kb * KBUF + 65 * KP + hx] = (_Float16)(mu - (float)mh);
    }
  };
  // (values first: centroid rows requested just before can arrive meanwhile)
  auto dequant = [&](int tile, const Pre& c, int kb, int vbuf, auto rag) {
    dequant_v(tile, c, kb, vbuf, rag);
    dequant_k(tile, c, kb, rag);
  };

  // ---- S^T = Khat Q^T for the 64 tokens of key buffer kb, row r of slab
  // t holding token slab_token(t, r): PSAC k-step first, then hi (and lo,
  // TWO) of every k-step.  One pass (window keys): cst gets the level-1
  // points' products, rows 4g and 4g + 1 (hi, lo) of every lane group.
  auto qk = [&](int kb, f4 (&s)[kNT][4], auto two, f4 (&cst)[kNT]) {
    constexpr bool TWO = decltype(two)::value;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      cst[nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 4; ++t) s[nt][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const _Float16* kh = khi + kb * KBUF;
    const _Float16* kl = klo + kb * LBUF;
    if (R > 0) {
      h8 qp[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        qp[nt] = QPL ? *reinterpret_cast<const h8*>(&qpl[((wave * kNT + nt) * 16 + c16) * 16 + (g == 1 ? 8 : 0)])
                     : qpr[nt];
      // row slab_token(t, c16) of the coefficient tile (k 0..23)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int cr = slab_token(t, c16);
        const h8 ca = *reinterpret_cast<const h8*>(&coef[kb * 64 * 32 + cr * 32 + 8 * (g ^ ((cr >> 2) & 3))]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca, qp[nt], s[nt][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      h8 ka[4], kl2[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // (a token's parity is c16's, which picks the unit swap)
        const int off = slab_token(t, c16) * KP + ks * 32 + 8 * (g ^ (c16 & 1));
        ka[t] = *reinterpret_cast<const h8*>(&kh[off]);
        if (TWO) kl2[t] = *reinterpret_cast<const h8*>(&kl[off]);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[t], qreg[nt][ks], s[nt][t], 0, 0, 0);
      if (TWO) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            s[nt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl2[t], qreg[nt][ks], s[nt][t], 0, 0, 0);
      } else if (KM == 0) {
        // A rows c16 = 4i (hi), 4i + 1 (lo) of the level-1 points, others zero
        const int mr = 64 + ((c16 & 3) < 2 ? (c16 & 3) : 2);
        const h8 am = *reinterpret_cast<const h8*>(&kh[mr * KP + ks * 32 + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          cst[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, qreg[nt][ks], cst[nt], 0, 0, 0);
      }
    }
  };

  // ---- O^T += Vc^T P^T and the row sums, for value buffer vbuf
  auto pv = [&](int vbuf, const h8 (&pb)[kNT][2]) {
    const _Float16* vb = vt + vbuf * VBUF;
    const _Float16* mb = mut + vbuf * MBUF;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const h8 va = *reinterpret_cast<const h8*>(&vb[(dt * 16 + c16) * VP + kk * 32 + 8 * (g ^ ((c16 >> 1) & 1))]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[nt][kk], o[nt][dt], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < NMU; ++u) {
        const int r = u * 16 + c16;
        const h8 ma = *reinterpret_cast<const h8*>(&mb[r * VP + kk * 32 + 8 * (g ^ ((r >> 1) & 1))]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          ol[nt][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ma, pb[nt][kk], ol[nt][u], 0, 0, 0);
      }
    }
  };

  // ---- online softmax (base 2) of a tile's scores into P (fp16); lane
  // owns row nt*16 + c16, scores s[nt][t][i] of token slab_token(t, 4g + i)
  // plus the row's bias (window keys: the level-1 points' product).
  // row_max returns whether some row's reference maximum must move (then
  // `grow`).
  auto row_max = [&](const f4 (&s)[kNT][4], const float (&bias)[kNT], float (&lm)[kNT]) {
    bool gr = false;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float m = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 4; ++t)
        m = fmaxf(fmaxf(m, fmaxf(s[nt][t][0], s[nt][t][1])), fmaxf(s[nt][t][2], s[nt][t][3]));
      lm[nt] = m + bias[nt];
      gr |= lm[nt] > thr[nt];
    }
    return gr;
  };
  auto grow = [&](const float (&lm)[kNT]) {
    // a real branch: without this the compiler may run the rescale of
    // every accumulator unconditionally (by an alpha of 1)
    asm volatile("");
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float m = lm[nt];
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const float mn = fmaxf(m_run[nt], m * a.scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - mn);   // 0 on the first tile
      m_run[nt] = mn;
      thr[nt] = (mn + kLazyLog2) * inv_scale_log2;
#pragma unroll
      for (int u = 0; u < NMU; ++u) ol[nt][u] *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[nt][dt] *= alpha;
    }
  };
  // P: the B operands of the two PV k-steps; dword m of k-step kk pairs the
  // m-th scores of slabs 2 kk and 2 kk + 1 (tokens 8 apart)
  auto probs = [&](const f4 (&s)[kNT][4], const float (&bias)[kNT], h8 (&pb)[kNT][2]) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const float off = __builtin_fmaf(bias[nt], a.scale_log2, -m_run[nt]);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t pw[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nt][2 * kk][m], a.scale_log2, off));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nt][2 * kk + 1][m], a.scale_log2, off));
          pw[m] = pk_rne(p0, p1);
        }
        pb[nt][kk] = as_h8(pw[0], pw[1], pw[2], pw[3]);
      }
    }
  };
  // RAG: the scores of tokens at or past the length are masked
  auto softmax = [&](f4 (&s)[kNT][4], const float (&bias)[kNT], h8 (&pb)[kNT][2], int t0, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    if (RAG) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + slab_token(t, 4 * g + i) >= n) s[nt][t][i] = -__builtin_inff();
    }
    float lm[kNT];
    if (__builtin_expect(__any(row_max(s, bias, lm)), 0)) grow(lm);
    probs(s, bias, pb);
  };

  // P of the previous tile, S of the current one
  h8 pb[kNT][2];
  f4 sc[kNT][4], cst[kNT];
  float bias[kNT] = {};
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[nt][kk][j] = (_Float16)0.0f;

  // ---- ping-pong over the SIMDs.  Waves w and w + 4 share a SIMD; each
  // alternates a matrix phase (QK of tile k, PV of tile k - 1) with a
  // vector phase (softmax of tile k, its share of the dequantisation of a
  // later tile, the next loads), one barrier per phase.  The second group
  // (waves 4..7) runs one phase behind the first, so in every phase one
  // wave of each SIMD feeds the matrix pipe while the other keeps the
  // vector pipe busy.  Tile k + 1 is dequantised by the first group in its
  // vector phase k and by the second in its vector phase k - 1, both
  // before either group's matrix phase k + 1; with the phase offset a key
  // buffer is rewritten two phases after its last read (two buffers) and
  // a value buffer four (three buffers).  The first group (threads
  // 0..255) stages the parameter words, two tiles ahead.  Packed codes are
  // requested a matrix phase before their vector phase, which first asks
  // for the centroid rows they index, then forms P and dequantises values
  // while those arrive.  (A wave whose rows
  // are all past the end only dequantises and keeps the barriers.)
  auto phase = [&]() {
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // cur: the packed words (and centroid rows) of the tile this wave
  // dequantises next, requested a matrix phase ahead; par: parameter
  // words, stored the phase pair after they arrive.  The loop's loads are
  // unconditional (a tile index past the end reads the last full tile
  // again), so no loaded register is copied at the loop's end, which would
  // wait for the load.
  Pre cur;
  Par par;
  const int nfull = full_end - tile_begin;
  if (nfull > 0) {
    const int last = full_end - 1;
    load_codes(tile_begin, cur, std::false_type{});
    if (!flip) load_params(tile_begin, par, std::false_type{});
    prefetch_cent(cur);
    if (!flip) {
      store_params(tile_begin, par);
      if (nfull > 1) {
        load_params(tile_begin + 1, par, std::false_type{});
        store_params(tile_begin + 1, par);
      }
    }
    __syncthreads();
    dequant(tile_begin, cur, 0, 0, std::false_type{});
    load_codes(min(tile_begin + 1, last), cur, std::false_type{});
    load_params(min(tile_begin + 2, last), par, std::false_type{});
    if (flip) {   // the second group's vector phase -1: its share of tile 1
      phase();
      prefetch_cent(cur);
      if (nfull > 1) dequant(tile_begin + 1, cur, 1, 1, std::false_type{});
      load_codes(min(tile_begin + 2, last), cur, std::false_type{});
    }
    for (int k = 0; k < nfull; ++k) {
      const int dq = k + 1 + (flip ? 1 : 0);   // the tile this wave dequantises next
      phase();   // ---- matrix phase k
      if (live) {
        // (at k = 0, P is zero and value buffer 2 still holds its zeros)
        __builtin_amdgcn_s_setprio(1);
        qk(k & 1, sc, std::integral_constant<bool, KM != 0>{}, cst);
        pv((k + 2) % 3, pb);
        mfma_read_order<(R > 0 ? (QPL ? 6 : 4) : 0) + (KM != 0 ? 8 : 5) * NKS + 2 * (NDT + NMU), 6>();
        __builtin_amdgcn_s_setprio(0);
        if (KM == 0) {
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) bias[nt] = cst[nt][0] + cst[nt][1];
        }
      }
      phase();   // ---- vector phase k
      prefetch_cent(cur);   // (its index arrived during the matrix phase)
      if (live) softmax(sc, bias, pb, 0, std::false_type{});
      if (dq < nfull) dequant(tile_begin + dq, cur, dq & 1, dq % 3, std::false_type{});
      if (!flip && k + 2 < nfull) store_params(tile_begin + k + 2, par);
      load_codes(min(tile_begin + dq + 1, last), cur, std::false_type{});
      load_params(min(tile_begin + k + 3, last), par, std::false_type{});
    }
    if (!flip) phase();   // meets the second group's last vector phase
    // PV of the last full tile
    if (live) pv((nfull - 1) % 3, pb);
  }

  // ---- the ragged last tile, unpipelined
  if (has_ragged) {
    const int tile = tile_end - 1;
    __syncthreads();   // every buffer is free
    load_codes(tile, cur, std::true_type{});
    if (!flip) load_params(tile, par, std::true_type{});
    prefetch_cent(cur);
    if (!flip) store_params(tile, par);
    __syncthreads();
    dequant(tile, cur, 0, 0, std::true_type{});
    __syncthreads();
    if (live) {
      const float zero[kNT] = {};
      qk(0, sc, std::true_type{}, cst);
      softmax(sc, zero, pb, tile * 64, std::true_type{});
      pv(0, pb);
    }
  }

  // ---- epilogue: l of row c16 sits in lane c16 (row 0 of the row-sum
  // tile); the midpoint sums of row r in lane 16 (r % 16 / 4) + c16,
  // element r % 4, of row-sum tile r / 16
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const float l = __shfl(ol[nt][0][0], c16, 64);
    constexpr int MM = Shape<D, VM>::M;
    float mus[MM][NG];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        const int rh = 1 + m * NG + gr, rl = 1 + MM * NG + m * NG + gr;
        // a runtime M below MM leaves rows that hold zeros
        const float vh = __shfl(ol[nt][rh / 16][rh % 4], ((rh % 16) / 4) * 16 + c16, 64);
        const float vl = __shfl(ol[nt][rl / 16][rl % 4], ((rl % 16) / 4) * 16 + c16, 64);
        mus[m][gr] = vh + vl;
      }
    float v[NDT][4];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = dt * 16 + 4 * g + i, gr = dt >> 1;
        float add = mus[0][gr];
        if (VM == 2) {
          add = 0.0f;
#pragma unroll
          for (int m = 0; m < MM; ++m) {
            if (m < M) {
              const uint32_t sw = a.vsigns[((int64_t)h * M + m) * (D / 32) + ch / 32];
              add += ((sw >> (ch & 31)) & 1u) ? -mus[m][gr] : mus[m][gr];
            }
          }
        }
        v[dt][i] = o[nt][dt][i] + add;
      }
    const int row = row0 + nt * 16 + c16;
    if (a.S > 1) {
      // partial (o, m, l) for the merge
      if (row < a.Lq) {
        float* dst = a.ws + ((((int64_t)split * gridDim.z + b) * a.Lq + row) * a.Hq + hq) * (D + 2);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<float4*>(dst + dt * 16 + 4 * g) =
              make_float4(v[dt][0], v[dt][1], v[dt][2], v[dt][3]);
        if (g == 0) {
          dst[D] = m_run[nt];
          dst[D + 1] = l;
        }
      }
      continue;
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[dt][i] *= inv;
    if (HAD) {
      // dim = dt*16 + 4g + i: bits 0-1 in-lane (i), bits 2-3 across lanes
      // (g: xor 16, 32), bits 4.. in-lane (dt)
#pragma unroll
      for (int hh = 1; hh < 4; hh <<= 1)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((i & hh) == 0) {
              const float x0 = v[dt][i], x1 = v[dt][i + hh];
              v[dt][i] = x0 + x1;
              v[dt][i + hh] = x0 - x1;
            }
#pragma unroll
      for (int sg = 1; sg < 4; sg <<= 1) {
        const bool upper = (g & sg) != 0;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ot = __shfl_xor(v[dt][i], 16 * sg, 64);
            v[dt][i] = upper ? (ot - v[dt][i]) : (v[dt][i] + ot);
          }
      }
#pragma unroll
      for (int hh = 1; hh < NDT; hh <<= 1)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          if ((dt & hh) == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x0 = v[dt][i], x1 = v[dt + hh][i];
              v[dt][i] = x0 + x1;
              v[dt + hh][i] = x0 - x1;
            }
      const float cn = (D == 128) ? 0.08838834764831845f : 0.125f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[dt][i] *= cn;
    }
    if (row < a.Lq) {
      const int64_t base = (((int64_t)b * a.Lq + row) * a.Hq + hq) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d0 = dt * 16 + 4 * g;
        if (a.out_bf16) {
          uint32_t w2[2];
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            uint32_t u0 = __float_as_uint(v[dt][i]), u1 = __float_as_uint(v[dt][i + 1]);
            u0 += 0x7FFFu + ((u0 >> 16) & 1u);
            u1 += 0x7FFFu + ((u1 >> 16) & 1u);
            w2[i / 2] = (u0 >> 16) | (u1 & 0xFFFF0000u);
          }
          *reinterpret_cast<uint2*>((uint16_t*)a.out + base + d0) = make_uint2(w2[0], w2[1]);
        } else {
          *reinterpret_cast<float4*>((float*)a.out + base + d0) =
              make_float4(v[dt][0], v[dt][1], v[dt][2], v[dt][3]);
        }
      }
      if (g == 0 && a.lse != nullptr)
        a.lse[((int64_t)b * a.Hq + hq) * a.Lq + row] = (m_run[nt] + log2f(l)) * kLn2;
    }
  }
}

// Merges the split partials of one output row r = (b * Lq + row) * Hq + hq:
// out, lse, and the inverse rotation of rotated values.
template <int D, bool HAD>
__global__ __launch_bounds__(D) void chunk_merge_kernel(const ChunkArgs a) {
  __shared__ float xs[D];
  const int r = blockIdx.x, c = threadIdx.x;
  const int64_t rows = (int64_t)gridDim.x;
  float M = -__builtin_inff(), L = 0.0f, acc = 0.0f;
  for (int s0 = 0; s0 < a.S; s0 += 16) {
    float mv[16], lv[16], pv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      mv[k] = -__builtin_inff();
      lv[k] = pv[k] = 0.0f;
      if (s0 + k < a.S) {
        const float* p = a.ws + ((int64_t)(s0 + k) * rows + r) * (D + 2);
        mv[k] = p[D];
        lv[k] = p[D + 1];
        pv[k] = p[c];
      }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < 16; ++k) Mn = fmaxf(Mn, mv[k]);
    if (Mn == -__builtin_inff()) continue;
    const float sc = (M == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float f = (mv[k] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mv[k] - Mn);
      L = __builtin_fmaf(f, lv[k], L);
      acc = __builtin_fmaf(f, pv[k], acc);
    }
    M = Mn;
  }
  float v = acc / L;
  if (HAD) {
    xs[c] = v;
    __syncthreads();
    for (int hh = 1; hh < D; hh <<= 1) {
      const float other = xs[c ^ hh];
      const float nv = (c & hh) ? (other - v) : (v + other);
      __syncthreads();
      xs[c] = v = nv;
      __syncthreads();
    }
    v *= (D == 128 ? 0.08838834764831845f : 0.125f);
  }
  if (a.out_bf16) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    ((uint16_t*)a.out)[(int64_t)r * D + c] = (uint16_t)(u >> 16);
  } else {
    ((float*)a.out)[(int64_t)r * D + c] = v;
  }
  if (c == 0 && a.lse != nullptr) {
    const int hq = r % a.Hq;
    const int64_t br = r / a.Hq;                 // b * Lq + row
    const int row = (int)(br % a.Lq);
    const int64_t bb = br / a.Lq;
    a.lse[(bb * a.Hq + hq) * a.Lq + row] = (M + log2f(L)) * kLn2;
  }
}

template <int D, int KM, int VM, int R>
hipError_t launch_t(const ChunkArgs& a, int B, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_rb * a.S), (unsigned)a.Hq, (unsigned)B);
  chunk_kernel<D, KM, VM, R><<<grid, kThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S == 1) return e;
  chunk_merge_kernel<D, VM != 0><<<(unsigned)((int64_t)B * a.Lq * a.Hq), D, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int KM, int VM>
hipError_t launch_r(const ChunkArgs& a, int R, int B, hipStream_t st) {
  if constexpr (KM != 0) {
    if (R == 8) return launch_t<D, KM, VM, 8>(a, B, st);
  }
  return launch_t<D, KM, VM, 0>(a, B, st);
}

template <int D, int KM>
hipError_t launch_v(const ChunkArgs& a, int value_mode, int R, int B, hipStream_t st) {
  if (value_mode == KVQ_VAL_HADAMARD_MODAL) return launch_r<D, KM, 2>(a, R, B, st);
  if (value_mode == KVQ_VAL_HADAMARD) return launch_r<D, KM, 1>(a, R, B, st);
  return launch_r<D, KM, 0>(a, R, B, st);
}

template <int D>
hipError_t launch_d(const ChunkArgs& a, int key_mode, int value_mode, int R, int B, hipStream_t st) {
  if (key_mode == KVQ_KEY_WINDOW) return launch_v<D, 0>(a, value_mode, 0, B, st);
  return launch_v<D, 1>(a, value_mode, R, B, st);
}

// Token splits.  One block of 8 waves is resident per CU; among split counts
// whose splits keep at least 16 tiles, the one with the fewest, fullest
// rounds wins (cost = rounds x (tiles per split + 4 tiles of per-block
// overhead)).
void chunk_splits(const kvq_layout* L, int q_len, int q_heads, int n_tokens, int* S, int* per) {
  const int n_tiles = (n_tokens + 63) / 64;
  const int64_t blocks = (int64_t)((q_len + kBM - 1) / kBM) * q_heads * L->batch;
  const int cus = device_cus();
  int best = 1, best_per = n_tiles > 0 ? n_tiles : 1;
  double best_cost = 1e300;
  for (int s = 1; s <= 64; ++s) {
    const int p = (n_tiles + s - 1) / s;
    if (s > 1 && p < 16) break;
    if ((n_tiles + p - 1) / p != s) continue;
    const double rounds = (double)((blocks * s + cus - 1) / cus);
    const double cost = rounds * (p + 4.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
      best_per = p;
    }
  }
  *S = best;
  *per = best_per;
}

}  // namespace

size_t chunk_workspace_bytes(const kvq_layout* L, int q_len, int q_heads, int n_tokens) {
  int S = 1, per = 1;
  chunk_splits(L, q_len, q_heads, n_tokens, &S, &per);
  if (S == 1) return 0;
  return (size_t)S * L->batch * q_len * q_heads * (L->head_dim + 2) * sizeof(float);
}

hipError_t launch_chunk(const kvq_cache* c, int n_tokens, const void* q, int q_len,
                        int q_heads, float scale, void* out, int out_dtype, float* lse,
                        void* ws, hipStream_t stream) {
  const kvq_layout& L = c->layout;
  ChunkArgs a;
  a.kcodes = (const uint8_t*)c->k_codes;
  a.kparams = (const uint32_t*)c->k_params;
  a.ktail = (const uint16_t*)c->k_tail;
  a.kidx = (const uint8_t*)c->k_idx;
  a.cent = (const float*)c->centroids;
  a.basis = (const float*)c->psac_basis;
  a.kpsac = (const uint16_t*)c->k_psac;
  a.psac_int8 = L.key_mode != KVQ_KEY_WINDOW && L.psac_rank > 0 && L.psac_format == KVQ_PSAC_INT8;
  a.kpsac_sc = a.psac_int8 ? reinterpret_cast<const uint16_t*>(
                                 reinterpret_cast<const uint8_t*>(c->k_psac) +
                                 (size_t)L.batch * L.kv_heads * L.capacity * L.psac_rank)
                           : nullptr;
  a.vcodes = (const uint8_t*)c->v_codes;
  a.vparams = (const uint32_t*)c->v_params;
  const bool modal = L.value_mode == KVQ_VAL_HADAMARD_MODAL;
  a.vsigns = modal ? (const uint32_t*)c->v_signs : nullptr;
  a.vmodal = modal ? (const uint8_t*)c->v_modality : nullptr;
  a.M = modal ? L.n_modalities : 1;
  a.q = (const uint16_t*)q;
  a.out = out;
  a.lse = lse;
  a.ws = (float*)ws;
  a.H = L.kv_heads;
  a.Hq = q_heads;
  a.Tcap = L.capacity;
  a.C = L.n_centroids;
  a.n_tokens = n_tokens;
  a.Lq = q_len;
  a.out_bf16 = out_dtype == KVQ_BF16;
  a.scale_log2 = scale * kLog2e;
  a.n_rb = (q_len + kBM - 1) / kBM;
  chunk_splits(&L, q_len, q_heads, n_tokens, &a.S, &a.tiles_per_split);
  const int R = (L.key_mode == KVQ_KEY_WINDOW) ? 0 : L.psac_rank;
  return (L.head_dim == 128) ? launch_d<128>(a, L.key_mode, L.value_mode, R, L.batch, stream)
                             : launch_d<64>(a, L.key_mode, L.value_mode, R, L.batch, stream);
}

}  // namespace kvq
