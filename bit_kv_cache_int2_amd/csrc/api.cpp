// The kvint2 C ABI: argument validation, buffer sizes and dispatch.
// Everything here runs on the host; nothing is launched until every check
// has passed, so error returns leave all outputs untouched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "internal.h"
#include "kvint2.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_layout(const kvq_layout* L) {
  if (!L) return KVQ_EINVAL;
  if (L->batch < 1 || L->kv_heads < 1 || L->capacity < KVQ_WINDOW ||
      L->capacity % KVQ_WINDOW != 0)
    return KVQ_EINVAL;
  if (L->key_mode < KVQ_KEY_WINDOW || L->key_mode > KVQ_KEY_CENTROID_QSAC) return KVQ_EINVAL;
  if (L->value_mode != KVQ_VAL_GROUP && L->value_mode != KVQ_VAL_HADAMARD &&
      L->value_mode != KVQ_VAL_HADAMARD_MODAL)
    return KVQ_EINVAL;
  if (L->value_mode == KVQ_VAL_HADAMARD_MODAL && (L->n_modalities < 1 || L->n_modalities > 3))
    return KVQ_EUNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return KVQ_EUNSUPPORTED;
  if (L->key_mode != KVQ_KEY_WINDOW) {
    if (L->n_centroids < 1 || L->n_centroids > 256) return KVQ_EUNSUPPORTED;
    if (L->psac_rank != 0 && L->psac_rank != 8) return KVQ_EUNSUPPORTED;
  } else if (L->psac_rank != 0) {
    return KVQ_EUNSUPPORTED;
  }
  if (L->key_mode == KVQ_KEY_CENTROID_QSAC &&
      (L->qsac_topk < 1 || L->qsac_topk > 8 || L->qsac_topk > L->n_centroids))
    return KVQ_EINVAL;
  if (L->key_mode == KVQ_KEY_CENTROID_QSAC && L->qsac_score != KVQ_QSAC_EXACT &&
      L->qsac_score != KVQ_QSAC_RANGE)
    return KVQ_EINVAL;
  if (L->psac_rank > 0 && L->psac_format != KVQ_PSAC_F16 && L->psac_format != KVQ_PSAC_INT8)
    return KVQ_EINVAL;
  if (L->key_mode != KVQ_KEY_WINDOW && L->centroid_key_split != 0 && L->centroid_key_split != 1)
    return KVQ_EINVAL;
  if ((int64_t)L->batch * L->kv_heads * L->capacity > ((int64_t)1 << 40)) return KVQ_EINVAL;
  // grid dimensions (sequences and heads index grid y/z, at most 65535) and
  // 32-bit token-row offsets within one (sequence, head)
  if (L->batch > kvq::kMaxGridYZ || L->kv_heads > kvq::kMaxGridYZ) return KVQ_EUNSUPPORTED;
  if (L->capacity > kvq::kMaxCapacity) return KVQ_EUNSUPPORTED;
  return KVQ_OK;
}

bool uses(const kvq_layout* L, int which) {
  const bool win = L->key_mode == KVQ_KEY_WINDOW;
  switch (which) {
    case KVQ_BUF_K_CODES:
    case KVQ_BUF_K_PARAMS:
    case KVQ_BUF_V_CODES:
    case KVQ_BUF_V_PARAMS: return true;
    case KVQ_BUF_K_TAIL: return win;
    case KVQ_BUF_K_IDX:
    case KVQ_BUF_CENTROIDS: return !win;
    case KVQ_BUF_SENS_W: return L->key_mode == KVQ_KEY_CENTROID_QSAC;
    case KVQ_BUF_PSAC_BASIS:
    case KVQ_BUF_K_PSAC: return !win && L->psac_rank > 0;
    case KVQ_BUF_V_SIGNS:
    case KVQ_BUF_V_MODALITY: return L->value_mode == KVQ_VAL_HADAMARD_MODAL;
    default: return false;
  }
}

const void* buf(const kvq_cache* c, int which) {
  switch (which) {
    case KVQ_BUF_K_CODES: return c->k_codes;
    case KVQ_BUF_K_PARAMS: return c->k_params;
    case KVQ_BUF_K_TAIL: return c->k_tail;
    case KVQ_BUF_K_IDX: return c->k_idx;
    case KVQ_BUF_CENTROIDS: return c->centroids;
    case KVQ_BUF_SENS_W: return c->sens_w;
    case KVQ_BUF_PSAC_BASIS: return c->psac_basis;
    case KVQ_BUF_K_PSAC: return c->k_psac;
    case KVQ_BUF_V_CODES: return c->v_codes;
    case KVQ_BUF_V_PARAMS: return c->v_params;
    case KVQ_BUF_V_SIGNS: return c->v_signs;
    case KVQ_BUF_V_MODALITY: return c->v_modality;
    default: return nullptr;
  }
}

int check_cache(const kvq_cache* c) {
  if (!c) return KVQ_EINVAL;
  const int st = check_layout(&c->layout);
  if (st != KVQ_OK) return st;
  for (int w = 0; w < KVQ_BUF_COUNT; ++w)
    if (uses(&c->layout, w) && (!buf(c, w) || !aligned16(buf(c, w)))) return KVQ_EINVAL;
  return KVQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_EHIP; }

int check_attention(const kvq_cache* c, int32_t n_tokens, const void* q, int32_t q_heads,
                    const void* out, int32_t out_dtype, const void* lse) {
  const int st = check_cache(c);
  if (st != KVQ_OK) return st;
  const kvq_layout& L = c->layout;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return KVQ_EINVAL;
  if (lse && ((uintptr_t)lse & 3u)) return KVQ_EINVAL;
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16) return KVQ_EINVAL;
  if (q_heads < 1 || q_heads % L.kv_heads != 0) return KVQ_EINVAL;
  const int G = q_heads / L.kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVQ_EUNSUPPORTED;
  if (q_heads > kvq::kMaxGridYZ) return KVQ_EUNSUPPORTED;
  if (n_tokens < 1) return KVQ_EINVAL;
  if (n_tokens > L.capacity) return KVQ_ECAPACITY;
  return KVQ_OK;
}

}  // namespace

namespace kvq {

// Compute units of the current device, queried once per device.
int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDev) {
    const int v = cus[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  if (dev >= 0 && dev < kMaxDev) cus[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace kvq

extern "C" {

int kvq_layout_check(const kvq_layout* L) { return check_layout(L); }

size_t kvq_buffer_bytes(const kvq_layout* L, int32_t which) {
  if (check_layout(L) != KVQ_OK || which < 0 || which >= KVQ_BUF_COUNT || !uses(L, which))
    return 0;
  const size_t BH = (size_t)L->batch * L->kv_heads, T = (size_t)L->capacity,
               D = (size_t)L->head_dim;
  switch (which) {
    case KVQ_BUF_K_CODES:
    case KVQ_BUF_V_CODES: return BH * T * (D / 4);
    case KVQ_BUF_K_PARAMS:
      return L->key_mode == KVQ_KEY_WINDOW ? BH * (T / KVQ_WINDOW) * D * 4
                                           : BH * T * (D / KVQ_GROUP) * 4;
    case KVQ_BUF_V_PARAMS: return BH * T * (D / KVQ_GROUP) * 4;
    case KVQ_BUF_V_SIGNS: return (size_t)L->kv_heads * L->n_modalities * (D / 32) * 4;
    case KVQ_BUF_V_MODALITY: return (size_t)L->batch * T;
    case KVQ_BUF_K_TAIL: return BH * KVQ_WINDOW * D * 2;
    case KVQ_BUF_K_IDX: return BH * T;
    case KVQ_BUF_CENTROIDS: return BH * (size_t)L->n_centroids * D * 4;
    case KVQ_BUF_SENS_W: return BH * D * 4;
    case KVQ_BUF_PSAC_BASIS: return BH * D * (size_t)L->psac_rank * 4;
    case KVQ_BUF_K_PSAC:
      return L->psac_format == KVQ_PSAC_INT8 ? BH * T * ((size_t)L->psac_rank + 2)
                                             : BH * T * (size_t)L->psac_rank * 2;
    default: return 0;
  }
}

int kv_quantize_append(const kvq_cache* cache, const void* k_bf16, const void* v_bf16,
                       int32_t cur_len, int32_t n_new, void* stream) {
  const int st = check_cache(cache);
  if (st != KVQ_OK) return st;
  if (cur_len < 0 || n_new < 0) return KVQ_EINVAL;
  if ((int64_t)cur_len + n_new > cache->layout.capacity) return KVQ_ECAPACITY;
  if (n_new == 0) return KVQ_OK;
  if (!k_bf16 || !v_bf16 || !aligned16(k_bf16) || !aligned16(v_bf16)) return KVQ_EINVAL;
  // the windows an append touches index grid x (up to 2^31 - 1 blocks), so
  // the capacity limit of check_cache bounds them
  return hip_status(kvq::launch_quantize_append(cache, k_bf16, v_bf16, cur_len, n_new,
                                                (hipStream_t)stream));
}

int kv_cluster_assign(const void* keys, int64_t n, int32_t head_dim, int64_t key_stride,
                      const float* centroids, int32_t n_centroids, const float* sens_w,
                      int32_t topk, int32_t* idx_out, void* stream) {
  if (n < 0) return KVQ_EINVAL;
  if (head_dim != 64 && head_dim != 128) return KVQ_EUNSUPPORTED;
  if (n_centroids < 1 || n_centroids > 256) return KVQ_EUNSUPPORTED;
  if (n == 0) return KVQ_OK;
  if (!keys || !centroids || !idx_out || !aligned16(keys) || !aligned16(centroids) ||
      ((uintptr_t)idx_out & 3u))
    return KVQ_EINVAL;
  if (key_stride < head_dim || key_stride % 8 != 0) return KVQ_EINVAL;
  if (n > ((int64_t)1 << 31) - 256) return KVQ_EINVAL;
  if (sens_w && (topk < 1 || topk > 8 || ((uintptr_t)sens_w & 15u))) return KVQ_EINVAL;
  return hip_status(kvq::launch_cluster_assign(keys, n, head_dim, key_stride, centroids,
                                               n_centroids, sens_w, topk, idx_out,
                                               (hipStream_t)stream));
}

size_t kv_kmeans_workspace(int32_t batch, int32_t heads, int64_t n) {
  if (batch < 0 || heads < 0 || n < 0 || n > ((int64_t)1 << 31) - 256) return 0;
  return kvq::kmeans_workspace_bytes(batch, heads, n);
}

int kv_kmeans(const void* keys, int32_t batch, int64_t n, int32_t heads, int32_t head_dim,
              int64_t key_stride, int64_t head_stride, int64_t batch_stride, float* centroids,
              int32_t n_centroids, int32_t iters, int32_t* assign_out, void* ws, size_t ws_bytes,
              void* stream) {
  if (n < 0 || batch < 0 || heads < 0 || iters < 0) return KVQ_EINVAL;
  if (head_dim != 64 && head_dim != 128) return KVQ_EUNSUPPORTED;
  if (n_centroids < 1 || n_centroids > 256) return KVQ_EUNSUPPORTED;
  if (batch > 65535 || heads > 65535) return KVQ_EUNSUPPORTED;   // grid dimensions
  if (n == 0 || batch == 0 || heads == 0) return KVQ_OK;
  if (!keys || !centroids || !aligned16(keys) || !aligned16(centroids) ||
      ((uintptr_t)assign_out & 3u))
    return KVQ_EINVAL;
  if (key_stride < head_dim || key_stride % 8 != 0 || head_stride < 0 || head_stride % 8 != 0 ||
      batch_stride < 0 || batch_stride % 8 != 0)
    return KVQ_EINVAL;
  if (n > ((int64_t)1 << 31) - 256) return KVQ_EINVAL;
  const size_t need = kv_kmeans_workspace(batch, heads, n);
  if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < need) return KVQ_EWORKSPACE;
  return hip_status(kvq::launch_kmeans(keys, batch, n, heads, head_dim, key_stride, head_stride,
                                       batch_stride, centroids, n_centroids, iters, assign_out,
                                       ws, (hipStream_t)stream));
}

size_t attn_int2_decode_workspace(const kvq_layout* L, int32_t q_heads, int32_t n_tokens) {
  if (check_layout(L) != KVQ_OK || q_heads < 1 || n_tokens < 1) return 0;
  return kvq::decode_workspace_bytes(L, q_heads, n_tokens);
}

int attn_int2_decode(const kvq_cache* cache, int32_t n_tokens, const void* q, int32_t q_dtype,
                     int32_t q_heads, float scale, void* out, int32_t out_dtype, float* lse,
                     void* ws, size_t ws_bytes, void* stream) {
  int st = check_attention(cache, n_tokens, q, q_heads, out, out_dtype, lse);
  if (st != KVQ_OK) return st;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_EINVAL;
  const size_t need = kvq::decode_workspace_bytes(&cache->layout, q_heads, n_tokens);
  if (!ws || !aligned16(ws) || ws_bytes < need) return KVQ_EWORKSPACE;
  return hip_status(kvq::launch_decode(cache, n_tokens, q, q_dtype, q_heads, scale, out,
                                       out_dtype, lse, ws, (hipStream_t)stream));
}

int attn_int2_decode_noalloc(const kvq_cache* cache, int32_t n_tokens, const void* q,
                             int32_t q_dtype, int32_t q_heads, float scale, void* out,
                             int32_t out_dtype, float* lse, void* stream) {
  int st = check_attention(cache, n_tokens, q, q_heads, out, out_dtype, lse);
  if (st != KVQ_OK) return st;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_EINVAL;
  if (kvq::decode_workspace_bytes(&cache->layout, q_heads, n_tokens) > KVQ_NOALLOC_SCRATCH_BYTES)
    return KVQ_ESCRATCH;
  void* ws = nullptr;
  if (kvq::decode_scratch(&ws) != hipSuccess || !ws) return KVQ_EHIP;
  return hip_status(kvq::launch_decode(cache, n_tokens, q, q_dtype, q_heads, scale, out,
                                       out_dtype, lse, ws, (hipStream_t)stream));
}

size_t attn_int2_chunk_workspace(const kvq_layout* L, int32_t q_len, int32_t q_heads,
                                 int32_t n_tokens) {
  if (check_layout(L) != KVQ_OK || q_heads < 1 || n_tokens < 1 || q_len < 1) return 0;
  return kvq::chunk_workspace_bytes(L, q_len, q_heads, n_tokens);
}

int attn_int2_chunk(const kvq_cache* cache, int32_t n_tokens, const void* q, int32_t q_len,
                    int32_t q_heads, float scale, void* out, int32_t out_dtype, float* lse,
                    void* ws, size_t ws_bytes, void* stream) {
  int st = check_attention(cache, n_tokens, q, q_heads, out, out_dtype, lse);
  if (st != KVQ_OK) return st;
  if (q_len < 1) return KVQ_EINVAL;
  const size_t need = kvq::chunk_workspace_bytes(&cache->layout, q_len, q_heads, n_tokens);
  if (need > 0 && (!ws || !aligned16(ws) || ws_bytes < need)) return KVQ_EWORKSPACE;
  return hip_status(kvq::launch_chunk(cache, n_tokens, q, q_len, q_heads, scale, out,
                                      out_dtype, lse, ws, (hipStream_t)stream));
}

int attn_int2_top1(const kvq_cache* cache, int32_t n_tokens, const void* q, int32_t q_len,
                   int32_t q_heads, int32_t* idx_out, float* logit_out, void* stream) {
  int st = check_attention(cache, n_tokens, q, q_heads, idx_out, KVQ_F32, logit_out);
  if (st != KVQ_OK) return st;
  if (q_len < 1) return KVQ_EINVAL;
  if (cache->layout.batch > 65535 || q_heads > 65535) return KVQ_EUNSUPPORTED;
  return hip_status(kvq::launch_top1(cache, n_tokens, q, q_len, q_heads, idx_out, logit_out,
                                     (hipStream_t)stream));
}

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_ECAPACITY: return "exceeds cache capacity";
    case KVQ_EWORKSPACE: return "workspace missing or too small";
    case KVQ_EHIP: return "HIP launch error";
    case KVQ_ESCRATCH: return "exceeds the fixed scratch buffer of the allocation-free decode";
    default: return "unknown status";
  }
}

}  // extern "C"
