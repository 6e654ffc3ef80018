// Host-side launcher interface between the C ABI (api.cpp) and the kernel
// translation units.  Arguments reaching these functions have already been
// validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>

#include "kvint2.h"

namespace kvq {

// Largest grid y / z dimension (sequences, heads; an append's windows index x).
constexpr int kMaxGridYZ = 65535;
// Largest cache capacity per (sequence, head): token-row offsets inside one
// (sequence, head) stay within 32 bits.
constexpr int kMaxCapacity = 1 << 24;

// Compute units of the current device (queried once per device).
int device_cus();

hipError_t launch_quantize_append(const kvq_cache* c, const void* k_bf16,
                                  const void* v_bf16, int cur_len, int n_new,
                                  hipStream_t stream);

// Key side of quantize-append for centroid keys (after the values).
hipError_t launch_centroid_append(const kvq_cache* c, const void* k_bf16, int cur_len,
                                  int n_new, hipStream_t stream);

hipError_t launch_cluster_assign(const void* keys, int64_t n, int head_dim,
                                 int64_t key_stride, const float* centroids,
                                 int n_centroids, const float* sens_w, int topk,
                                 int32_t* idx_out, hipStream_t stream);

// Lloyd k-means of every (sequence, head) key set (assignment + fp64 mean
// update per round) in a workspace of kmeans_workspace_bytes() bytes.
size_t kmeans_workspace_bytes(int batch, int heads, int64_t n);
hipError_t launch_kmeans(const void* keys, int batch, int64_t n, int heads, int head_dim,
                         int64_t key_stride, int64_t head_stride, int64_t batch_stride,
                         float* centroids, int n_centroids, int iters, int32_t* assign_out,
                         void* ws, hipStream_t stream);

// Number of token splits the decode uses, and the workspace they need.
int decode_splits(const kvq_layout* L, int q_heads, int n_tokens);
size_t decode_workspace_bytes(const kvq_layout* L, int q_heads, int n_tokens);

hipError_t launch_decode(const kvq_cache* c, int n_tokens, const void* q,
                         int q_dtype, int q_heads, float scale, void* out,
                         int out_dtype, float* lse, void* ws, hipStream_t stream);

// Device address of the fixed decode scratch buffer on the current device
// (KVQ_NOALLOC_SCRATCH_BYTES bytes; looked up once per device).
hipError_t decode_scratch(void** ptr);

size_t chunk_workspace_bytes(const kvq_layout* L, int q_len, int q_heads,
                             int n_tokens);

// Top-1 cached token per query row (fp32 logits over the dequantised cache).
hipError_t launch_top1(const kvq_cache* c, int n_tokens, const void* q, int q_len, int q_heads,
                       int32_t* idx_out, float* logit_out, hipStream_t stream);
hipError_t launch_chunk(const kvq_cache* c, int n_tokens, const void* q,
                        int q_len, int q_heads, float scale, void* out,
                        int out_dtype, float* lse, void* ws, hipStream_t stream);

}  // namespace kvq
