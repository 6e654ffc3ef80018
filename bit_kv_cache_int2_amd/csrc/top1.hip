// Top-1 cached token per query row over the packed cache: the
// attention-shift diagnostic of "QuantWM: Training-Free 2-bit KV Cache
// Quantization for Stable Video World Models" (Figure 2; "Experimental
// Validation", Table 1 counts how often key quantization moves a query's
// highest-scoring history token).
//
// Logit of query row q and cached token t, in fp32: the fma chain over the
// channels in order of q_d * khat_{t,d}, then (PSAC) the chain over m of
// q'_m * a_{t,m} with q' = U^T q (fp32, channel order).  khat is
// dequantised per element in fp32: fma(code, s, z) for window keys, the
// bf16 tail as is, centroid + fma(code, s, z) for centroid keys; a is the
// fp16 coefficient or the INT8 code times its fp16 scale.  The row's token
// is the first of the largest logit.
//
// Block = 256 threads, 64 query rows of one (sequence, query head); the
// cached tokens stream through 64 at a time as a transposed fp32 LDS tile.
// Thread (rg, tg) owns rows 4 rg .. 4 rg + 3 and tile tokens 4 tg .. 4 tg + 3
// (16 chains); the sixteen threads of a row group, adjacent lanes of one
// wave, reduce their best (logit, token) at the end.  VALU-bound by design:
// a diagnostic, not a hot path.
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

struct Top1Args {
  const uint8_t* kcodes;
  const uint32_t* kparams;
  const uint16_t* ktail;
  const uint8_t* kidx;
  const float* cent;
  const float* basis;
  const uint16_t* kpsac;      // fp16 coefficients, or INT8 codes (psac_int8)
  const uint16_t* kpsac_sc;   // INT8: per-token fp16 scales
  const uint16_t* q;
  int32_t* idx_out;
  float* logit_out;
  int H, Hq, Tcap, C, n_tokens, Lq, psac_int8;
};

constexpr int kRows = 64;

template <int D, int KM, int R>
__global__ __launch_bounds__(256) void top1_kernel(const Top1Args a) {
  constexpr int NG = D / kGroup;
  __shared__ __align__(16) float qT[D][kRows];     // queries, transposed
  __shared__ __align__(16) float kT[D][kWindow];   // dequantised key tile, transposed
  __shared__ __align__(16) float pq[R > 0 ? R : 1][kRows];      // q' = U^T q
  __shared__ __align__(16) float akT[R > 0 ? R : 1][kWindow];   // PSAC coefficients

  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * kRows;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int h = hq / (a.Hq / a.H);
  const int64_t bh = (int64_t)b * a.H + h;
  const int n = a.n_tokens;

  // ---- queries (rows past the end are zero)
  for (int e = tid; e < D * kRows; e += 256) {
    const int r = e / D, d = e % D, row = row0 + r;
    qT[d][r] = row < a.Lq ? bf16_to_f32(a.q[(((int64_t)b * a.Lq + row) * a.Hq + hq) * D + d]) : 0.0f;
  }
  __syncthreads();
  if (R > 0) {
    for (int e = tid; e < R * kRows; e += 256) {
      const int r = e % kRows, m = e / kRows;
      const float* U = a.basis + bh * D * (R > 0 ? R : 1);
      float acc = 0.0f;
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(U[d * R + m], qT[d][r], acc);
      pq[m][r] = acc;
    }
  }

  const int rg = tid >> 4, tg = tid & 15;
  float bv[4];
  int bi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bv[i] = -__builtin_inff();
    bi[i] = -1;
  }
  const int n_tiles = (n + kWindow - 1) / kWindow, n_full = n / kWindow;
  // dequantisation share: token dt, channels 32 dc .. 32 dc + 31
  const int dt = tid & 63, dc = tid >> 6;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * kWindow;
    __syncthreads();   // the previous tile is consumed (and pq is visible)
    const int t = t0 + dt;
    const int64_t tr = bh * a.Tcap + t;
    if (dc < NG) {   // head_dim 64: two channel groups, threads 128.. only load PSAC
      float kv[kGroup];
      if (t >= n) {
#pragma unroll
        for (int i = 0; i < kGroup; ++i) kv[i] = 0.0f;
      } else if (KM == 0 && tile >= n_full) {
        const uint16_t* kt = a.ktail + (bh * kWindow + (t % kWindow)) * D + kGroup * dc;
#pragma unroll
        for (int i = 0; i < kGroup; ++i) kv[i] = bf16_to_f32(kt[i]);
      } else {
        const uint2 cw = *reinterpret_cast<const uint2*>(a.kcodes + tr * (D / 4) + 8 * dc);
        if (KM == 0) {
          const uint32_t* pw = a.kparams + (bh * (a.Tcap / kWindow) + tile) * D + kGroup * dc;
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            const uint32_t code = ((i < 16 ? cw.x : cw.y) >> (2 * (i & 15))) & 3u;
            kv[i] = __builtin_fmaf((float)code, f16_bits_to_f32(pw[i] & 0xFFFFu),
                                   f16_bits_to_f32(pw[i] >> 16));
          }
        } else {
          const uint32_t pw = a.kparams[tr * NG + dc];
          const float s = f16_bits_to_f32(pw & 0xFFFFu), z = f16_bits_to_f32(pw >> 16);
          const float* cr = a.cent + (bh * a.C + a.kidx[tr]) * D + kGroup * dc;
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            const uint32_t code = ((i < 16 ? cw.x : cw.y) >> (2 * (i & 15))) & 3u;
            kv[i] = cr[i] + __builtin_fmaf((float)code, s, z);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) kT[kGroup * dc + i][dt] = kv[i];
    }
    if (R > 0) {
      for (int m = dc; m < R; m += 4) {
        float am = 0.0f;
        if (t < n) {
          if (a.psac_int8)
            am = (float)reinterpret_cast<const int8_t*>(a.kpsac)[tr * R + m] *
                 f16_bits_to_f32(a.kpsac_sc[tr]);
          else
            am = f16_bits_to_f32(a.kpsac[tr * R + m]);
        }
        akT[m][dt] = am;
      }
    }
    __syncthreads();
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      const float4 q4 = *reinterpret_cast<const float4*>(&qT[d][4 * rg]);
      const float4 k4 = *reinterpret_cast<const float4*>(&kT[d][4 * tg]);
      const float qa[4] = {q4.x, q4.y, q4.z, q4.w}, ka[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(qa[i], ka[j], acc[i][j]);
    }
    if (R > 0) {
#pragma unroll
      for (int m = 0; m < (R > 0 ? R : 1); ++m) {
        const float4 q4 = *reinterpret_cast<const float4*>(&pq[m][4 * rg]);
        const float4 k4 = *reinterpret_cast<const float4*>(&akT[m][4 * tg]);
        const float qa[4] = {q4.x, q4.y, q4.z, q4.w}, ka[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(qa[i], ka[j], acc[i][j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 4 * tg + j;
      if (t < n) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (bi[i] < 0 || acc[i][j] > bv[i]) {
            bv[i] = acc[i][j];
            bi[i] = t;
          }
      }
    }
  }
  // ---- the row group's sixteen lanes: largest logit, then the lower token
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float v = __shfl_xor(bv[i], o, 64);
      const int x = __shfl_xor(bi[i], o, 64);
      if (x >= 0 && (bi[i] < 0 || v > bv[i] || (v == bv[i] && x < bi[i]))) {
        bv[i] = v;
        bi[i] = x;
      }
    }
  }
  if (tg == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 4 * rg + i;
      if (row < a.Lq) {
        const int64_t o = ((int64_t)b * a.Hq + hq) * a.Lq + row;
        a.idx_out[o] = bi[i];
        if (a.logit_out) a.logit_out[o] = bv[i];
      }
    }
  }
}

template <int D, int KM>
hipError_t launch_km(const Top1Args& a, int R, dim3 grid, hipStream_t st) {
  if (R == 8) top1_kernel<D, KM, 8><<<grid, 256, 0, st>>>(a);
  else top1_kernel<D, KM, 0><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Top1Args& a, int key_mode, int R, dim3 grid, hipStream_t st) {
  return key_mode == KVQ_KEY_WINDOW ? launch_km<D, 0>(a, 0, grid, st) : launch_km<D, 1>(a, R, grid, st);
}

}  // namespace

hipError_t launch_top1(const kvq_cache* c, int n_tokens, const void* q, int q_len, int q_heads,
                       int32_t* idx_out, float* logit_out, hipStream_t stream) {
  const kvq_layout& L = c->layout;
  Top1Args a;
  a.kcodes = (const uint8_t*)c->k_codes;
  a.kparams = (const uint32_t*)c->k_params;
  a.ktail = (const uint16_t*)c->k_tail;
  a.kidx = (const uint8_t*)c->k_idx;
  a.cent = (const float*)c->centroids;
  a.basis = (const float*)c->psac_basis;
  a.kpsac = (const uint16_t*)c->k_psac;
  const int R = (L.key_mode == KVQ_KEY_WINDOW) ? 0 : L.psac_rank;
  a.psac_int8 = R > 0 && L.psac_format == KVQ_PSAC_INT8;
  a.kpsac_sc = a.psac_int8 ? reinterpret_cast<const uint16_t*>(
                                 reinterpret_cast<const uint8_t*>(c->k_psac) +
                                 (size_t)L.batch * L.kv_heads * L.capacity * R)
                           : nullptr;
  a.q = (const uint16_t*)q;
  a.idx_out = idx_out;
  a.logit_out = logit_out;
  a.H = L.kv_heads;
  a.Hq = q_heads;
  a.Tcap = L.capacity;
  a.C = L.n_centroids;
  a.n_tokens = n_tokens;
  a.Lq = q_len;
  const dim3 grid((unsigned)((q_len + kRows - 1) / kRows), (unsigned)q_heads, (unsigned)L.batch);
  return L.head_dim == 128 ? launch_d<128>(a, L.key_mode, R, grid, stream)
                           : launch_d<64>(a, L.key_mode, R, grid, stream);
}

}  // namespace kvq
