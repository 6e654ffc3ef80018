// Quantise-append into the packed INT2 cache, and centroid assignment.
//
//  * values ([OKV] rotated values, optional): one token row per D/8 lanes,
//    8 channels (16 bytes of bf16) per lane, so a 32-channel parameter group
//    is one lane quad and its min/max is two xor-shuffles.  The
//    Walsh-Hadamard rotation runs in registers: three in-lane butterfly
//    stages, then one xor-shuffle stage per remaining bit.
//  * window keys ([OKV] per-window key ranges): one 256-thread block per
//    (64-token window, sequence, head); the window is staged in LDS, each
//    channel's min/max is a column scan, codes are packed row-wise and
//    written as contiguous 8-byte pieces.  The block of the first window also
//    writes the new tail after it has read the old one, so the two never race.
//  * centroid keys ([QWM] 1): one lane per token keeps its key in registers
//    and scans centroids staged 64 at a time in LDS (broadcast reads), in
//    index order with the channel-order fp32 distance; QSAC keeps the best
//    candidates in a sorted register list and scores each candidate's INT2
//    residual; PSAC coefficients accumulate in channel order as the chosen
//    residual is quantised.
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------- values
// Walsh-Hadamard rotation of one token row spread over D/8 lanes (8
// elements per lane, element index = lane-in-row * 8 + k).  Stages run with
// h = 1, 2, 4 in-lane and then h = 8, 16, ... across lanes, each pair (i,
// i+h) becoming (a+b, a-b); finally every element is scaled by
// fp32(1/sqrt(D)) and canonicalised.
template <int D>
KVQ_DEV void wht_row(float (&x)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((k & h) == 0) {
        const float a = x[k], b = x[k + h];
        x[k] = a + b;
        x[k + h] = a - b;
      }
    }
  }
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 1; s < D / 8; s <<= 1) {
    const bool upper = (lane & s) != 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float o = __shfl_xor(x[k], s, 64);
      x[k] = upper ? (o - x[k]) : (x[k] + o);
    }
  }
  const float c = __uint_as_float(D == 128 ? 0x3DB504F3u : 0x3E000000u);
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = x[k] * c + 0.0f;
}

// Quantise the 8-channel slice this lane holds of one token row (a row is
// spread over D/8 consecutive lanes, so every lane of the row must take
// part; `ok` false lanes only join the shuffles).
template <int D, bool HAD>
KVQ_DEV void value_slice(const uint16_t* src, bool ok, int j, uint8_t* code_row,
                         uint32_t* prm_row) {
  float x[8];
  if (ok) {
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(src + j * 8), x);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.0f;
  }
  if (HAD) wht_row<D>(x);
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    mn = fminf(mn, x[k]);
    mx = fmaxf(mx, x[k]);
  }
  mn = fminf(mn, __shfl_xor(mn, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  mn = fminf(mn, __shfl_xor(mn, 2, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  const Q2 q = q2_make(mn, mx);
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) bits |= q2_code(x[k], q) << (2 * k);
  if (ok) {
    *reinterpret_cast<uint16_t*>(code_row + j * 2) = (uint16_t)bits;
    if ((j & 3) == 0) prm_row[j >> 2] = q.word;
  }
}

// Values only (centroid-key modes): rows (b, h, i) with i fastest.
template <int D, bool HAD>
__global__ __launch_bounds__(256) void quant_values_kernel(
    const uint16_t* __restrict__ vin, uint8_t* __restrict__ vcodes,
    uint32_t* __restrict__ vparams, int H, int Tcap, int cur_len, int n_new,
    int64_t rows) {
  constexpr int LPR = D / 8;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int j = threadIdx.x & (LPR - 1);
  const bool ok = row < rows;
  const int64_t i = ok ? row % n_new : 0, bh = ok ? row / n_new : 0;
  const int64_t h = bh % H, b = bh / H;
  const int64_t orow = bh * Tcap + cur_len + i;
  value_slice<D, HAD>(vin + ((b * n_new + i) * H + h) * D, ok, j, vcodes + orow * (D / 4),
                      vparams + orow * (D / kGroup));
}

// ---------------------------------------------------------------- window keys
// One block per (64-token window touched by the append, head, sequence):
// the window's new value rows, then -- if the append completes the window --
// its keys, quantised per channel over the 64 tokens (old tokens from the
// tail, new ones from the input).  Block 0 also writes the tokens of the
// window left unfinished into the tail, after its own reads of the old tail.
template <int D, bool HAD>
__global__ __launch_bounds__(256) void window_append_kernel(
    const uint16_t* __restrict__ kin, const uint16_t* __restrict__ vin,
    uint8_t* __restrict__ kcodes, uint32_t* __restrict__ kparams,
    uint16_t* __restrict__ ktail, uint8_t* __restrict__ vcodes,
    uint32_t* __restrict__ vparams, int H, int Tcap, int cur_len, int n_new) {
  constexpr int LPR = D / 8, RPP = 256 / LPR;  // lanes per row, rows per pass
  constexpr int PARTS = 256 / D;              // threads per channel
  constexpr int TPP = kWindow / PARTS;        // tokens per thread
  __shared__ __align__(16) uint16_t tile[kWindow][D + 8];
  __shared__ __align__(16) uint8_t codes[kWindow][D];
  __shared__ float red_mn[PARTS][D], red_mx[PARTS][D];

  const int job = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * H + h;
  const int end = cur_len + n_new;
  const int tid = threadIdx.x;
  const int w = cur_len / kWindow + job;
  const int t_lo = max(w * kWindow, cur_len), t_hi = min(w * kWindow + kWindow, end);
  const uint16_t* tail = ktail + bh * kWindow * D;

  for (int base = t_lo; base < t_hi; base += RPP) {
    const int t = base + tid / LPR;
    const bool ok = t < t_hi;
    const int64_t orow = bh * Tcap + (ok ? t : t_lo);
    value_slice<D, HAD>(vin + (((int64_t)b * n_new + (t - cur_len)) * H + h) * D, ok,
                        tid % LPR, vcodes + orow * (D / 4), vparams + orow * (D / kGroup));
  }

  if (w * kWindow + kWindow <= end) {
    for (int e = tid; e < kWindow * D / 8; e += 256) {
      const int t = e / (D / 8), jj = e % (D / 8);
      const int p = w * kWindow + t;
      const uint16_t* src =
          (p < cur_len) ? tail + (int64_t)(p & (kWindow - 1)) * D
                        : kin + (((int64_t)b * n_new + (p - cur_len)) * H + h) * D;
      *reinterpret_cast<uint4*>(&tile[t][jj * 8]) = *reinterpret_cast<const uint4*>(src + jj * 8);
    }
    __syncthreads();
    const int c = tid % D, part = tid / D;
    float mn = bf16_to_f32(tile[part * TPP][c]) + 0.0f, mx = mn;
    for (int t = part * TPP + 1; t < (part + 1) * TPP; ++t) {
      const float x = bf16_to_f32(tile[t][c]) + 0.0f;
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    red_mn[part][c] = mn;
    red_mx[part][c] = mx;
    __syncthreads();
#pragma unroll
    for (int p2 = 0; p2 < PARTS; ++p2) {
      mn = fminf(mn, red_mn[p2][c]);
      mx = fmaxf(mx, red_mx[p2][c]);
    }
    const Q2 q = q2_make(mn, mx);
    for (int t = part * TPP; t < (part + 1) * TPP; ++t)
      codes[t][c] = (uint8_t)q2_code(bf16_to_f32(tile[t][c]) + 0.0f, q);
    if (part == 0) kparams[(bh * (Tcap / kWindow) + w) * D + c] = q.word;
    __syncthreads();
    // pack: each thread emits 8 bytes (32 codes) of one token row
    for (int e = tid; e < kWindow * (D / 32); e += 256) {
      const int t = e / (D / 32), qd = e % (D / 32);
      const uint4 c0 = *reinterpret_cast<const uint4*>(&codes[t][qd * 32]);
      const uint4 c1 = *reinterpret_cast<const uint4*>(&codes[t][qd * 32 + 16]);
      const uint32_t in[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      uint32_t outw[2] = {0u, 0u};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // four one-byte codes -> one packed byte
        const uint32_t v = in[k];
        const uint32_t byte = (v & 3u) | ((v >> 6) & 0xCu) | ((v >> 12) & 0x30u) | ((v >> 18) & 0xC0u);
        outw[k >> 2] |= byte << (8 * (k & 3));
      }
      *reinterpret_cast<uint2*>(kcodes + (bh * Tcap + (int64_t)w * kWindow + t) * (D / 4) + qd * 8) =
          make_uint2(outw[0], outw[1]);
    }
  }
  if (job == 0) {
    __syncthreads();  // the first window has read the old tail
    int ts = (end / kWindow) * kWindow;
    if (ts < cur_len) ts = cur_len;
    uint16_t* tw = ktail + bh * kWindow * D;
    for (int e = tid; e < (end - ts) * (D / 8); e += 256) {
      const int p = ts + e / (D / 8), jj = e % (D / 8);
      const uint4 u = *reinterpret_cast<const uint4*>(
          kin + (((int64_t)b * n_new + (p - cur_len)) * H + h) * D + jj * 8);
      *reinterpret_cast<uint4*>(tw + (int64_t)(p & (kWindow - 1)) * D + jj * 8) = u;
    }
  }
}

// ---------------------------------------------------------------- centroids
constexpr int kCandMax = 8;
constexpr int kChunk = 64;  // centroids staged in LDS at a time

// INT2-quantise the residual r = k - c per group of 32 (inputs
// canonicalised), returning the weighted squared error of the dequantised
// residual (fp32, channel order; 0 when w == nullptr).  Optionally emits the
// packed codes, the parameter words and the PSAC accumulators.
template <int D, int R, bool EMIT>
KVQ_DEV float residual_q2(const float (&k)[D], const float* __restrict__ c,
                          const float* w, const float* U, uint32_t* codes,
                          uint32_t* prm, float* pacc) {
  float E = 0.0f;
#pragma unroll
  for (int g = 0; g < D / kGroup; ++g) {
    float r[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; i += 4) {
      const float4 c4 = *reinterpret_cast<const float4*>(c + g * kGroup + i);
      r[i] = (k[g * kGroup + i] - c4.x) + 0.0f;
      r[i + 1] = (k[g * kGroup + i + 1] - c4.y) + 0.0f;
      r[i + 2] = (k[g * kGroup + i + 2] - c4.z) + 0.0f;
      r[i + 3] = (k[g * kGroup + i + 3] - c4.w) + 0.0f;
    }
    float mn = r[0], mx = r[0];
#pragma unroll
    for (int i = 1; i < kGroup; ++i) {
      mn = fminf(mn, r[i]);
      mx = fmaxf(mx, r[i]);
    }
    const Q2 q = q2_make(mn, mx);
    if (EMIT) prm[g] = q.word;
    uint32_t wlo = 0, whi = 0;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const uint32_t code = q2_code(r[i], q);
      if (i < 16) wlo |= code << (2 * i);
      else whi |= code << (2 * (i - 16));
      const float e = r[i] - __builtin_fmaf((float)code, q.s, q.z);
      const int d = g * kGroup + i;
      if (w != nullptr) {
        const float we = w[d] * e;
        E = __builtin_fmaf(we, e, E);
      }
      if (EMIT && R > 0) {
#pragma unroll
        for (int m = 0; m < R; ++m) pacc[m] = __builtin_fmaf(U[d * R + m], e, pacc[m]);
      }
    }
    if (EMIT) {
      codes[2 * g] = wlo;
      codes[2 * g + 1] = whi;
    }
  }
  return E;
}

// One lane per key.  TO_CACHE: write idx/codes/params/PSAC into the cache
// rows at cur_len + i; otherwise write the i32 index to idx_out.
template <int D, bool QSAC, int R, bool TO_CACHE>
__global__ __launch_bounds__(256) void centroid_kernel(
    const uint16_t* __restrict__ kin, int64_t key_stride, int64_t head_stride,
    int64_t batch_stride, int64_t n, const float* __restrict__ cent, int C,
    const float* __restrict__ sens_w, int topk, const float* __restrict__ basis,
    int32_t* __restrict__ idx_out, uint8_t* __restrict__ kidx,
    uint8_t* __restrict__ kcodes, uint32_t* __restrict__ kparams,
    uint16_t* __restrict__ kpsac, int H, int Tcap, int cur_len) {
  __shared__ float cs[kChunk * D];
  __shared__ float wl[D];
  __shared__ float ul[D * (R > 0 ? R : 1)];
  const int tid = threadIdx.x;
  const int64_t bh = (int64_t)blockIdx.z * H + blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + tid;
  const bool ok = i < n;
  const float* cb = cent + bh * (int64_t)C * D;

  float k[D];
  if (ok) {
    const uint16_t* src = kin + blockIdx.z * batch_stride + i * key_stride + blockIdx.y * head_stride;
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      float x[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(src + j * 8), x);
#pragma unroll
      for (int t = 0; t < 8; ++t) k[j * 8 + t] = x[t];
    }
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) k[d] = 0.0f;
  }
  if (QSAC)
    for (int d = tid; d < D; d += 256) wl[d] = sens_w[bh * D + d];
  if (R > 0)
    for (int d = tid; d < D * R; d += 256) ul[d] = basis[bh * D * R + d];

  float bd = __builtin_inff();
  int best = 0;
  float cd[kCandMax];
  int cj[kCandMax];
#pragma unroll
  for (int t = 0; t < kCandMax; ++t) {
    cd[t] = __builtin_inff();
    cj[t] = 0;
  }
  for (int c0 = 0; c0 < C; c0 += kChunk) {
    const int nc = min(kChunk, C - c0);
    __syncthreads();
    for (int e = tid * 4; e < nc * D; e += 1024)
      *reinterpret_cast<float4*>(cs + e) = *reinterpret_cast<const float4*>(cb + (int64_t)c0 * D + e);
    __syncthreads();
    for (int jj = 0; jj < nc; ++jj) {
      const float* cr = cs + jj * D;
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 c4 = *reinterpret_cast<const float4*>(cr + d);
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float t = k[d + u] - cc[u];
          if (QSAC) {
            const float wt = wl[d + u] * t;
            acc = __builtin_fmaf(wt, t, acc);
          } else {
            acc = __builtin_fmaf(t, t, acc);
          }
        }
      }
      const int j = c0 + jj;
      if (QSAC) {
        float vd = acc;
        int vj = j;
#pragma unroll
        for (int t = 0; t < kCandMax; ++t) {
          if (vd < cd[t]) {
            const float td = cd[t];
            const int tj = cj[t];
            cd[t] = vd;
            cj[t] = vj;
            vd = td;
            vj = tj;
          }
        }
      } else if (acc < bd) {
        bd = acc;
        best = j;
      }
    }
  }
  if (QSAC) {
    float bE = 0.0f;
    best = -1;
#pragma unroll
    for (int t = 0; t < kCandMax; ++t) {
      if (t < topk && t < C) {
        const int j = cj[t];
        const float E = residual_q2<D, 0, false>(k, cb + (int64_t)j * D, wl, nullptr,
                                                 nullptr, nullptr, nullptr);
        if (best < 0 || E < bE || (E == bE && j < best)) {
          best = j;
          bE = E;
        }
      }
    }
  }
  if (!ok) return;
  if (!TO_CACHE) {
    idx_out[i] = best;
    return;
  }
  uint32_t codes[D / 16];
  uint32_t prm[D / kGroup];
  float pacc[R > 0 ? R : 1];
#pragma unroll
  for (int m = 0; m < (R > 0 ? R : 1); ++m) pacc[m] = 0.0f;
  residual_q2<D, R, true>(k, cb + (int64_t)best * D, nullptr, ul, codes, prm, pacc);
  const int64_t orow = bh * Tcap + cur_len + i;
  kidx[orow] = (uint8_t)best;
  uint4* cdst = reinterpret_cast<uint4*>(kcodes + orow * (D / 4));
#pragma unroll
  for (int q = 0; q < D / 64; ++q)
    cdst[q] = make_uint4(codes[4 * q], codes[4 * q + 1], codes[4 * q + 2], codes[4 * q + 3]);
  uint32_t* pdst = kparams + orow * (D / kGroup);
#pragma unroll
  for (int g = 0; g < D / kGroup; ++g) pdst[g] = prm[g];
  if (R > 0) {
    uint32_t hw[(R > 0 ? R : 2) / 2];
#pragma unroll
    for (int m = 0; m < R; m += 2)
      hw[m / 2] = f32_to_f16_bits(pacc[m]) | (f32_to_f16_bits(pacc[m + 1]) << 16);
    uint32_t* ps = reinterpret_cast<uint32_t*>(kpsac + orow * (R > 0 ? R : 1));
#pragma unroll
    for (int m = 0; m < R / 2; ++m) ps[m] = hw[m];
  }
}

template <int D>
hipError_t launch_values(const kvq_cache* c, const void* v, int cur_len, int n_new,
                         hipStream_t st) {
  const kvq_layout& L = c->layout;
  const int64_t rows = (int64_t)L.batch * L.kv_heads * n_new;
  const int64_t threads = rows * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (L.value_mode == KVQ_VAL_HADAMARD)
    quant_values_kernel<D, true><<<grid, 256, 0, st>>>(
        (const uint16_t*)v, (uint8_t*)c->v_codes, (uint32_t*)c->v_params, L.kv_heads,
        L.capacity, cur_len, n_new, rows);
  else
    quant_values_kernel<D, false><<<grid, 256, 0, st>>>(
        (const uint16_t*)v, (uint8_t*)c->v_codes, (uint32_t*)c->v_params, L.kv_heads,
        L.capacity, cur_len, n_new, rows);
  return hipGetLastError();
}

template <int D>
hipError_t launch_window_append(const kvq_cache* c, const void* k, const void* v, int cur_len,
                                int n_new, hipStream_t st) {
  const kvq_layout& L = c->layout;
  const int end = cur_len + n_new;
  const int jobs = (end - 1) / kWindow - cur_len / kWindow + 1;
  const dim3 grid((unsigned)jobs, (unsigned)L.kv_heads, (unsigned)L.batch);
  auto args = [&](auto kern) {
    kern<<<grid, 256, 0, st>>>((const uint16_t*)k, (const uint16_t*)v, (uint8_t*)c->k_codes,
                               (uint32_t*)c->k_params, (uint16_t*)c->k_tail,
                               (uint8_t*)c->v_codes, (uint32_t*)c->v_params, L.kv_heads,
                               L.capacity, cur_len, n_new);
  };
  if (L.value_mode == KVQ_VAL_HADAMARD) args(window_append_kernel<D, true>);
  else args(window_append_kernel<D, false>);
  return hipGetLastError();
}

template <int D, bool QSAC, int R>
hipError_t launch_centroid_cache(const kvq_cache* c, const void* k, int cur_len, int n_new,
                                 hipStream_t st) {
  const kvq_layout& L = c->layout;
  const dim3 grid((unsigned)((n_new + 255) / 256), (unsigned)L.kv_heads, (unsigned)L.batch);
  centroid_kernel<D, QSAC, R, true><<<grid, 256, 0, st>>>(
      (const uint16_t*)k, (int64_t)L.kv_heads * D, D, (int64_t)n_new * L.kv_heads * D, n_new,
      (const float*)c->centroids, L.n_centroids, (const float*)c->sens_w, L.qsac_topk,
      (const float*)c->psac_basis, nullptr, (uint8_t*)c->k_idx, (uint8_t*)c->k_codes,
      (uint32_t*)c->k_params, (uint16_t*)c->k_psac, L.kv_heads, L.capacity, cur_len);
  return hipGetLastError();
}

template <int D>
hipError_t launch_append(const kvq_cache* c, const void* k, const void* v, int cur_len,
                         int n_new, hipStream_t st) {
  const kvq_layout& L = c->layout;
  if (L.key_mode == KVQ_KEY_WINDOW) return launch_window_append<D>(c, k, v, cur_len, n_new, st);
  hipError_t e = launch_values<D>(c, v, cur_len, n_new, st);
  if (e != hipSuccess) return e;
  const bool qsac = L.key_mode == KVQ_KEY_CENTROID_QSAC;
  if (L.psac_rank == 8)
    return qsac ? launch_centroid_cache<D, true, 8>(c, k, cur_len, n_new, st)
                : launch_centroid_cache<D, false, 8>(c, k, cur_len, n_new, st);
  return qsac ? launch_centroid_cache<D, true, 0>(c, k, cur_len, n_new, st)
              : launch_centroid_cache<D, false, 0>(c, k, cur_len, n_new, st);
}

template <int D, bool QSAC>
hipError_t launch_assign_t(const void* keys, int64_t n, int64_t stride, const float* cent,
                           int C, const float* w, int topk, int32_t* out, hipStream_t st) {
  const dim3 grid((unsigned)((n + 255) / 256), 1, 1);
  centroid_kernel<D, QSAC, 0, false><<<grid, 256, 0, st>>>(
      (const uint16_t*)keys, stride, 0, 0, n, cent, C, w, topk, nullptr, out, nullptr,
      nullptr, nullptr, nullptr, 1, 0, 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_append(const kvq_cache* c, const void* k_bf16,
                                  const void* v_bf16, int cur_len, int n_new,
                                  hipStream_t stream) {
  if (n_new == 0) return hipSuccess;
  return (c->layout.head_dim == 128) ? launch_append<128>(c, k_bf16, v_bf16, cur_len, n_new, stream)
                                     : launch_append<64>(c, k_bf16, v_bf16, cur_len, n_new, stream);
}

hipError_t launch_cluster_assign(const void* keys, int64_t n, int head_dim,
                                 int64_t key_stride, const float* centroids,
                                 int n_centroids, const float* sens_w, int topk,
                                 int32_t* idx_out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (head_dim == 128)
    return sens_w ? launch_assign_t<128, true>(keys, n, key_stride, centroids, n_centroids, sens_w, topk, idx_out, stream)
                  : launch_assign_t<128, false>(keys, n, key_stride, centroids, n_centroids, nullptr, 1, idx_out, stream);
  return sens_w ? launch_assign_t<64, true>(keys, n, key_stride, centroids, n_centroids, sens_w, topk, idx_out, stream)
                : launch_assign_t<64, false>(keys, n, key_stride, centroids, n_centroids, nullptr, 1, idx_out, stream);
}

}  // namespace kvq
