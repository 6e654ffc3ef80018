// Decode attention read straight from the packed INT2 cache ([OKV]: the
// 2-bit cache is unpacked inside attention, no dense cache is built).
//
// Split-K over cached tokens: block (split, kv head, sequence) with four
// waves; each wave walks 64-token windows of its split with one token per
// lane for the logits, and one channel pair per lane for P.V.
//  * window keys: the query is folded into each window's per-channel
//    parameters once per window (q~ = q * s_w, bias = q . z_w), so a logit is
//    bias + sum_c q~_c code_c over the raw 2-bit codes;
//  * centroid keys: q . C_j is tabulated once per block, a logit is
//    (q.C)[idx] + sum_g s_g (q_g . codes_g) + z_g sum(q_g) [+ (U^T q) . a];
//  * values: p~ = p * s_(t,g) goes through LDS, each lane reads its channels'
//    64-token code rows straight from the channel-major value tile, and the z
//    part is a per-lane running sum sum_t p_t z_(t,g).
// The online softmax works in base 2 (logits pre-scaled by log2 e) with
// wave-shuffle maxima; each block merges its four waves and writes one
// partial (o, m, l); a second kernel merges the splits, rotates rotated
// values back and writes out/lse.
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

KVQ_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct DecodeArgs {
  const uint8_t* kcodes;
  const uint32_t* kparams;
  const uint16_t* ktail;
  const uint8_t* kidx;
  const float* cent;
  const float* basis;
  const uint16_t* kpsac;
  const uint8_t* vcodes;
  const uint32_t* vparams;
  const void* q;
  float* ws;
  int q_bf16, H, Hq, Tcap, C, n_tokens, split_len, S;
  float scale_log2;
};

template <int D, int G, int KM, int R>
__global__ __launch_bounds__(256) void decode_partial_kernel(const DecodeArgs a) {
  constexpr int NG = D / kGroup;      // parameter groups per row
  constexpr int CPL = D / kWave;      // P.V channels per lane
  __shared__ float qs[D][G];
  __shared__ float qc[KM == 1 ? G : 1][KM == 1 ? 256 : 1];
  __shared__ float qsum[G][NG];
  __shared__ float qp[G][R > 0 ? R : 1];
  __shared__ float qt[4][D][G];
  __shared__ float pt[4][kWave][NG][G];
  __shared__ float wm[4][G], wlv[4][G], wo[4][G][D];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t bh = (int64_t)b * a.H + h;
  const int hq0 = h * G;

  // ---- per-block query setup
  for (int e = tid; e < G * D; e += 256) {
    const int g = e / D, c = e % D;
    const int64_t qi = ((int64_t)b * a.Hq + hq0 + g) * D + c;
    qs[c][g] = a.q_bf16 ? bf16_to_f32(((const uint16_t*)a.q)[qi]) : ((const float*)a.q)[qi];
  }
  __syncthreads();
  if (KM == 1) {
    const float* cb = a.cent + bh * (int64_t)a.C * D;
    for (int e = tid; e < G * a.C; e += 256) {
      const int g = e / a.C, j = e % a.C;
      float acc = 0.0f;
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qs[d][g], cb[(int64_t)j * D + d], acc);
      qc[g][j] = acc;
    }
    for (int e = tid; e < G * NG; e += 256) {
      const int g = e / NG, gr = e % NG;
      float acc = 0.0f;
      for (int i = 0; i < kGroup; ++i) acc += qs[gr * kGroup + i][g];
      qsum[g][gr] = acc;
    }
    if (R > 0) {
      const float* U = a.basis + bh * D * R;
      for (int e = tid; e < G * R; e += 256) {
        const int g = e / R, m = e % R;
        float acc = 0.0f;
        for (int d = 0; d < D; ++d) acc = __builtin_fmaf(U[d * R + m], qs[d][g], acc);
        qp[g][m] = acc;
      }
    }
  }
  __syncthreads();

  const int t_begin = s * a.split_len;
  const int t_end = min(t_begin + a.split_len, a.n_tokens);
  const int n_full_win = a.n_tokens / kWindow;
  const int w_begin = t_begin / kWindow, w_end = (t_end + kWindow - 1) / kWindow;

  float m_run[G], l_lane[G], pz[G][NG], o[G][CPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -__builtin_inff();
    l_lane[g] = 0.0f;
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) pz[g][gr] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[g][c] = 0.0f;
  }

  for (int win = w_begin + wave; win < w_end; win += 4) {
    const int t = win * kWindow + lane;
    const bool valid = t < t_end;
    float lg[G];
    if (KM == 0) {
      if (win < n_full_win) {
        // fold the query into this window's parameters
        float bias[G];
#pragma unroll
        for (int g = 0; g < G; ++g) bias[g] = 0.0f;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          const int c = lane + cc * kWave;
          const uint32_t pw = a.kparams[(bh * (a.Tcap / kWindow) + win) * D + c];
          const float sc = f16_bits_to_f32(pw), zc = f16_bits_to_f32(pw >> 16);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            qt[wave][c][g] = qs[c][g] * sc;
            bias[g] = __builtin_fmaf(qs[c][g], zc, bias[g]);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = wave_sum(bias[g]);
        wave_lds_sync();
        const uint4* row = reinterpret_cast<const uint4*>(a.kcodes + (bh * a.Tcap + t) * (D / 4));
#pragma unroll
        for (int v = 0; v < D / 64; ++v) {
          const uint4 u = row[v];
          const uint32_t dw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int sh = 0; sh < 4; ++sh) {
              const uint32_t x = (dw[k] >> (2 * sh)) & 0x03030303u;
              const float cf[4] = {ubyte_f32<0>(x), ubyte_f32<1>(x), ubyte_f32<2>(x), ubyte_f32<3>(x)};
#pragma unroll
              for (int by = 0; by < 4; ++by) {
                const int c = v * 64 + k * 16 + by * 4 + sh;
#pragma unroll
                for (int g = 0; g < G; ++g) lg[g] = __builtin_fmaf(qt[wave][c][g], cf[by], lg[g]);
              }
            }
          }
        }
      } else {
        // unfinished window: bf16 keys from the tail
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = 0.0f;
        if (valid) {
          const uint16_t* kt = a.ktail + (bh * kWindow + lane) * D;
#pragma unroll
          for (int v = 0; v < D / 8; ++v) {
            float x[8];
            bf16x8_to_f32(*reinterpret_cast<const uint4*>(kt + v * 8), x);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
              for (int g = 0; g < G; ++g) lg[g] = __builtin_fmaf(qs[v * 8 + u][g], x[u], lg[g]);
          }
        }
      }
    } else {
      // centroid + residual keys
#pragma unroll
      for (int g = 0; g < G; ++g) lg[g] = 0.0f;
      if (valid) {
        const int64_t tr = bh * a.Tcap + t;
        const int j = a.kidx[tr];
        uint32_t pw[NG];
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) pw[gr] = a.kparams[tr * NG + gr];
        const uint4* row = reinterpret_cast<const uint4*>(a.kcodes + tr * (D / 4));
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) {
          const uint4 u = row[gr / 2];
          const uint32_t w0 = (gr & 1) ? u.z : u.x, w1 = (gr & 1) ? u.w : u.y;
          float dg[G];
#pragma unroll
          for (int g = 0; g < G; ++g) dg[g] = 0.0f;
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            const uint32_t wv = (i < 16) ? w0 : w1;
            const float cf = (float)((wv >> (2 * (i & 15))) & 3u);
#pragma unroll
            for (int g = 0; g < G; ++g) dg[g] = __builtin_fmaf(qs[gr * kGroup + i][g], cf, dg[g]);
          }
          const float sc = f16_bits_to_f32(pw[gr]), zc = f16_bits_to_f32(pw[gr] >> 16);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            lg[g] = __builtin_fmaf(sc, dg[g], lg[g]);
            lg[g] = __builtin_fmaf(zc, qsum[g][gr], lg[g]);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] += qc[g][j];
        if (R > 0) {
          const uint16_t* ap = a.kpsac + tr * R;
#pragma unroll
          for (int m = 0; m < R; ++m) {
            const float am = f16_bits_to_f32(ap[m]);
#pragma unroll
            for (int g = 0; g < G; ++g) lg[g] = __builtin_fmaf(qp[g][m], am, lg[g]);
          }
        }
      }
    }

    // ---- online softmax (base 2)
    float p[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float x = valid ? lg[g] * a.scale_log2 : -__builtin_inff();
      const float mw = wave_max(x);
      const float mn = fmaxf(m_run[g], mw);
      const float alpha = exp2f(m_run[g] - mn);
      p[g] = exp2f(x - mn);
      l_lane[g] = __builtin_fmaf(l_lane[g], alpha, p[g]);
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[g][c] *= alpha;
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) pz[g][gr] *= alpha;
      m_run[g] = mn;
    }

    // ---- values: p~ through LDS; each lane reads its channels' tile rows
    {
      uint32_t vw[NG];
      if (valid) {
        const int64_t tr = bh * a.Tcap + t;
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) vw[gr] = a.vparams[tr * NG + gr];
      } else {
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) vw[gr] = 0u;
      }
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        const float sc = f16_bits_to_f32(vw[gr]), zc = f16_bits_to_f32(vw[gr] >> 16);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pg = valid ? p[g] : 0.0f;
          pt[wave][lane][gr][g] = pg * sc;
          pz[g][gr] = __builtin_fmaf(pg, zc, pz[g][gr]);
        }
      }
    }
    wave_lds_sync();
    {
      // lane -> channels lane*CPL .. lane*CPL+CPL-1; a channel's 64 codes
      // of this window are one 16-byte tile row (token tt at bits 2tt)
      const int c0 = lane * CPL;
      const int gr = c0 / kGroup;
      uint4 crow[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        crow[c] = *reinterpret_cast<const uint4*>(
            a.vcodes + ((bh * (a.Tcap / kWindow) + win) * D + c0 + c) * 16);
      for (int tt = 0; tt < kWave; ++tt) {
        float cf[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const uint32_t wd = (tt < 16) ? crow[c].x : (tt < 32) ? crow[c].y : (tt < 48) ? crow[c].z : crow[c].w;
          cf[c] = (float)((wd >> (2 * (tt & 15))) & 3u);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pg = pt[wave][tt][gr][g];
#pragma unroll
          for (int c = 0; c < CPL; ++c) o[g][c] = __builtin_fmaf(pg, cf[c], o[g][c]);
        }
      }
    }
    wave_lds_sync();
  }

  // ---- wave partial -> block partial
  {
    const int c0 = lane * CPL;
    const int gr = c0 / kGroup;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float l = wave_sum(l_lane[g]);
      float zsum[NG];
#pragma unroll
      for (int q = 0; q < NG; ++q) zsum[q] = wave_sum(pz[g][q]);
#pragma unroll
      for (int c = 0; c < CPL; ++c) wo[wave][g][c0 + c] = o[g][c] + zsum[gr];
      if (lane == 0) {
        wm[wave][g] = m_run[g];
        wlv[wave][g] = l;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < G * (D + 2); e += 256) {
    const int g = e / (D + 2), c = e % (D + 2);
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (wm[w][g] == -__builtin_inff()) ? 0.0f : exp2f(wm[w][g] - M);
      const float v = (c < D) ? wo[w][g][c] : wlv[w][g];
      acc = __builtin_fmaf(f, v, acc);
    }
    float* dst = a.ws + (((int64_t)s * gridDim.z + b) * a.Hq + hq0 + g) * (D + 2);
    if (c < D) dst[c] = acc;
    else if (c == D) dst[D] = M;
    else dst[D + 1] = acc;
  }
}

template <int D, bool HAD>
__global__ __launch_bounds__(128) void decode_reduce_kernel(const float* __restrict__ ws, int S,
                                                            int BHq, void* out, int out_bf16,
                                                            float* __restrict__ lse) {
  __shared__ float xs[D];
  const int r = blockIdx.x, c = threadIdx.x;
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, ws[((int64_t)s * BHq + r) * (D + 2) + D]);
  float L = 0.0f, acc = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float* p = ws + ((int64_t)s * BHq + r) * (D + 2);
    const float f = exp2f(p[D] - M);
    L = __builtin_fmaf(f, p[D + 1], L);
    if (c < D) acc = __builtin_fmaf(f, p[c], acc);
  }
  float v = acc / L;
  if (HAD) {
    if (c < D) xs[c] = v;
    __syncthreads();
    for (int hh = 1; hh < D; hh <<= 1) {
      float nv = 0.0f;
      if (c < D) {
        const float other = xs[c ^ hh];
        nv = (c & hh) ? (other - xs[c]) : (xs[c] + other);
      }
      __syncthreads();
      if (c < D) xs[c] = nv;
      __syncthreads();
    }
    v = (c < D) ? xs[c] * (D == 128 ? 0.08838834764831845f : 0.125f) : 0.0f;
  }
  if (c < D) {
    if (out_bf16) {
      uint32_t u = __float_as_uint(v);
      u += 0x7FFFu + ((u >> 16) & 1u);
      ((uint16_t*)out)[(int64_t)r * D + c] = (uint16_t)(u >> 16);
    } else {
      ((float*)out)[(int64_t)r * D + c] = v;
    }
  }
  if (c == 0 && lse != nullptr) lse[r] = (M + log2f(L)) * kLn2;
}

template <int D, int G, int KM, int R>
hipError_t launch_partial(const DecodeArgs& a, int B, hipStream_t st) {
  const dim3 grid((unsigned)a.S, (unsigned)a.H, (unsigned)B);
  decode_partial_kernel<D, G, KM, R><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_partial_mode(const DecodeArgs& a, int key_mode, int R, int B, hipStream_t st) {
  if (key_mode == KVQ_KEY_WINDOW) return launch_partial<D, G, 0, 0>(a, B, st);
  if (R == 8) return launch_partial<D, G, 1, 8>(a, B, st);
  return launch_partial<D, G, 1, 0>(a, B, st);
}

template <int D>
hipError_t launch_partial_g(const DecodeArgs& a, int G, int key_mode, int R, int B,
                            hipStream_t st) {
  switch (G) {
    case 1: return launch_partial_mode<D, 1>(a, key_mode, R, B, st);
    case 2: return launch_partial_mode<D, 2>(a, key_mode, R, B, st);
    case 4: return launch_partial_mode<D, 4>(a, key_mode, R, B, st);
    default: return launch_partial_mode<D, 8>(a, key_mode, R, B, st);
  }
}

}  // namespace

int decode_splits(const kvq_layout* L, int q_heads, int n_tokens) {
  (void)q_heads;
  const int n_win = (n_tokens + kWindow - 1) / kWindow;
  const int units = L->batch * L->kv_heads;
  int S = (2048 + units - 1) / units;
  if (S > n_win) S = n_win;
  if (S < 1) S = 1;
  const int per = (n_win + S - 1) / S;
  return (n_win + per - 1) / per;
}

size_t decode_workspace_bytes(const kvq_layout* L, int q_heads, int n_tokens) {
  const int S = decode_splits(L, q_heads, n_tokens);
  return (size_t)S * L->batch * q_heads * (L->head_dim + 2) * sizeof(float);
}

hipError_t launch_decode(const kvq_cache* c, int n_tokens, const void* q, int q_dtype,
                         int q_heads, float scale, void* out, int out_dtype, float* lse,
                         void* ws, hipStream_t stream) {
  const kvq_layout& L = c->layout;
  const int S = decode_splits(&L, q_heads, n_tokens);
  const int n_win = (n_tokens + kWindow - 1) / kWindow;
  const int per = (n_win + S - 1) / S;
  DecodeArgs a;
  a.kcodes = (const uint8_t*)c->k_codes;
  a.kparams = (const uint32_t*)c->k_params;
  a.ktail = (const uint16_t*)c->k_tail;
  a.kidx = (const uint8_t*)c->k_idx;
  a.cent = (const float*)c->centroids;
  a.basis = (const float*)c->psac_basis;
  a.kpsac = (const uint16_t*)c->k_psac;
  a.vcodes = (const uint8_t*)c->v_codes;
  a.vparams = (const uint32_t*)c->v_params;
  a.q = q;
  a.ws = (float*)ws;
  a.q_bf16 = (q_dtype == KVQ_BF16);
  a.H = L.kv_heads;
  a.Hq = q_heads;
  a.Tcap = L.capacity;
  a.C = L.n_centroids;
  a.n_tokens = n_tokens;
  a.split_len = per * kWindow;
  a.S = S;
  a.scale_log2 = scale * kLog2e;
  const int G = q_heads / L.kv_heads;
  const int R = (L.key_mode == KVQ_KEY_WINDOW) ? 0 : L.psac_rank;
  hipError_t e = (L.head_dim == 128)
                     ? launch_partial_g<128>(a, G, L.key_mode, R, L.batch, stream)
                     : launch_partial_g<64>(a, G, L.key_mode, R, L.batch, stream);
  if (e != hipSuccess) return e;
  const int BHq = L.batch * q_heads;
  const bool had = L.value_mode == KVQ_VAL_HADAMARD;
  const int ob = out_dtype == KVQ_BF16;
  if (L.head_dim == 128) {
    if (had) decode_reduce_kernel<128, true><<<BHq, 128, 0, stream>>>((const float*)ws, S, BHq, out, ob, lse);
    else decode_reduce_kernel<128, false><<<BHq, 128, 0, stream>>>((const float*)ws, S, BHq, out, ob, lse);
  } else {
    if (had) decode_reduce_kernel<64, true><<<BHq, 64, 0, stream>>>((const float*)ws, S, BHq, out, ob, lse);
    else decode_reduce_kernel<64, false><<<BHq, 64, 0, stream>>>((const float*)ws, S, BHq, out, ob, lse);
  }
  return hipGetLastError();
}

}  // namespace kvq
