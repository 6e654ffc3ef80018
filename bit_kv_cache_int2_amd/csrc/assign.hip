// Centroid assignment of keys ([QWM] 1, QSAC [QWM] 1, PSAC [QWM] 2): the
// key side of quantize-append for centroid keys, and kv_cluster_assign.
// Each key gets the centroid of smallest fp32 squared distance (channel
// order, fma; lowest index on ties), or with QSAC the best of the top-k
// weighted distances by the weighted error of its INT2 residual; the
// residual is INT2-quantised per group of 32 and, with PSAC, its error is
// projected on the query principal directions.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace kvq {
namespace {


// A key row held as packed bf16 pairs (channel d in word d / 2, low half
// first); the fp32 value is exact.
template <int D>
struct KeyRow {
  uint32_t w[D / 2];
  KVQ_DEV float operator[](int d) const {
    return __uint_as_float((d & 1) ? (w[d >> 1] & 0xFFFF0000u) : (w[d >> 1] << 16));
  }
};

// INT2-quantise the residual r = k - c per group of 32 (inputs
// canonicalised), returning the weighted squared error of the dequantised
// residual (fp32, channel order; 0 when w == nullptr).  Optionally emits the
// packed codes, the parameter words and the PSAC accumulators.
template <int D, int R, bool EMIT>
KVQ_DEV float residual_q2(const KeyRow<D>& k, const float* __restrict__ c,
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

// QSAC range-based estimate of candidate c ([QWM] 1: dynamic range and
// sensitivity): sum over groups of fma(s_g * s_g, W_g), s_g the fp16 step
// the quantizer would store for the residual group, W_g the group's summed
// weights (fp32, channel order).
template <int D>
KVQ_DEV float range_estimate(const KeyRow<D>& k, const float* __restrict__ c,
                             const float* Wg) {
  float E = 0.0f;
#pragma unroll
  for (int g = 0; g < D / kGroup; ++g) {
    float mn = __builtin_inff(), mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kGroup; i += 4) {
      const float4 c4 = *reinterpret_cast<const float4*>(c + g * kGroup + i);
      const float r0 = k[g * kGroup + i] - c4.x, r1 = k[g * kGroup + i + 1] - c4.y,
                  r2 = k[g * kGroup + i + 2] - c4.z, r3 = k[g * kGroup + i + 3] - c4.w;
      mn = fminf(fminf(mn, r0), fminf(fminf(r1, r2), r3));
      mx = fmaxf(fmaxf(mx, r0), fmaxf(fmaxf(r1, r2), r3));
    }
    const float s = f16_bits_to_f32(f32_to_f16_bits(div3(mx - mn)));
    E = __builtin_fmaf(s * s, Wg[g], E);
  }
  return E;
}

// INT8 PSAC coefficients ([QWM] 2): one fp16 scale per token,
// sc = fp16(max |a| / 127), q_m = rint(a_m / sc) clamped to [-127, 127],
// zero when sc is 0.  Returns the scale's bits; q packed low byte first.
template <int R>
KVQ_DEV uint32_t psac_int8(const float (&a)[R], uint32_t (&q)[R / 4]) {
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < R; ++m) amax = fmaxf(amax, fabsf(a[m]));
  const uint32_t sh = f32_to_f16_bits(amax / 127.0f);
  const float sc = f16_bits_to_f32(sh);
#pragma unroll
  for (int m = 0; m < R / 4; ++m) q[m] = 0u;
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const float v = sc == 0.0f ? 0.0f : fminf(fmaxf(__builtin_rintf(a[m] / sc), -127.0f), 127.0f);
    q[m / 4] |= ((uint32_t)(int32_t)v & 0xFFu) << (8 * (m % 4));
  }
  return sh;
}

// Exact squared distance of key row kr (bf16) to centroid row cr (fp32): the
// fp32 sum in channel order with fma, t = k - c; QSAC weighs each term as
// fma(w t, t) with w t rounded first.
// All rows' loads are issued before the sum when ALL (one memory round
// trip; the queue drain, where nothing else is live), else 32 channels at a
// time.
template <int D, bool QSAC, bool ALL = false>
KVQ_DEV float exact_dist(const uint16_t* __restrict__ kr, const float* __restrict__ cr, const float* w) {
  constexpr int kStep = ALL ? D : 32;
  float acc = 0.0f;
#pragma unroll 1
  for (int d0 = 0; d0 < D; d0 += kStep) {
    uint4 kv[kStep / 8];
    float4 cv[kStep / 4];
#pragma unroll
    for (int u = 0; u < kStep / 8; ++u) kv[u] = *reinterpret_cast<const uint4*>(kr + d0 + 8 * u);
#pragma unroll
    for (int u = 0; u < kStep / 4; ++u) cv[u] = *reinterpret_cast<const float4*>(cr + d0 + 4 * u);
#pragma unroll
    for (int u = 0; u < kStep / 8; ++u) {
      float x[8];
      bf16x8_to_f32(kv[u], x);
      const float cc[8] = {cv[2 * u].x, cv[2 * u].y, cv[2 * u].z, cv[2 * u].w,
                           cv[2 * u + 1].x, cv[2 * u + 1].y, cv[2 * u + 1].z, cv[2 * u + 1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = x[e] - cc[e];
        const int d = d0 + 8 * u + e;
        acc = QSAC ? __builtin_fmaf(w[d] * t, t, acc) : __builtin_fmaf(t, t, acc);
      }
    }
  }
  return acc;
}

// Two floats to bf16 (round to nearest even), packed low = a, high = b.
KVQ_DEV uint32_t bf16_pack2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}

// Rescoring queue entry: the top 18 bits of a float at most the pair's
// lower end (a NaN end counts as -inf, so the pair is kept), the key's slot
// in the wave (6 bits) and the centroid index (8 bits).
KVQ_DEV uint32_t queue_entry(float lower, int kl, int j) {
  uint32_t b = __float_as_uint(lower != lower ? -__builtin_inff() : lower);
  if ((b >> 31) && (b & 0x3FFFu)) b += 0x4000u;   // negative: round the magnitude up
  return (b & 0xFFFFC000u) | ((uint32_t)kl << 8) | (uint32_t)j;
}

// Distance (bits, non-negative) and index packed so that the u64 order is
// the lexicographic order (distance, index) of the assignment rules.
KVQ_DEV unsigned long long dist_key(float dist, int j) {
  return ((unsigned long long)__float_as_uint(dist) << 32) | (uint32_t)j;
}

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Centroid assignment with the exact result and most of the work on MFMA.
//
// Block = 4 waves x 64 keys.  The centroid table streams through LDS 64 rows
// at a time, split into bf16 hi + lo parts (c ~ hi + lo within 2^-18 |c|;
// QSAC uses the rows w*c).  Per wave, bf16 MFMAs give every (key,
// centroid) pair  d~ = |c|^2 - 2 k.c  (the key's |k|^2 is common to all
// centroids and left out), whose distance to the exact fp32 distance of
// the assignment rule (less |k|^2) is below 2^-13 (|k| + |c|)^2 (MFMA
// accumulation, the hi/lo split, the fp32 rounding of the rule itself; the
// norms are weighted for QSAC).  With the margin M = 2^-11 (|k|^2 + |c|^2) +
// 1e-30, at least twice that, each pair has an interval [d~ - M, d~ + M]
// around its exact value.
// A key keeps U = the smallest upper end seen so far (QSAC: at most the
// 4th smallest, merged from the four lanes that share the key), and every
// centroid whose lower end is at most U goes to a per-wave queue in LDS
// (with its lower end rounded down); the winner (QSAC: each of the top-4)
// has its lower end below the final U, so it is always queued.  Once the
// table has been seen, entries above the key's final threshold are
// dropped; a key left with one entry (QSAC: exactly topk = 4) has its
// answer, the others are rescored with the rule's own arithmetic and tie
// order, all 64 lanes draining the queue together: the best (distance,
// index) per key by a 64-bit LDS atomic min (QSAC: a list per key).  A key
// whose queue or list overflows, weights that are negative or not finite,
// or topk > 4 fall back to the exact scan of every centroid, lane per key.
// Then, lane per key: QSAC scores its top-k candidates by the INT2 residual
// error (or the range estimate), and TO_CACHE writes idx/codes/params/PSAC
// into the cache rows at cur_len + i (otherwise the i32 index goes to
// idx_out).
constexpr int kCandMax = 8;    // QSAC candidates (topk <= kCandMax)
constexpr int kCChunk = 64;    // centroids per LDS chunk
constexpr int kQueue = 1024;   // per-wave rescoring queue
constexpr int kList = 8;       // QSAC: candidates kept per key (more: the exact scan)
constexpr float kMarginRel = 1.0f / 4096.0f;
constexpr int kFlagRange = 1;   // QSAC: range-based perturbation estimate
constexpr int kFlagInt8 = 2;    // PSAC: INT8 coefficients + fp16 scale
constexpr float kMarginAbs = 1e-30f;

template <int D, bool QSAC, int R, bool TO_CACHE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void centroid_kernel(
    const uint16_t* __restrict__ kin, int64_t key_stride, int64_t head_stride,
    int64_t batch_stride, int64_t n, const float* __restrict__ cent, int C,
    const float* __restrict__ sens_w, int topk, const float* __restrict__ basis,
    int32_t* __restrict__ idx_out, uint8_t* __restrict__ kidx,
    uint8_t* __restrict__ kcodes, uint32_t* __restrict__ kparams,
    uint16_t* __restrict__ kpsac, int H, int Tcap, int cur_len, int flags,
    uint16_t* __restrict__ kpsac_sc) {
  // flags: kFlagRange = QSAC range-based estimate, kFlagInt8 = INT8 PSAC
  // coefficients (kpsac then holds the codes, kpsac_sc the scales)
  constexpr int NKS = D / 32;
  constexpr int CP = D + 16;   // chunk row pitch (bf16): conflict-free operand reads
  __shared__ __align__(16) __bf16 chi[kCChunk * CP];
  __shared__ __align__(16) __bf16 clo[kCChunk * CP];
  __shared__ __align__(16) float cup[kCChunk], clo_[kCChunk];   // |c|^2 + Mc, |c|^2 - Mc
  __shared__ float wl[D];
  __shared__ float wg[QSAC ? D / kGroup : 1];   // per-group weight sums
  __shared__ float ul[D * (R > 0 ? R : 1)];
  __shared__ uint32_t queue[4][kQueue];
  __shared__ int qcount[4];
  __shared__ unsigned long long best[QSAC ? 1 : 256];
  __shared__ unsigned long long clist[QSAC ? 256 * kList : 1];
  __shared__ int ccount[QSAC ? 256 : 1];
  __shared__ float thrf[256];     // final threshold U + 2 Mk per key
  __shared__ int nsurv[256];      // queue entries per key that pass it
  __shared__ uint32_t sj[QSAC ? 1 : 256];   // their lowest centroid index
  __shared__ int bad_w;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = (int64_t)blockIdx.z * H + blockIdx.y;
  const int64_t kbase = (int64_t)blockIdx.x * 256 + wave * 64;   // this wave's 64 keys
  const float* cb = cent + bh * (int64_t)C * D;
  const uint16_t* kb = kin + blockIdx.z * batch_stride + blockIdx.y * head_stride;

  if (QSAC)
    for (int d = tid; d < D; d += 256) wl[d] = sens_w[bh * D + d];
  if (R > 0)
    for (int d = tid; d < D * R; d += 256) ul[d] = basis[bh * D * R + d];
  if (tid == 0) bad_w = 0;
  if (QSAC) ccount[tid] = 0;
  else {
    best[tid] = ~0ull;
    sj[tid] = ~0u;
  }
  nsurv[tid] = 0;
  if (lane == 0) qcount[wave] = 0;
  __syncthreads();
  if (QSAC && tid < D && !(wl[tid] >= 0.0f && wl[tid] < __builtin_inff())) bad_w = 1;
  if (QSAC && tid < D / kGroup) {
    float W = 0.0f;
    for (int i = 0; i < kGroup; ++i) W = W + wl[tid * kGroup + i];
    wg[tid] = W;
  }
  __syncthreads();
  const bool exact_scan = (QSAC && (bad_w != 0 || topk > 4));

  // ---- this wave's keys as the B operand (bf16 is exact); lane (g, c16)
  // holds dims 32 ks + 8 g .. + 7 of key 16 nt + c16
  bf8 kop[4][NKS];
  float mk[4];     // Mk = 2^-11 |k|^2 + 1e-30 (|k| weighted for QSAC)
  bool kok[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t i = kbase + nt * 16 + c16;
    kok[nt] = i < n;
    // slots past the end read the last key; they never push a candidate
    const uint16_t* krow = kb + (kok[nt] ? i : n - 1) * key_stride;
    float s2 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 u = *reinterpret_cast<const uint4*>(krow + ks * 32 + 8 * g);
      kop[nt][ks] = __builtin_bit_cast(bf8, u);
      float x[8];
      bf16x8_to_f32(u, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) s2 = __builtin_fmaf(QSAC ? wl[ks * 32 + 8 * g + e] * x[e] : x[e], x[e], s2);
    }
    s2 += __shfl_xor(s2, 16, 64);
    s2 += __shfl_xor(s2, 32, 64);
    mk[nt] = __builtin_fmaf(2.0f * kMarginRel, s2, kMarginAbs);   // the key's part of the margin
  }
  // U (plain) or this lane's four smallest upper ends (QSAC), per key slot
  float U[4], t4[4][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    U[nt] = __builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) t4[nt][r] = __builtin_inff();
  }

  for (int c0 = 0; c0 < C && !exact_scan; c0 += kCChunk) {
    __syncthreads();   // the previous chunk is consumed
    {
      // thread -> row tid / 4, a quarter of its channels
      const int r = tid >> 2, q = tid & 3, j = c0 + r;
      // rows past the table repeat the last row; their bounds are +inf
      const float* crow = cb + (int64_t)(j < C ? j : C - 1) * D;
      float s2 = 0.0f;
#pragma unroll
      for (int d = q * (D / 4); d < (q + 1) * (D / 4); d += 4) {
        const float4 v = *reinterpret_cast<const float4*>(crow + d);
        const float x[4] = {v.x, v.y, v.z, v.w};
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = QSAC ? wl[d + e] * x[e] : x[e];
          s2 = __builtin_fmaf(y[e], x[e], s2);
        }
        // hi = bf16(y) (round to nearest even), lo = bf16(y - hi)
        const uint2 hb = make_uint2(bf16_pack2(y[0], y[1]), bf16_pack2(y[2], y[3]));
        const float h[4] = {__uint_as_float(hb.x << 16), __uint_as_float(hb.x & 0xFFFF0000u),
                            __uint_as_float(hb.y << 16), __uint_as_float(hb.y & 0xFFFF0000u)};
        const uint2 lb = make_uint2(bf16_pack2(y[0] - h[0], y[1] - h[1]), bf16_pack2(y[2] - h[2], y[3] - h[3]));
        *reinterpret_cast<uint2*>(&chi[r * CP + d]) = hb;
        *reinterpret_cast<uint2*>(&clo[r * CP + d]) = lb;
      }
      s2 += __shfl_xor(s2, 1, 64);
      s2 += __shfl_xor(s2, 2, 64);
      if (q == 0) {
        // s2 = |c|^2 (sum w c^2 for QSAC); the centroid's part of the margin
        // is Mc = 2^-11 |c|^2; rows past the table never qualify
        const float mc = 2.0f * kMarginRel * s2;
        cup[r] = (j < C) ? s2 + mc : __builtin_inff();
        clo_[r] = (j < C) ? s2 - mc : __builtin_inff();
      }
    }
    __syncthreads();

    // ---- S = C_chunk K^T: row = centroid 16 mt + 4 g + i, column = key 16 nt + c16
    f4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int off = (mt * 16 + c16) * CP + ks * 32 + 8 * g;
        const bf8 ah = *reinterpret_cast<const bf8*>(&chi[off]);
        const bf8 al = *reinterpret_cast<const bf8*>(&clo[off]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, kop[nt][ks], acc[mt][nt], 0, 0, 0);
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, kop[nt][ks], acc[mt][nt], 0, 0, 0);
        }
      }

    // ---- intervals, U, candidates.  With M = Mk + Mc >= 2^-12 (|k| + |c|)^2
    // (as (a + b)^2 <= 2 a^2 + 2 b^2) the ends are
    //   upper = (|c|^2 + Mc - 2 k.c) + Mk,  lower = (|c|^2 - Mc - 2 k.c) - Mk,
    // so U = min upper = min(vu) + Mk and lower <= U  <=>  vl <= min(vu) + 2 Mk.
    float cuv[4][4], clv[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 au = *reinterpret_cast<const float4*>(&cup[mt * 16 + 4 * g]);
      const float4 al = *reinterpret_cast<const float4*>(&clo_[mt * 16 + 4 * g]);
      cuv[mt][0] = au.x; cuv[mt][1] = au.y; cuv[mt][2] = au.z; cuv[mt][3] = au.w;
      clv[mt][0] = al.x; clv[mt][1] = al.y; clv[mt][2] = al.z; clv[mt][3] = al.w;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float vl[4][4];
      float um = __builtin_inff();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float vu = __builtin_fmaf(-2.0f, acc[mt][nt][i], cuv[mt][i]);
          vl[mt][i] = __builtin_fmaf(-2.0f, acc[mt][nt][i], clv[mt][i]);
          if (QSAC) {
            // keep this lane's four smallest (upper ends less Mk)
            float v = vu;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float a0 = t4[nt][r];
              t4[nt][r] = fminf(a0, v);
              v = fmaxf(a0, v);
            }
          } else {
            um = fminf(um, vu);
          }
        }
      float uu;
      if (QSAC) {
        // 4th smallest over the four lanes of the key (disjoint centroid
        // sets): two bitonic merges of sorted 4-lists
        float m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = fminf(t4[nt][r], __shfl_xor(t4[nt][3 - r], 16, 64));
        const float a0 = fminf(m[0], m[2]), a2 = fmaxf(m[0], m[2]), a1 = fminf(m[1], m[3]), a3 = fmaxf(m[1], m[3]);
        const float srt[4] = {fminf(a0, a1), fmaxf(a0, a1), fminf(a2, a3), fmaxf(a2, a3)};
        float top = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r) top = fmaxf(top, fminf(srt[r], __shfl_xor(srt[3 - r], 32, 64)));
        uu = top;
      } else {
        uu = um;
        uu = fminf(uu, __shfl_xor(uu, 16, 64));
        uu = fminf(uu, __shfl_xor(uu, 32, 64));
      }
      U[nt] = fminf(U[nt], uu);
      const float thr = U[nt] + 2.0f * mk[nt];
      // candidate mask, bit 4 mt + i (a NaN bound counts as a candidate;
      // rows past the table are +inf)
      uint32_t cm = 0;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) cm |= (uint32_t)!(vl[mt][i] > thr) << (4 * mt + i);
      if (!kok[nt]) cm = 0;
      if (__ballot(cm != 0)) {
        while (cm) {
          const int b = __builtin_ctz(cm);
          cm &= cm - 1;
          const int j = c0 + (b >> 2) * 16 + 4 * g + (b & 3);
          float vb = vl[0][0];   // vl[b / 4][b % 4], selected without a register index
#pragma unroll
          for (int q = 1; q < 16; ++q) vb = b == q ? vl[q >> 2][q & 3] : vb;
          const int pos = atomicAdd(&qcount[wave], 1);
          if (pos < kQueue) queue[wave][pos] = queue_entry(vb, nt * 16 + c16, j);
        }
      }
    }
  }

  // ---- drain the queue once.  Entries whose lower end exceeds the key's
  // final threshold cannot win (plain) or be in the top 4 (QSAC) and are
  // dropped.  Plain: a key with a single entry left has its winner without
  // rescoring (the winner's lower end never exceeds the final threshold);
  // QSAC with topk 4: a key with exactly four entries left has its top-4
  // set (the order inside it does not matter: the residual score decides).
  // The others are rescored exactly, lanes in parallel.
  if (g == 0) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) thrf[wave * 64 + nt * 16 + c16] = U[nt] + 2.0f * mk[nt];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const int cnt = __builtin_amdgcn_readfirstlane(qcount[wave]);
  const bool overflow = cnt > kQueue;   // wave-uniform
  auto live = [&](uint32_t ent) {       // j past the table: only when every bound was infinite
    const int kl = (int)((ent >> 8) & 63u), j = (int)(ent & 255u);
    return j < C && !(__uint_as_float(ent & 0xFFFFC000u) > thrf[wave * 64 + kl]);
  };
  if (!overflow && !exact_scan) {
    for (int e = lane; e < cnt; e += 64) {
      const uint32_t ent = queue[wave][e];
      if (live(ent)) {
        const int kl = (int)((ent >> 8) & 63u);
        atomicAdd(&nsurv[wave * 64 + kl], 1);
        if (!QSAC) atomicMin(&sj[wave * 64 + kl], ent & 255u);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    for (int e = lane; e < cnt; e += 64) {
      const uint32_t ent = queue[wave][e];
      const int kl = (int)((ent >> 8) & 63u), j = (int)(ent & 255u);
      const int ns = nsurv[wave * 64 + kl];
      if (live(ent) && (QSAC || ns > 1)) {
        // QSAC: exactly topk survivors are the top-k set itself (the four
        // smallest upper ends always survive), listed without distances
        const float dist = (QSAC && ns == topk)
                               ? 0.0f
                               : exact_dist<D, QSAC, !QSAC>(kb + (kbase + kl) * key_stride,
                                                            cb + (int64_t)j * D, wl);
        if (QSAC) {
          const int pos = atomicAdd(&ccount[wave * 64 + kl], 1);
          if (pos < kList) clist[(wave * 64 + kl) * kList + pos] = dist_key(dist, j);
        } else {
          atomicMin(&best[wave * 64 + kl], dist_key(dist, j));
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

  // ---- lane per key
  const int64_t i = kbase + lane;
  const bool ok = i < n;
  if (!ok) return;
  const uint16_t* kr = kb + i * key_stride;
  int bestj = 0;
  int cj[kCandMax];
#pragma unroll
  for (int t = 0; t < kCandMax; ++t) cj[t] = 0;
  bool scan = exact_scan || overflow;
  if (QSAC && !scan) {
    const int m = ccount[wave * 64 + lane];
    if (m > kList) {
      scan = true;
    } else {
      // the top-k of the scored list in (distance, index) order
      unsigned long long prev = 0ull;
      bool first = true;
#pragma unroll
      for (int t = 0; t < kCandMax; ++t) {
        if (t < topk && t < C) {
          unsigned long long mv = ~0ull;
          for (int e = 0; e < m; ++e) {
            const unsigned long long v = clist[(wave * 64 + lane) * kList + e];
            if ((first || v > prev) && v < mv) mv = v;
          }
          cj[t] = (int)(mv & 0xFFFFFFFFull);
          prev = mv;
          first = false;
        }
      }
    }
  } else if (!QSAC && !scan) {
    bestj = nsurv[wave * 64 + lane] == 1 ? (int)sj[wave * 64 + lane]
                                         : (int)(best[wave * 64 + lane] & 0xFFFFFFFFull);
  }
  if (scan) {
    // every centroid, in index order, with the rule's arithmetic
    float bd = __builtin_inff();
    float cd[kCandMax];
#pragma unroll
    for (int t = 0; t < kCandMax; ++t) {
      cd[t] = __builtin_inff();
      cj[t] = 0;
    }
    for (int j = 0; j < C; ++j) {
      const float dist = exact_dist<D, QSAC>(kr, cb + (int64_t)j * D, wl);
      if (QSAC) {
        // insertion in (distance, index) order: a displaced entry carries a
        // lower index than the entries it may pass, so ties compare indices
        float vd = dist;
        int vj = j;
#pragma unroll
        for (int t = 0; t < kCandMax; ++t) {
          if (vd < cd[t] || (vd == cd[t] && vj < cj[t])) {
            const float td = cd[t];
            const int tj = cj[t];
            cd[t] = vd;
            cj[t] = vj;
            vd = td;
            vj = tj;
          }
        }
      } else if (dist < bd) {
        bd = dist;
        bestj = j;
      }
    }
  }
  // the key as packed bf16 (half the registers of an fp32 row), loaded only
  // now: the list selection and the scan above read it from memory
  KeyRow<D> k;
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    const uint4 u = *reinterpret_cast<const uint4*>(kr + j * 8);
    k.w[4 * j] = u.x;
    k.w[4 * j + 1] = u.y;
    k.w[4 * j + 2] = u.z;
    k.w[4 * j + 3] = u.w;
  }
  if (QSAC) {
    float bE = 0.0f;
    bestj = -1;
#pragma unroll
    for (int t = 0; t < kCandMax; ++t) {
      if (t < topk && t < C) {
        const int j = cj[t];
        const float E = (flags & kFlagRange)
                            ? range_estimate<D>(k, cb + (int64_t)j * D, wg)
                            : residual_q2<D, 0, false>(k, cb + (int64_t)j * D, wl, nullptr,
                                                       nullptr, nullptr, nullptr);
        if (bestj < 0 || E < bE || (E == bE && j < bestj)) {
          bestj = j;
          bE = E;
        }
      }
    }
  }
  if (!TO_CACHE) {
    idx_out[bh * n + i] = bestj;
    return;
  }
  uint32_t codes[D / 16];
  uint32_t prm[D / kGroup];
  float pacc[R > 0 ? R : 1];
#pragma unroll
  for (int m = 0; m < (R > 0 ? R : 1); ++m) pacc[m] = 0.0f;
  residual_q2<D, R, true>(k, cb + (int64_t)bestj * D, nullptr, ul, codes, prm, pacc);
  const int64_t orow = bh * Tcap + cur_len + i;
  kidx[orow] = (uint8_t)bestj;
  uint4* cdst = reinterpret_cast<uint4*>(kcodes + orow * (D / 4));
#pragma unroll
  for (int q = 0; q < D / 64; ++q)
    cdst[q] = make_uint4(codes[4 * q], codes[4 * q + 1], codes[4 * q + 2], codes[4 * q + 3]);
  uint32_t* pdst = kparams + orow * (D / kGroup);
#pragma unroll
  for (int gq = 0; gq < D / kGroup; ++gq) pdst[gq] = prm[gq];
  if constexpr (R > 0) {
    if (flags & kFlagInt8) {
      uint32_t qw[R / 4];
      const uint32_t sh = psac_int8<R>(pacc, qw);
      uint32_t* ps = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(kpsac) + orow * R);
#pragma unroll
      for (int m = 0; m < R / 4; ++m) ps[m] = qw[m];
      kpsac_sc[orow] = (uint16_t)sh;
      return;
    }
  }
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

template <int D, bool QSAC, int R>
hipError_t launch_centroid_cache(const kvq_cache* c, const void* k, int cur_len, int n_new,
                                 hipStream_t st) {
  const kvq_layout& L = c->layout;
  const dim3 grid((unsigned)((n_new + 255) / 256), (unsigned)L.kv_heads, (unsigned)L.batch);
  const bool int8 = R > 0 && L.psac_format == KVQ_PSAC_INT8;
  const int flags = (QSAC && L.qsac_score == KVQ_QSAC_RANGE ? kFlagRange : 0) | (int8 ? kFlagInt8 : 0);
  // INT8 coefficients: R codes per token, then the fp16 scales
  uint16_t* psac_sc =
      int8 ? reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(c->k_psac) +
                                         (size_t)L.batch * L.kv_heads * L.capacity * R)
           : nullptr;
  centroid_kernel<D, QSAC, R, true><<<grid, 256, 0, st>>>(
      (const uint16_t*)k, (int64_t)L.kv_heads * D, D, (int64_t)n_new * L.kv_heads * D, n_new,
      (const float*)c->centroids, L.n_centroids, (const float*)c->sens_w, L.qsac_topk,
      (const float*)c->psac_basis, nullptr, (uint8_t*)c->k_idx, (uint8_t*)c->k_codes,
      (uint32_t*)c->k_params, (uint16_t*)c->k_psac, L.kv_heads, L.capacity, cur_len, flags,
      psac_sc);
  return hipGetLastError();
}

template <int D, bool QSAC>
hipError_t launch_assign_t(const void* keys, int64_t n, int64_t stride, const float* cent,
                           int C, const float* w, int topk, int32_t* out, hipStream_t st) {
  const dim3 grid((unsigned)((n + 255) / 256), 1, 1);
  centroid_kernel<D, QSAC, 0, false><<<grid, 256, 0, st>>>(
      (const uint16_t*)keys, stride, 0, 0, n, cent, C, w, topk, nullptr, out, nullptr,
      nullptr, nullptr, nullptr, 1, 0, 0, 0, nullptr);
  return hipGetLastError();
}


// Lloyd update.  The members of each centroid are first listed in key
// order by a stable counting sort of the assignment (per chunk of 256 keys:
// counts, a prefix over chunks and centroids, then a scatter ranked within
// the chunk by ballots), then one block per centroid sums each channel of
// its members in that order in fp64 and writes the f32 mean (no members:
// the centroid is left as it is).
constexpr int kSortChunk = 256;

struct KmWs {          // workspace carve-up, per (sequence, head) blocks
  int32_t* idx;        // [BH][n] assignment of the current round
  int32_t* members;    // [BH][n] key indices grouped by centroid, key order
  int32_t* cnt;        // [BH][nch][256] per-chunk counts, then offsets
  int32_t* start;      // [BH][256] first slot of each centroid's members
  int32_t* count;      // [BH][256] member counts
};

inline size_t km_align(size_t b) { return (b + 255) & ~(size_t)255; }

inline int64_t km_chunks(int64_t n) { return (n + kSortChunk - 1) / kSortChunk; }

// Bitmask of the lanes of this wave whose 8-bit value equals this lane's
// (keys past the end hold 256 and match only each other).
KVQ_DEV uint64_t match8(int32_t v) {
  uint64_t m = __ballot(1);
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {          // bit 8: the "no key" mark
    const bool set = (v >> bit) & 1;
    const uint64_t b = __ballot(set);
    m &= set ? b : ~b;
  }
  return m;
}

KVQ_DEV int rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// counts of each centroid in chunk blockIdx.x of (sequence, head) bh
__global__ __launch_bounds__(kSortChunk) void km_count_kernel(const int32_t* __restrict__ idx,
                                                              int64_t n, int32_t* __restrict__ cnt) {
  __shared__ int32_t h[256];
  const int t = threadIdx.x;
  const int64_t bh = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int64_t nch = gridDim.x;
  h[t] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kSortChunk + t;
  if (i < n) atomicAdd(&h[idx[bh * n + i]], 1);
  __syncthreads();
  cnt[(bh * nch + blockIdx.x) * 256 + t] = h[t];
}

// per (sequence, head): chunk counts -> global slots (centroid base + the
// members of earlier chunks), centroid starts and counts.  Thread (q, j)
// covers centroid j over quarter q of the chunks.
__global__ __launch_bounds__(1024) void km_offset_kernel(int64_t nch, int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ start,
                                                         int32_t* __restrict__ count) {
  __shared__ int32_t part[4][256];
  __shared__ int32_t sc[256];
  const int j = threadIdx.x & 255, q = threadIdx.x >> 8;
  const int64_t bh = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t per = (nch + 3) / 4, c0 = q * per, c1 = min(nch, c0 + per);
  int32_t* c = cnt + bh * nch * 256 + j;
  int32_t tot = 0;
#pragma unroll 8
  for (int64_t ch = c0; ch < c1; ++ch) tot += c[ch * 256];
  part[q][j] = tot;
  __syncthreads();
  if (q == 0) {
    const int32_t t = part[0][j] + part[1][j] + part[2][j] + part[3][j];
    sc[j] = t;
    count[bh * 256 + j] = t;
  }
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {     // inclusive scan over centroids
    const int32_t v = (q == 0 && j >= o) ? sc[j - o] : 0;
    __syncthreads();
    if (q == 0) sc[j] += v;
    __syncthreads();
  }
  int32_t run = sc[j] - (part[0][j] + part[1][j] + part[2][j] + part[3][j]);
  if (q == 0) start[bh * 256 + j] = run;
  for (int u = 0; u < q; ++u) run += part[u][j];
#pragma unroll 8
  for (int64_t ch = c0; ch < c1; ++ch) {
    const int32_t v = c[ch * 256];
    c[ch * 256] = run;
    run += v;
  }
}

// stable scatter of the key indices of chunk blockIdx.x to their slots
__global__ __launch_bounds__(kSortChunk) void km_scatter_kernel(const int32_t* __restrict__ idx,
                                                                int64_t n,
                                                                const int32_t* __restrict__ cnt,
                                                                int32_t* __restrict__ members) {
  __shared__ int32_t wc[kSortChunk / 64][256];
  const int t = threadIdx.x, w = t >> 6;
  const int64_t bh = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const int64_t nch = gridDim.x;
  for (int e = t; e < (kSortChunk / 64) * 256; e += kSortChunk) (&wc[0][0])[e] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kSortChunk + t;
  const int32_t j = i < n ? idx[bh * n + i] : 256;
  const uint64_t m = match8(j);
  const int r = rank_below(m);
  if (j < 256 && r == 0) wc[w][j] = __builtin_popcountll(m);   // the group's first lane
  __syncthreads();
  if (j < 256) {
    int32_t slot = cnt[(bh * nch + blockIdx.x) * 256 + j] + r;
    for (int u = 0; u < w; ++u) slot += wc[u][j];
    members[bh * n + slot] = (int32_t)i;
  }
}

// One wave per centroid; lane l owns channels CPL*l .. CPL*l + CPL - 1.
// Member rows are gathered kBatch at a time with no per-load branch (the
// tail batch repeats the last member and drops it from the sum), and the
// next batch's member indices are fetched while the rows are in flight.
template <int D>
__global__ __launch_bounds__(64) void km_mean_kernel(const uint16_t* __restrict__ keys_all,
                                                     int64_t n, int64_t stride, int64_t head_stride,
                                                     int64_t batch_stride,
                                                     const int32_t* __restrict__ members,
                                                     const int32_t* __restrict__ start,
                                                     const int32_t* __restrict__ count,
                                                     float* __restrict__ cent_all, int C) {
  constexpr int CPL = D / 64;                  // 2 (head_dim 128) or 1 (64)
  using W = typename std::conditional<CPL == 2, uint32_t, uint16_t>::type;
  constexpr int kBatch = 32;
  const int j = blockIdx.x, l = threadIdx.x;
  const int64_t bh = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
  const uint16_t* keys = keys_all + blockIdx.z * batch_stride + blockIdx.y * head_stride + CPL * l;
  const int32_t m = count[bh * 256 + j];
  if (m == 0) return;
  const int32_t* mem = members + bh * n + start[bh * 256 + j];
  double acc[CPL] = {};
  int32_t r[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) r[u] = mem[u < m ? u : m - 1];
  for (int e = 0; e < m; e += kBatch) {
    W v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      v[u] = *reinterpret_cast<const W*>(keys + (int64_t)r[u] * stride);
    const int e2 = e + kBatch;
    if (e2 < m) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) r[u] = mem[e2 + u < m ? e2 + u : m - 1];
    }
    // a dropped slot adds +0.0, which leaves the sum's bits unchanged: it
    // starts at +0.0 and so is never -0.0
    const int valid = m - e < kBatch ? m - e : kBatch;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const double x = (double)bf16_to_f32((uint16_t)((uint32_t)v[u] >> (16 * c)));
        acc[c] += u < valid ? x : 0.0;
      }
    }
  }
  float* out = cent_all + (bh * C + j) * D + CPL * l;
#pragma unroll
  for (int c = 0; c < CPL; ++c) out[c] = (float)(acc[c] / (double)m);
}

template <int D>
hipError_t launch_kmeans_d(const void* keys, int B, int64_t n, int H, int64_t stride,
                           int64_t head_stride, int64_t batch_stride, float* cent, int C,
                           int iters, int32_t* assign_out, const KmWs& ws, hipStream_t st) {
  const dim3 agrid((unsigned)((n + 255) / 256), (unsigned)H, (unsigned)B);
  const int64_t nch = km_chunks(n);
  const dim3 sgrid((unsigned)nch, (unsigned)H, (unsigned)B);
  auto assign = [&](int32_t* a) {
    centroid_kernel<D, false, 0, false><<<agrid, 256, 0, st>>>(
        (const uint16_t*)keys, stride, head_stride, batch_stride, n, cent, C, nullptr, 1,
        nullptr, a, nullptr, nullptr, nullptr, nullptr, H, 0, 0, 0, nullptr);
    return hipGetLastError();
  };
  for (int it = 0; it < iters; ++it) {
    // the last round's assignment is the one reported
    int32_t* a = (it == iters - 1 && assign_out) ? assign_out : ws.idx;
    hipError_t e = assign(a);
    if (e != hipSuccess) return e;
    km_count_kernel<<<sgrid, kSortChunk, 0, st>>>(a, n, ws.cnt);
    km_offset_kernel<<<dim3((unsigned)H, (unsigned)B), 1024, 0, st>>>(nch, ws.cnt, ws.start,
                                                                     ws.count);
    km_scatter_kernel<<<sgrid, kSortChunk, 0, st>>>(a, n, ws.cnt, ws.members);
    km_mean_kernel<D><<<dim3((unsigned)C, (unsigned)H, (unsigned)B), 64, 0, st>>>(
        (const uint16_t*)keys, n, stride, head_stride, batch_stride, ws.members, ws.start,
        ws.count, cent, C);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (iters == 0 && assign_out) return assign(assign_out);
  return hipSuccess;
}

template <int D>
hipError_t launch_centroid_append_d(const kvq_cache* c, const void* k, int cur_len, int n_new,
                                   hipStream_t st) {
  const kvq_layout& L = c->layout;
  const bool qsac = L.key_mode == KVQ_KEY_CENTROID_QSAC;
  if (L.psac_rank == 8)
    return qsac ? launch_centroid_cache<D, true, 8>(c, k, cur_len, n_new, st)
                : launch_centroid_cache<D, false, 8>(c, k, cur_len, n_new, st);
  return qsac ? launch_centroid_cache<D, true, 0>(c, k, cur_len, n_new, st)
              : launch_centroid_cache<D, false, 0>(c, k, cur_len, n_new, st);
}

}  // namespace

hipError_t launch_centroid_append(const kvq_cache* c, const void* k_bf16, int cur_len,
                                  int n_new, hipStream_t stream) {
  if (n_new == 0) return hipSuccess;
  return (c->layout.head_dim == 128) ? launch_centroid_append_d<128>(c, k_bf16, cur_len, n_new, stream)
                                     : launch_centroid_append_d<64>(c, k_bf16, cur_len, n_new, stream);
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

size_t kmeans_workspace_bytes(int batch, int heads, int64_t n) {
  const size_t bh = (size_t)batch * heads;
  return km_align(bh * n * 4) * 2 + km_align(bh * km_chunks(n) * 256 * 4) +
         km_align(bh * 256 * 4) * 2;
}

hipError_t launch_kmeans(const void* keys, int batch, int64_t n, int heads, int head_dim,
                         int64_t key_stride, int64_t head_stride, int64_t batch_stride,
                         float* centroids, int n_centroids, int iters, int32_t* assign_out,
                         void* ws, hipStream_t stream) {
  if (n == 0 || batch == 0 || heads == 0) return hipSuccess;
  const size_t bh = (size_t)batch * heads;
  char* p = (char*)ws;
  KmWs w;
  w.idx = (int32_t*)p;
  p += km_align(bh * n * 4);
  w.members = (int32_t*)p;
  p += km_align(bh * n * 4);
  w.cnt = (int32_t*)p;
  p += km_align(bh * km_chunks(n) * 256 * 4);
  w.start = (int32_t*)p;
  p += km_align(bh * 256 * 4);
  w.count = (int32_t*)p;
  return head_dim == 128
             ? launch_kmeans_d<128>(keys, batch, n, heads, key_stride, head_stride, batch_stride,
                                    centroids, n_centroids, iters, assign_out, w, stream)
             : launch_kmeans_d<64>(keys, batch, n, heads, key_stride, head_stride, batch_stride,
                                   centroids, n_centroids, iters, assign_out, w, stream);
}

}  // namespace kvq
