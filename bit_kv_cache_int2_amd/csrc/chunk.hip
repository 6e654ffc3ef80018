// Chunk attention: a block of query rows (e.g. the frames being generated)
// against the packed INT2 cache, on the MFMA units.
//
// Block = 4 waves x 32 query rows of one (sequence, query head).  The
// cached tokens stream through in 64-token tiles: the packed codes and
// parameter words are staged in LDS, dequantised by all 256 threads into
// fp16 tiles (keys row-major, values transposed), and consumed by
// v_mfma_f32_16x16x32_f16:
//   S^T = Khat Q^T  (A = key tile from LDS, B = the wave's queries, kept in
//                    registers for the whole loop),
//   O^T += Vhat^T P^T (A = transposed value tile, B = P straight from the
//                    score registers: the token order inside each 32-token
//                    k-step is permuted so that every lane already holds
//                    the eight P values it must supply).
// Each lane owns whole query rows, so the online-softmax max needs only two
// cross-lane steps.  Precision: fp16 operands with fp32 accumulation;
// window-range keys (whose per-channel scales make logits large) are split
// as Khat = hi + lo, both fp16, and multiplied twice; centroid keys use one
// fp16 copy.  PSAC ([QWM] 2) adds (U^T q) . a as one more 16x16x16 MFMA
// k-step.  Rotated values ([OKV]) are rotated back in registers at the end.
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNT = 2;              // 16-row query tiles per wave
constexpr int kBM = 4 * kNT * 16;   // query rows per block

struct ChunkArgs {
  const uint8_t* kcodes;
  const uint32_t* kparams;
  const uint16_t* ktail;
  const uint8_t* kidx;
  const float* cent;
  const float* basis;
  const uint16_t* kpsac;
  const uint8_t* vcodes;
  const uint32_t* vparams;
  const uint16_t* q;
  void* out;
  float* lse;
  int H, Hq, Tcap, C, n_tokens, Lq, out_bf16;
  float scale_log2;
};

KVQ_DEV _Float16 to_h(float x) { return (_Float16)x; }

template <int D, int KM, bool HAD, int R>
__global__ __launch_bounds__(256) void chunk_kernel(const ChunkArgs a) {
  constexpr int NKS = D / 32;        // QK k-steps
  constexpr int NDT = D / 16;        // PV output dim tiles
  constexpr bool LO = (KM == 0);     // hi/lo split keys
  constexpr int KP = D + 8;          // key tile pitch (halfs)
  constexpr int VP = 64 + 8;         // transposed value tile pitch (halfs)
  constexpr int RB = D / 4;          // packed bytes per token row
  constexpr int NG = D / kGroup;     // parameter groups per row
  constexpr int TPT = 64 * RB / 256; // tokens per thread in the dequant
  __shared__ __align__(16) _Float16 khi[64 * KP];
  __shared__ __align__(16) _Float16 klo[LO ? 64 * KP : 8];
  __shared__ __align__(16) _Float16 vt[D * VP];
  __shared__ __align__(16) _Float16 coef[R > 0 ? 64 * 16 : 8];
  __shared__ __align__(16) uint8_t kc[64 * RB];
  __shared__ __align__(16) uint8_t vc[64 * RB];
  __shared__ __align__(16) uint32_t vpw[64 * NG];
  __shared__ __align__(16) uint32_t kpw[KM == 0 ? D : 64 * NG];
  __shared__ int kix[64];

  const int qt = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.H, h = hq / G;
  const int64_t bh = (int64_t)b * a.H + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int row0 = qt * kBM + wave * kNT * 16;
  const int n = a.n_tokens;

  // ---- queries (B operand), fp16, resident for the whole loop
  h8 qreg[kNT][NKS];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int row = row0 + nt * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      h8 v;
      if (row < a.Lq) {
        const uint4 u = *reinterpret_cast<const uint4*>(
            a.q + (((int64_t)b * a.Lq + row) * a.Hq + hq) * D + ks * 32 + 8 * g);
        float x[8];
        bf16x8_to_f32(u, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = to_h(x[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (_Float16)0.0f;
      }
      qreg[nt][ks] = v;
    }
  }
  // ---- PSAC: q' = U^T q (lane supplies q'[4g .. 4g+3] of its row, g < 2)
  h4 qp[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) qp[nt][j] = (_Float16)0.0f;
    if (R > 0) {
      const int row = row0 + nt * 16 + c16;
      if (g < 2 && row < a.Lq) {
        const uint16_t* qr = a.q + (((int64_t)b * a.Lq + row) * a.Hq + hq) * D;
        const float* U = a.basis + bh * D * (R > 0 ? R : 1);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int d = 0; d < D; ++d) {
          const float qd = bf16_to_f32(qr[d]);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(U[d * R + 4 * g + j], qd, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) qp[nt][j] = to_h(acc[j]);
      }
    }
  }

  float m_run[kNT], l_run[kNT];
  f4 o[kNT][NDT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    m_run[nt] = -__builtin_inff();
    l_run[nt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[nt][dt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int n_tiles = (n + 63) / 64;
  const int n_full = n / 64;
  const int bc = tid % RB, tg = tid / RB;   // dequant: 4 channels x TPT tokens

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int t0 = tile * 64;
    const int64_t rowbase = bh * a.Tcap + t0;
    __syncthreads();  // the previous tile's LDS tiles are consumed
    // ---- stage packed data (the tile lies inside the capacity)
    // key rows [token][D/4]; the value tile is channel-major [D][16]
    const int64_t vtile = (bh * (a.Tcap / 64) + tile) * (int64_t)D * 16;
    for (int e = tid; e < 64 * RB / 16; e += 256) {
      reinterpret_cast<uint4*>(kc)[e] = reinterpret_cast<const uint4*>(a.kcodes + rowbase * RB)[e];
      reinterpret_cast<uint4*>(vc)[e] = reinterpret_cast<const uint4*>(a.vcodes + vtile)[e];
    }
    for (int e = tid; e < 64 * NG; e += 256) vpw[e] = a.vparams[rowbase * NG + e];
    if (KM == 0) {
      if (tile < n_full)
        for (int e = tid; e < D; e += 256) kpw[e] = a.kparams[(bh * (a.Tcap / 64) + tile) * D + e];
    } else {
      for (int e = tid; e < 64 * NG; e += 256) kpw[e] = a.kparams[rowbase * NG + e];
      if (tid < 64) kix[tid] = a.kidx[rowbase + tid];
    }
    if (R > 0) {
      for (int e = tid; e < 64 * 16; e += 256) {
        const int t = e >> 4, m = e & 15;
        coef[e] = (m < R && t0 + t < n)
                      ? __builtin_bit_cast(_Float16, a.kpsac[(rowbase + t) * R + m])
                      : (_Float16)0.0f;
      }
    }
    __syncthreads();
    // ---- dequantise keys -> khi (+ klo), row-major [token][dim]
    {
      float s4[4], z4[4];
      if (KM == 0 && tile < n_full) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s4[j] = f16_bits_to_f32(kpw[4 * bc + j]);
          z4[j] = f16_bits_to_f32(kpw[4 * bc + j] >> 16);
        }
      }
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int t = tg * TPT + u;
        float kv[4];
        if (t0 + t >= n) {
#pragma unroll
          for (int j = 0; j < 4; ++j) kv[j] = 0.0f;
        } else if (KM == 0) {
          if (tile < n_full) {
            const uint32_t byte = kc[t * RB + bc];
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[j] = __builtin_fmaf((float)((byte >> (2 * j)) & 3u), s4[j], z4[j]);
          } else {
            const uint16_t* kt = a.ktail + (bh * 64 + t) * D + 4 * bc;
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[j] = bf16_to_f32(kt[j]);
          }
        } else {
          const uint32_t byte = kc[t * RB + bc];
          const uint32_t pw = kpw[t * NG + (4 * bc) / kGroup];
          const float s = f16_bits_to_f32(pw), z = f16_bits_to_f32(pw >> 16);
          const float4 cc = *reinterpret_cast<const float4*>(
              a.cent + (bh * a.C + kix[t]) * D + 4 * bc);
          const float cv[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            kv[j] = cv[j] + __builtin_fmaf((float)((byte >> (2 * j)) & 3u), s, z);
        }
        h4 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hi[j] = to_h(kv[j]);
          lo[j] = to_h(kv[j] - (float)hi[j]);
        }
        *reinterpret_cast<h4*>(&khi[t * KP + 4 * bc]) = hi;
        if (LO) *reinterpret_cast<h4*>(&klo[t * KP + 4 * bc]) = lo;
      }
    }
    // ---- dequantise values -> vt, transposed [dim][token]
    {
      _Float16 vv[4][TPT];
      uint32_t cw[4];   // codes of tokens tg*TPT .. +TPT for channels 4bc .. 4bc+3
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t* cr = &vc[(4 * bc + j) * 16 + (tg * TPT) / 4];
        cw[j] = (TPT == 8) ? (uint32_t)*reinterpret_cast<const uint16_t*>(cr) : (uint32_t)*cr;
      }
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int t = tg * TPT + u;
        const bool ok = t0 + t < n;
        const uint32_t pw = vpw[t * NG + (4 * bc) / kGroup];
        const float s = f16_bits_to_f32(pw), z = f16_bits_to_f32(pw >> 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vv[j][u] = ok ? to_h(__builtin_fmaf((float)((cw[j] >> (2 * u)) & 3u), s, z)) : (_Float16)0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        _Float16* dst = &vt[(4 * bc + j) * VP + tg * TPT];
#pragma unroll
        for (int u = 0; u < TPT; u += 4) {
          h4 w4 = {vv[j][u], vv[j][u + 1], vv[j][u + 2], vv[j][u + 3]};
          *reinterpret_cast<h4*>(dst + u) = w4;
        }
      }
    }
    __syncthreads();

    // ---- S^T = Khat Q^T
    f4 s[kNT][4];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int ts = 0; ts < 4; ++ts) s[nt][ts] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const h8 ka = *reinterpret_cast<const h8*>(&khi[(ts * 16 + c16) * KP + ks * 32 + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qreg[nt][ks], s[nt][ts], 0, 0, 0);
        if (LO) {
          const h8 kl = *reinterpret_cast<const h8*>(&klo[(ts * 16 + c16) * KP + ks * 32 + 8 * g]);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            s[nt][ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, qreg[nt][ks], s[nt][ts], 0, 0, 0);
        }
      }
      if (R > 0) {
        const h4 ca = *reinterpret_cast<const h4*>(&coef[(ts * 16 + c16) * 16 + 4 * g]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][ts] = __builtin_amdgcn_mfma_f32_16x16x16f16(ca, qp[nt], s[nt][ts], 0, 0, 0);
      }
    }

    // ---- online softmax (base 2); lane owns rows nt*16 + c16, tokens ts*16 + 4g + i
    h8 pb[kNT][2];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float x[4][4];
      float mx = -__builtin_inff();
#pragma unroll
      for (int ts = 0; ts < 4; ++ts)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = t0 + ts * 16 + 4 * g + i < n;
          x[ts][i] = ok ? s[nt][ts][i] * a.scale_log2 : -__builtin_inff();
          mx = fmaxf(mx, x[ts][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m_run[nt], mx);
      const float alpha = exp2f(m_run[nt] - mn);
      float ls = 0.0f;
#pragma unroll
      for (int ts = 0; ts < 4; ++ts)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(x[ts][i] - mn);
          ls += p;
          pb[nt][ts >> 1][(ts & 1) * 4 + i] = to_h(p);
        }
      l_run[nt] = __builtin_fmaf(l_run[nt], alpha, ls);
      m_run[nt] = mn;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[nt][dt] *= alpha;
    }

    // ---- O^T += Vhat^T P^T (k index j of lane group g <-> token
    //      kk*32 + (j < 4 ? 4g + j : 16 + 4g + j - 4))
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const _Float16* vr = &vt[(dt * 16 + c16) * VP + kk * 32 + 4 * g];
        const h4 v0 = *reinterpret_cast<const h4*>(vr);
        const h4 v1 = *reinterpret_cast<const h4*>(vr + 16);
        const h8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[nt][kk], o[nt][dt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalise, rotate back, store
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    float v[NDT][4];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[dt][i] = o[nt][dt][i] * inv;
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
      const float c = (D == 128) ? 0.08838834764831845f : 0.125f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[dt][i] *= c;
    }
    const int row = row0 + nt * 16 + c16;
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

template <int D, int KM, bool HAD, int R>
hipError_t launch_t(const ChunkArgs& a, int B, hipStream_t st) {
  const dim3 grid((unsigned)((a.Lq + kBM - 1) / kBM), (unsigned)a.Hq, (unsigned)B);
  chunk_kernel<D, KM, HAD, R><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ChunkArgs& a, int key_mode, bool had, int R, int B, hipStream_t st) {
  if (key_mode == KVQ_KEY_WINDOW)
    return had ? launch_t<D, 0, true, 0>(a, B, st) : launch_t<D, 0, false, 0>(a, B, st);
  if (R == 8)
    return had ? launch_t<D, 1, true, 8>(a, B, st) : launch_t<D, 1, false, 8>(a, B, st);
  return had ? launch_t<D, 1, true, 0>(a, B, st) : launch_t<D, 1, false, 0>(a, B, st);
}

}  // namespace

size_t chunk_workspace_bytes(const kvq_layout*, int, int, int) { return 0; }

hipError_t launch_chunk(const kvq_cache* c, int n_tokens, const void* q, int q_len,
                        int q_heads, float scale, void* out, int out_dtype, float* lse,
                        void*, hipStream_t stream) {
  const kvq_layout& L = c->layout;
  ChunkArgs a;
  a.kcodes = (const uint8_t*)c->k_codes;
  a.kparams = (const uint32_t*)c->k_params;
  a.ktail = (const uint16_t*)c->k_tail;
  a.kidx = (const uint8_t*)c->k_idx;
  a.cent = (const float*)c->centroids;
  a.basis = (const float*)c->psac_basis;
  a.kpsac = (const uint16_t*)c->k_psac;
  a.vcodes = (const uint8_t*)c->v_codes;
  a.vparams = (const uint32_t*)c->v_params;
  a.q = (const uint16_t*)q;
  a.out = out;
  a.lse = lse;
  a.H = L.kv_heads;
  a.Hq = q_heads;
  a.Tcap = L.capacity;
  a.C = L.n_centroids;
  a.n_tokens = n_tokens;
  a.Lq = q_len;
  a.out_bf16 = out_dtype == KVQ_BF16;
  a.scale_log2 = scale * kLog2e;
  const int R = (L.key_mode == KVQ_KEY_WINDOW) ? 0 : L.psac_rank;
  const bool had = L.value_mode == KVQ_VAL_HADAMARD;
  return (L.head_dim == 128) ? launch_d<128>(a, L.key_mode, had, R, L.batch, stream)
                             : launch_d<64>(a, L.key_mode, had, R, L.batch, stream);
}

}  // namespace kvq
