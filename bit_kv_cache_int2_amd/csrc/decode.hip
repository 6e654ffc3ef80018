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
//    part is a per-lane running sum sum_t p_t z_(t,g).  With per-modality
//    rotations each code takes the sign of its (token modality, channel) and
//    the z part is summed per modality, signed per channel at the end.
// The online softmax works in base 2 (logits pre-scaled by log2 e) with
// wave-shuffle maxima; each block merges its four waves and writes one
// partial (o, m, l); a second kernel merges the splits, rotates rotated
// values back and writes out/lse.
#include <mutex>

#include "code_operand.h"
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Most windows one split (one block) covers: eight per wave.
constexpr int kDecodeMaxWindows = 32;
constexpr double kBlockOverheadWindows = 16.0;   // see decode_splits
// Resident blocks per CU of the MFMA decode kernel (LDS and register use
// are sized for three).
constexpr int kDecodeBlocksPerCU = 3;
// Fourth word of a raw buffer resource (32-bit data format), and the
// non-temporal cache policy for streamed cache reads.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNT = 2;
// Prefetch distances (windows) of the MFMA decode's key and value streams.
// Pass 1 requests the first value windows during its last kKeyAhead steps
// and pass 2 requests window k + kValAhead at its step k, so every value
// window is requested exactly once only while kValAhead <= kKeyAhead.
constexpr int kKeyAhead = 3, kValAhead = 3;
static_assert(kValAhead <= kKeyAhead, "value windows kKeyAhead..kValAhead-1 would never be loaded");

// Orders one wave's LDS writes before its following LDS reads (data shared
// between lanes of a wave).  The fences are restricted to LDS ("local"), so
// they do not wait for the wave's outstanding global loads.
KVQ_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

struct DecodeArgs {
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
  const void* q;
  float* ws;
  int q_bf16, H, Hq, Tcap, C, n_tokens, split_len, S, psac_int8, M;
  float scale_log2;
};

template <int D, int G, int KM, int R, bool MOD>
__global__ __launch_bounds__(256) void decode_partial_kernel(const DecodeArgs a) {
  constexpr int NG = D / kGroup;      // parameter groups per row
  constexpr int CPL = D / kWave;      // P.V channels per lane
  constexpr int NM = MOD ? 3 : 1;     // modality z sums kept per lane
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

  // per-modality rotations: bit m of csgn[c] = sign of channel lane*CPL + c
  // in modality m
  uint32_t csgn[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    csgn[c] = 0u;
    if (MOD) {
      const int ch = lane * CPL + c;
      for (int m = 0; m < a.M; ++m)
        csgn[c] |= ((a.vsigns[((int64_t)h * a.M + m) * (D / 32) + ch / 32] >> (ch & 31)) & 1u) << m;
    }
  }

  float m_run[G], l_lane[G], pz[G][NM][NG], o[G][CPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -__builtin_inff();
    l_lane[g] = 0.0f;
#pragma unroll
    for (int mm = 0; mm < NM; ++mm)
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) pz[g][mm][gr] = 0.0f;
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
          // a_m: fp16, or INT8 code times the token's scale (exact in fp32)
          const uint16_t* ap = a.kpsac + tr * R;
          const int8_t* aq = reinterpret_cast<const int8_t*>(a.kpsac) + tr * R;
          const float sc = a.psac_int8 ? f16_bits_to_f32(a.kpsac_sc[tr]) : 0.0f;
#pragma unroll
          for (int m = 0; m < R; ++m) {
            const float am = a.psac_int8 ? (float)aq[m] * sc : f16_bits_to_f32(ap[m]);
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
      for (int mm = 0; mm < NM; ++mm)
#pragma unroll
        for (int gr = 0; gr < NG; ++gr) pz[g][mm][gr] *= alpha;
      m_run[g] = mn;
    }
    // this lane's token's modality (per-modality rotations)
    const int mt = MOD ? min((int)a.vmodal[(int64_t)b * a.Tcap + min(t, a.n_tokens - 1)], a.M - 1) : 0;

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
#pragma unroll
          for (int mm = 0; mm < NM; ++mm)
            pz[g][mm][gr] = __builtin_fmaf((mm == mt) ? pg : 0.0f, zc, pz[g][mm][gr]);
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
        // modality of token tt (wave-uniform): that of lane tt
        const int mtt = MOD ? __builtin_amdgcn_readlane(mt, tt) : 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const uint32_t wd = (tt < 16) ? crow[c].x : (tt < 32) ? crow[c].y : (tt < 48) ? crow[c].z : crow[c].w;
          cf[c] = (float)((wd >> (2 * (tt & 15))) & 3u);
          if (MOD) cf[c] = __uint_as_float(__float_as_uint(cf[c]) ^ (((csgn[c] >> mtt) & 1u) << 31));
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
      float zsum[NM][NG];
#pragma unroll
      for (int mm = 0; mm < NM; ++mm)
#pragma unroll
        for (int q = 0; q < NG; ++q) zsum[mm][q] = wave_sum(pz[g][mm][q]);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float zc = 0.0f;
#pragma unroll
        for (int mm = 0; mm < NM; ++mm)
          zc += ((csgn[c] >> mm) & 1u) ? -zsum[mm][gr] : zsum[mm][gr];
        wo[wave][g][c0 + c] = o[g][c] + zc;
      }
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

// ---------------------------------------------------------------- MFMA decode
// Window keys, head_dim 128, 4 query heads per kv head.  Both products run
// on v_mfma_f32_16x16x32_f16 with the 2-bit codes as one operand, encoded
// as exact fp16 values base + code: a code moved to mantissa bits 8-9 under
// exponent 2 reads 4 + code, bits 6-7 under exponent 4 read 16 + code,
// bits 4-5 under exponent 6 read 64 + code.  Code i of a 32-bit code word
// sits at bit 2i of its 16-bit half: shifts by 6, 0 and -6 bring codes
// (0, 1), (2, 3, 4) and (5, 6, 7) to those positions, and one and-or per
// operand dword places codes (i, i + 8), so a 16-code word costs two
// shifts and eight and-ors.  Position i has base {16, 4, 64, 16, 4, 64, 16,
// 4}[i].  All products are exact.
//   S^T[token][head] = sum_c (base_c + code[token][c]) qt[head][c] with the
//     hi and lo fp16 parts of qt = q * s_w * scale * log2 e in B columns
//     0..3 and 4..7 (the same code operand multiplies both; columns 8..15
//     are copies, never read), added after the MFMA, so lanes c16 < 4 of
//     each 16-lane row hold the logits of head c16; the window bias
//     sum_c q_c (z_c - base_c s_c), the hi columns' initial value, adds
//     the zero points and removes the base term;
//   O^T[c][col] = sum_t (base_t + code[t][c]) pt[t][col] with col = 4 group
//     + head and pt = fp16(p * s_(t,group)); only the columns of a channel's
//     own group are kept; the base term comes from one more MFMA against a
//     constant operand holding the bases (same fp16 pt values), and
//     sum_t p z_(t,group) is a per-lane fp32 sum.
// A wave owns at most eight windows of its split (every fourth one).  Pass
// 1 streams their key codes, stores the logits (base 2) in LDS and takes
// the exact per-head maximum; the partial window (bf16 key tail) of a
// sequence is scored with fp32 dot products.  Pass 2 streams the value
// codes and accumulates p = 2^(l - m) <= 1: no running rescale.  Each pass
// requests the wave's windows kKeyAhead (keys) or kValAhead (values) of its
// own windows ahead of the one it computes.

// Sums four per-lane values over the wave: afterwards every lane of row r
// (lanes 16r .. 16r + 15) holds the total of v[r].  Each xor exchange
// halves the values a lane keeps (lanes below 32 keep v[0], v[1]; then rows
// with bit 4 clear keep the first of the two), then rotations inside each
// row finish the sum.  (The permlane swap builtins would save two
// exchanges, but this compiler merges their two results when both feed
// one expression.)
// Lane exchanges without the generic shuffle's per-call index arithmetic
// (lane_xor in device.h); a broadcast from lane src is a bpermute.
KVQ_DEV float lane_read(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

KVQ_DEV float wave_sum4(const float v[4]) {
  const int lane = threadIdx.x & 63;
  const bool hi32 = (lane & 32) != 0, hi16 = (lane & 16) != 0;
  const float k0 = hi32 ? v[2] : v[0], k1 = hi32 ? v[3] : v[1];
  const float s0 = hi32 ? v[0] : v[2], s1 = hi32 ? v[1] : v[3];
  const float a0 = k0 + lane_xor<32>(s0), a1 = k1 + lane_xor<32>(s1);
  const float k = hi16 ? a1 : a0, sn = hi16 ? a0 : a1;
  float y = k + lane_xor<16>(sn);
  y += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), 0x128, 0xF, 0xF, false));
  y += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), 0x124, 0xF, 0xF, false));
  y += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), 0x122, 0xF, 0xF, false));
  y += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), 0x121, 0xF, 0xF, false));
  return y;
}

// Value of lane + 4 inside the 16-lane row (0 past its end).
KVQ_DEV float row_shl4(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x104, 0xF, 0xF, false));
}

// Sums sixteen per-lane values over the wave and returns, in each lane, the
// total of v[j] for j = jsel (0..15).  Four exchanges halve the values a lane
// keeps (partners across bits 5, 4, 3 and 2 of the lane: xor 32, xor 16,
// a rotation by 8 inside the row, a mirror inside each half row), so lane
// l ends with a partial of v[(l >> 2) & 15]; a quad sum completes it and
// one shuffle fetches the wanted total.
KVQ_DEV float wave_sum16_at(const float v[16], int jsel) {
  const int lane = threadIdx.x & 63;
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4;
  float a[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float keep = b5 ? v[m + 8] : v[m], send = b5 ? v[m] : v[m + 8];
    a[m] = keep + lane_xor<32>(send);
  }
  float c4[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float keep = b4 ? a[n + 4] : a[n], send = b4 ? a[n] : a[n + 4];
    c4[n] = keep + lane_xor<16>(send);
  }
  float c2[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float keep = b3 ? c4[r + 2] : c4[r], send = b3 ? c4[r] : c4[r + 2];
    c2[r] = keep + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                       0, __builtin_bit_cast(int, send), 0x128, 0xF, 0xF, false));   // row_ror:8
  }
  const float keep = b2 ? c2[1] : c2[0], send = b2 ? c2[0] : c2[1];
  float y = keep + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                       0, __builtin_bit_cast(int, send), 0x141, 0xF, 0xF, false));   // row_half_mirror
  y += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  y += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  return lane_read(y, 4 * jsel);
}

__global__ __launch_bounds__(256, 3) void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int D = 128, G = 4, MAXW = kDecodeMaxWindows / 4;
  __shared__ float qs[D][G];                                   // q * scale * log2 e
  // A wave's LDS accesses spread over the 64 banks: qb heads are padded
  // by 4 dwords, pb columns by 4.  sl is unpadded (the four heads' logit
  // writes share banks, but each write is one base register plus an
  // immediate offset).  After pass 2 a wave's sl region holds its partial
  // output.
  // qb (pass 1, two buffers) and pb (pass 2) share one region per wave.
  __shared__ __align__(16) uint32_t qpb[4][2][4][132];
  uint32_t (*const qb)[4][132] = qpb[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];   // [buf][head][(hi,lo) g ks] 8 halfs
  __shared__ __align__(16) float sl[4][MAXW][G][kWave];        // [wave][slot][head][token]
  _Float16 (*const pb)[72] = reinterpret_cast<_Float16 (*)[72]>(&qpb[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)][0][0][0]);   // [col][(g kk) 8 halfs]
  static_assert(sizeof(qpb[0]) >= 16 * 72 * sizeof(_Float16), "pb fits in a wave's share");
  __shared__ float wm[4][G], wlv[4][G];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  // the wave index is uniform in a wave; saying so keeps window offsets scalar
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t bh = (int64_t)b * a.H + h;
  const int hq0 = h * G;
  for (int e = tid; e < G * D; e += 256) {
    const int hh = e / D, c = e % D;
    const int64_t qi = ((int64_t)b * a.Hq + hq0 + hh) * D + c;
    const float qv = a.q_bf16 ? bf16_to_f32(((const uint16_t*)a.q)[qi]) : ((const float*)a.q)[qi];
    qs[c][hh] = qv * a.scale_log2;
  }
  __syncthreads();

  const int t_begin = s * a.split_len;
  const int t_end = min(t_begin + a.split_len, a.n_tokens);
  const int n_full_win = a.n_tokens / kWindow;
  const int w_end = (t_end + kWindow - 1) / kWindow;
  const int wf_end = min(w_end, n_full_win);
  const int w_first = t_begin / kWindow + wave;               // this wave's first window

  CodeOr kor = {0x54005400u, 0x4C004C00u, 0x44004400u};
  asm volatile("" : "+v"(kor.b64), "+v"(kor.b16), "+v"(kor.b4));
  // buffer views of this (sequence, kv head): window offsets go in the
  // scalar offset, per-lane offsets are fixed; lanes past the end read 0
  const int nwin_cap = a.Tcap / kWindow;
  const auto rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.kcodes + bh * a.Tcap * (D / 4)), (short)0, a.Tcap * (D / 4), kBufferWord3);
  const auto rkp = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.kparams + bh * nwin_cap * D), (short)0, nwin_cap * D * 4, kBufferWord3);
  const auto rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.vcodes + bh * nwin_cap * (int64_t)D * 16), (short)0, nwin_cap * D * 16, kBufferWord3);
  const auto rvp = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.vparams + bh * a.Tcap * 4), (short)0, a.n_tokens * 16, kBufferWord3);
  // a window past the wave's last one loads through an empty view: the
  // load instructions stay unconditional (so waits stay exact) and read 0
  const auto rnone = __builtin_amdgcn_make_buffer_rsrc((void*)a.kcodes, (short)0, 0, kBufferWord3);

  // ================= pass 1: logits
  // this lane's channel pair for the query fold: ca and ca + 8, position
  // fi of its code word (even: base 16, odd: base 4)
  const int fi = lane & 7;
  const int ca = (lane >> 3) * 16 + fi, cb = ca + 8;
  const int qks = 2 * ((lane >> 3) & 1) + (fi >> 2), qi2 = fi & 3, qg = lane >> 4;
  const float fbase = code_base(fi);
  float qa[G], qbv[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    qa[hh] = qs[ca][hh];
    qbv[hh] = qs[cb][hh];
  }
  struct KWin {
    uint2 kc[4];       // key codes: token ts*16 + c16, channels 32g .. 32g+31
    uint32_t pa, pb;   // window parameters of channels ca, cb
  };
  const int ko = c16 * (D / 4) + 8 * g, vo = c16 * 16 + 4 * g;
  auto fetch_keys = [&](int win, KWin& f, bool live) {
    const int w = __builtin_amdgcn_readfirstlane(win);
    const int so = w * kWindow * (D / 4), sp = w * D * 4;
    const auto r0 = live ? rk : rnone, r1 = live ? rkp : rnone;
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(r0, ko + ts * 16 * (D / 4), so, kNT);
      f.kc[ts] = make_uint2(v[0], v[1]);
    }
    f.pa = __builtin_amdgcn_raw_buffer_load_b32(r1, ca * 4, sp, kNT);
    f.pb = __builtin_amdgcn_raw_buffer_load_b32(r1, cb * 4, sp, kNT);
    // keep each window's loads together and in issue order: the wait for
    // window w then leaves every later window's loads in flight
    __builtin_amdgcn_sched_barrier(0);
  };
  struct VWin {
    uint32_t vcw[8];   // value codes: channel mt*16 + c16, tokens 16g .. 16g+15
    uint4 vp;          // value parameters of token lane
  };
  auto fetch_values = [&](int win, VWin& f, bool live) {
    const int w = __builtin_amdgcn_readfirstlane(win);
    const int so = w * D * 16;
    const auto r0 = live ? rv : rnone, r1 = live ? rvp : rnone;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      f.vcw[mt] = __builtin_amdgcn_raw_buffer_load_b32(r0, vo + mt * 256, so, kNT);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r1, lane * 16, w * kWindow * 16, kNT);
    f.vp = make_uint4(v[0], v[1], v[2], v[3]);
    __builtin_amdgcn_sched_barrier(0);
  };

  float mx = -__builtin_inff();        // running max of head (lane % 4)
  // Pass 1 is pipelined one window deep: the query fold of window k + 1
  // (q~ hi/lo into query buffer (k + 1) & 1, and its bias, whose lane
  // exchanges are long-latency) is issued while the MFMAs of window k run.
  // fold returns the accumulator's initial value for this lane: row r of
  // the bias sum is head r's, and only the hi columns (0..3) take it.
  auto fold = [&](const KWin& cur, int buf) -> float {
    const float sa = f16_bits_to_f32(cur.pa), za = f16_bits_to_f32(cur.pa >> 16);
    const float sb = f16_bits_to_f32(cur.pb), zb = f16_bits_to_f32(cur.pb >> 16);
    const float zca = __builtin_fmaf(-fbase, sa, za), zcb = __builtin_fmaf(-fbase, sb, zb);
    float bias[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const auto hi = __builtin_amdgcn_cvt_pkrtz(qa[hh] * sa, qbv[hh] * sb);
      const float la = __builtin_fmaf(qa[hh], sa, -(float)hi[0]);
      const float lb = __builtin_fmaf(qbv[hh], sb, -(float)hi[1]);
      const auto lo = __builtin_amdgcn_cvt_pkrtz(la, lb);
      qb[buf][hh][qg * 16 + qks * 4 + qi2] = __builtin_bit_cast(uint32_t, hi);
      qb[buf][hh][64 + qg * 16 + qks * 4 + qi2] = __builtin_bit_cast(uint32_t, lo);
      bias[hh] = __builtin_fmaf(qa[hh], zca, qbv[hh] * zcb);
    }
    const float bsum = wave_sum4(bias);
    const float bl = lane_read(bsum, (c16 & 3) * 16);
    return c16 < 4 ? bl : 0.0f;
  };
  // the logits of a window whose fold is in query buffer buf (already
  // ordered before this read by a wave_lds_sync) into sl slot `slot`;
  // `next` runs between the MFMAs' issue and the reads of their results
  auto window_logits = [&](const KWin& cur, int buf, float bc, int slot, auto next) {
    const f4 binit = f4{bc, bc, bc, bc};
    // B operand columns: 0..3 hi parts of heads 0..3, 4..7 lo parts,
    // 8..15 copies (never read)
    h8 bq[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bq[ks] = *reinterpret_cast<const h8*>(&qb[buf][c16 & 3][((c16 >> 2) & 1) * 64 + g * 16 + ks * 4]);
    // four independent accumulator chains (token slabs ts), step-major
    f4 sacc[4] = {binit, binit, binit, binit};
#pragma unroll
    for (int wd = 0; wd < 2; ++wd) {
      uint32_t kw[4][8];
#pragma unroll
      for (int ts = 0; ts < 4; ++ts) code_word(wd ? cur.kc[ts].y : cur.kc[ts].x, kor, kw[ts]);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
          sacc[ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              as_h8(kw[ts][4 * hf], kw[ts][4 * hf + 1], kw[ts][4 * hf + 2], kw[ts][4 * hf + 3]),
              bq[2 * wd + hf], sacc[ts], 0, 0, 0);
    }
    next();
    // hi + lo: column c16 < 4 adds column c16 + 4 (row shift by 4 lanes);
    // only lanes c16 < 4 carry logits from here on
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      float v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = sacc[ts][i];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] += row_shl4(v4[i]);
      mx = fmaxf(fmaxf(fmaxf(mx, v4[0]), v4[1]), fmaxf(v4[2], v4[3]));
      if (c16 < 4)
        *reinterpret_cast<f4*>(&sl[wave][slot][c16][ts * 16 + 4 * g]) = f4{v4[0], v4[1], v4[2], v4[3]};
    }
  };

  // windows of this wave: w_first + 4k for k < n_mine, the first n_full of
  // them full; slot k of sl holds window k.  Keys are fetched kKeyAhead
  // windows ahead, values kValAhead ahead (the first ones during pass 1).
  const int n_mine = w_first < w_end ? (w_end - w_first + 3) / 4 : 0;
  const int n_full = w_first < wf_end ? (wf_end - w_first + 3) / 4 : 0;
  // ================= pass 2 state: p = 2^(l - M), P.V
  float M[G];
  float l_lane[G], pz[G][4];
  f4 o[8], ocorr;
  // The value operand of token t is base + c (c the code); the P~ operand
  // rounds p s once per (token, group).  The output removes (base + 3/2)
  // per token through the vbase MFMA and adds z + 3/2 s through pz, so
  // what P~'s rounding multiplies is s (c - 3/2), which has both signs
  // within a group.  (Removing only the base would leave s c, of one sign,
  // and an inverse rotation gathers such same-signed errors into one
  // output channel: 2.0e-3 instead of 2.5e-4 on a rotated cache with value
  // ranges near 9.)  base + 3/2 is exact in fp16.
  // Dword j of k-step k2 holds the tokens of code-word positions
  // i = 4 k2 + j and i + 8.
  h8 vbase[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int j = 0; j < 8; ++j) vbase[k2][j] = (_Float16)(code_base(4 * k2 + j / 2) + 1.5f);
  // P~ -> LDS in the operand's token order: token 16 gk + o pairs with
  // o + 8; k index 2 i' + (o >= 8) of k-step (o % 8) / 4
  const int kk = (c16 & 7) >> 2, jj = 2 * (c16 & 3) + (c16 >> 3);
  auto window_pv = [&](const VWin& cur, int slot) {
    const uint32_t vw[4] = {cur.vp.x, cur.vp.y, cur.vp.z, cur.vp.w};
    float sc[4], zc[4];   // group scale, and zero + 3/2 scale (see vbase)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sc[q] = f16_bits_to_f32(vw[q]);
      zc[q] = __builtin_fmaf(1.5f, sc[q], f16_bits_to_f32(vw[q] >> 16));
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float p = __builtin_amdgcn_exp2f(sl[wave][slot][hh][lane] - M[hh]);
      l_lane[hh] += p;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pz[hh][q] = __builtin_fmaf(p, zc[q], pz[hh][q]);
        pb[4 * q + hh][g * 16 + kk * 8 + jj] = (_Float16)(p * sc[q]);
      }
    }
    wave_lds_sync();
    h8 bpv[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) bpv[k2] = *reinterpret_cast<const h8*>(&pb[c16][g * 16 + k2 * 8]);
#pragma unroll
    for (int m0 = 0; m0 < 8; m0 += 4) {
      uint32_t vx[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) code_word(cur.vcw[m0 + u], kor, vx[u]);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[m0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              as_h8(vx[u][4 * k2], vx[u][4 * k2 + 1], vx[u][4 * k2 + 2], vx[u][4 * k2 + 3]), bpv[k2],
              o[m0 + u], 0, 0, 0);
    }
    ocorr = __builtin_amdgcn_mfma_f32_16x16x32_f16(vbase[0], bpv[0], ocorr, 0, 0, 0);
    ocorr = __builtin_amdgcn_mfma_f32_16x16x32_f16(vbase[1], bpv[1], ocorr, 0, 0, 0);
    wave_lds_sync();
  };
  // Loads are unconditional (past-the-end windows read through the empty
  // view), so the compiler's waits name exactly the window needed next.
  KWin kbuf[MAXW];
  VWin vbuf[MAXW];
#pragma unroll
  for (int k = 0; k < kKeyAhead; ++k) fetch_keys(w_first + 4 * k, kbuf[k], k < n_full);
  float bc = 0.0f;
  if (n_full > 0) bc = fold(kbuf[0], 0);
  // once the key stream is fully requested, the value stream starts
#pragma unroll
  for (int k = 0; k < MAXW; ++k) {
    const int kn = k + kKeyAhead;
    if (kn < MAXW)
      fetch_keys(w_first + 4 * kn, kbuf[kn], kn < n_full);
    else if (kn - MAXW < kValAhead)
      fetch_values(w_first + 4 * (kn - MAXW), vbuf[kn - MAXW], kn - MAXW < n_mine);
    if (k < n_full) {
      wave_lds_sync();   // the fold of window k is in query buffer k & 1
      float bc_next = 0.0f;
      window_logits(kbuf[k], k & 1, bc, k, [&]() {
        if (k + 1 < MAXW && k + 1 < n_full) bc_next = fold(kbuf[k + 1 < MAXW ? k + 1 : k], (k + 1) & 1);
      });
      bc = bc_next;
    }
  }
  // lane c16 < 4 of each row holds head c16: reduce across the four rows
  mx = fmaxf(mx, lane_xor<16>(mx));
  mx = fmaxf(mx, lane_xor<32>(mx));
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    M[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), hh));
  // the unfinished window: bf16 keys from the tail, plain fp32 dot products
  if (n_mine > n_full) {
    const int wt = w_first + 4 * n_full;
    const int t = wt * kWindow + lane;
    float lg[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) lg[hh] = -__builtin_inff();
    if (t < t_end) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) lg[hh] = 0.0f;
      const uint16_t* kt = a.ktail + (bh * kWindow + lane) * D;
#pragma unroll 4
      for (int v = 0; v < D / 8; ++v) {
        float x[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(kt + v * 8), x);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int hh = 0; hh < G; ++hh) lg[hh] = __builtin_fmaf(qs[v * 8 + u][hh], x[u], lg[hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      sl[wave][n_full][hh][lane] = lg[hh];
      M[hh] = fmaxf(M[hh], wave_max(lg[hh]));
    }
  }
  wave_lds_sync();

#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    l_lane[hh] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) pz[hh][q] = 0.0f;
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  ocorr = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < MAXW; ++k) {
    const int kn = k + kValAhead;
    if (kn < MAXW) fetch_values(w_first + 4 * kn, vbuf[kn], kn < n_mine);
    if (k < n_mine) window_pv(vbuf[k], k);
  }
  float m_ref[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) m_ref[hh] = n_mine > 0 ? M[hh] : -__builtin_inff();

  // ---- wave partial: lane (col n = 4 q + head, g) keeps channels of group q
  {
    const int hh = c16 & 3, q = c16 >> 2;
    // zq = sum over the wave of pz[hh][q]; row r of ls holds sum l_lane[r]
    float zv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) zv[j] = pz[j & 3][j >> 2];
    const float zq = wave_sum16_at(zv, c16);
    const float ls = wave_sum4(l_lane);
    float lsum[G];
#pragma unroll
    for (int x = 0; x < G; ++x)
      lsum[x] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), 16 * x));
    // this lane's tiles are 2q and 2q + 1 (the channels of its group)
    f4 oa = o[0], ob = o[1];
#pragma unroll
    for (int qq = 1; qq < 4; ++qq)
      if (q == qq) {
        oa = o[2 * qq];
        ob = o[2 * qq + 1];
      }
    const f4 cz = ocorr - zq;
    float* wo = &sl[wave][0][0][0] + hh * D + 32 * q + 4 * g;
    *reinterpret_cast<f4*>(wo) = oa - cz;
    *reinterpret_cast<f4*>(wo + 16) = ob - cz;
    if (lane < G) {
      wm[wave][lane] = m_ref[lane];
      wlv[wave][lane] = lsum[lane];
    }
  }
  __syncthreads();
  for (int e = tid; e < G * (D + 2); e += 256) {
    const int hh = e / (D + 2), c = e % (D + 2);
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][hh]);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (wm[w][hh] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(wm[w][hh] - M);
      const float v = (c < D) ? (&sl[w][0][0][0])[hh * D + c] : wlv[w][hh];
      acc = __builtin_fmaf(f, v, acc);
    }
    float* dst = a.ws + (((int64_t)s * gridDim.z + b) * a.Hq + hq0 + hh) * (D + 2);
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
  // Splits are merged in chunks of 16: every load of a chunk is issued
  // before any is used (one memory round trip per chunk), and the running
  // (M, L, acc) is rescaled once per chunk.
  float M = -__builtin_inff(), L = 0.0f, acc = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 16) {
    float mv[16], lv[16], pv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int s = s0 + k;
      mv[k] = -__builtin_inff();
      lv[k] = 0.0f;
      pv[k] = 0.0f;
      if (s < S) {
        const float* p = ws + ((int64_t)s * BHq + r) * (D + 2);
        mv[k] = p[D];
        lv[k] = p[D + 1];
        if (c < D) pv[k] = p[c];
      }
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < 16; ++k) Mn = fmaxf(Mn, mv[k]);
    if (Mn == -__builtin_inff()) continue;
    const float sc = (M == -__builtin_inff()) ? 0.0f : exp2f(M - Mn);
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float f = (mv[k] == -__builtin_inff()) ? 0.0f : exp2f(mv[k] - Mn);
      L = __builtin_fmaf(f, lv[k], L);
      acc = __builtin_fmaf(f, pv[k], acc);
    }
    M = Mn;
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
  if (a.vmodal) decode_partial_kernel<D, G, KM, R, true><<<grid, 256, 0, st>>>(a);
  else decode_partial_kernel<D, G, KM, R, false><<<grid, 256, 0, st>>>(a);
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
  if (D == 128 && G == 4 && key_mode == KVQ_KEY_WINDOW && !a.vmodal) {
    const dim3 grid((unsigned)a.S, (unsigned)a.H, (unsigned)B);
    decode_mfma_kernel<<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  switch (G) {
    case 1: return launch_partial_mode<D, 1>(a, key_mode, R, B, st);
    case 2: return launch_partial_mode<D, 2>(a, key_mode, R, B, st);
    case 4: return launch_partial_mode<D, 4>(a, key_mode, R, B, st);
    default: return launch_partial_mode<D, 8>(a, key_mode, R, B, st);
  }
}

}  // namespace

// Splits per (sequence, kv head).  A split covers at most
// kDecodeMaxWindows windows.  Each block costs its windows plus a fixed
// overhead (pipeline fill and drain, the 4-wave merge, its share of the
// split merge) worth about kBlockOverheadWindows windows, and blocks beyond
// the device's resident slots queue behind the others: cost = max(1, blocks
// / slots) x (windows per split + kBlockOverheadWindows).  On the LLM decode
// workload (16 x 8 heads x 512 windows) decode time against the split count
// follows that cost with an overhead of 16 to 18 windows (16 splits: 80 us,
// 18: 86 us, 24: 93 us, 32: 107 us, 64: 167 us), so long splits win once the
// device is full and more splits only help while it is not.
int decode_splits(const kvq_layout* L, int q_heads, int n_tokens) {
  (void)q_heads;
  const int n_win = (n_tokens + kWindow - 1) / kWindow;
  if (n_win <= 0) return 1;
  const int64_t units = (int64_t)L->batch * L->kv_heads;
  const int cus = device_cus();
  const int64_t slots = (int64_t)cus * kDecodeBlocksPerCU;
  const int s_min = (n_win + kDecodeMaxWindows - 1) / kDecodeMaxWindows;
  const int s_max = n_win < s_min * 16 ? n_win : s_min * 16;
  int best = s_min;
  double best_cost = 1e300;
  for (int S = s_min; S <= s_max; ++S) {
    const int per = (n_win + S - 1) / S;
    if ((n_win + per - 1) / per != S) continue;     // same partition as a smaller S
    const double fill = (double)(units * S) / (double)slots;
    const double cost = (fill > 1.0 ? fill : 1.0) * (per + kBlockOverheadWindows);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

// The split partials of attn_int2_decode_noalloc: a fixed device array,
// one copy per device, kept until the process ends.  Its host-side name is
// not a device address; the address on each device comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) float scratch[KVQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
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
  const bool had = L.value_mode != KVQ_VAL_GROUP;
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
