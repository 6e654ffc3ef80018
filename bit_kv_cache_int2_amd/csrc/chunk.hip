// Chunk attention: a block of query rows (e.g. the frames being generated)
// against the packed INT2 cache, on the MFMA units.
//
// Block = 8 waves x 32 query rows (256 rows) of one (sequence, query head)
// and one range of cached tokens.  The cached tokens stream through in
// 64-token tiles.  Each thread loads one packed key word and one packed
// value word of the next tile while the current tile is being multiplied;
// the tile's parameters go through LDS, and every thread then dequantises
// its 16 keys and 16 values straight from its registers into fp16 LDS
// tiles (keys row-major; values transposed, tokens in the order the PV
// operand reads them).  A 2-bit code enters the arithmetic as the exact
// fp16 value base + code (the code-operand encoding of code_operand.h), so
// a dequantised element is one fma: (base + code) * s + (z - base s).
//   S^T = Khat Q^T  (A = key tile from LDS, B = the wave's queries, kept in
//                    registers for the whole loop),
//   O^T += Vhat^T P^T (A = transposed value tile, B = P straight from the
//                    score registers: the token order inside each 32-token
//                    k-step is permuted so that every lane already holds
//                    the eight P values it must supply),
//   l   += 1^T P^T   (one more MFMA against an all-ones operand row gives
//                    the softmax denominators from the same fp16 P).
// Probabilities are 2^(s * scale log2 e - m) with the hardware exp2, where
// m is a per-row reference maximum that is raised (and O, l rescaled) only
// when a probability relative to it would exceed 2^8; each lane tests its
// own scores, and the two cross-lane steps of a row maximum are taken only
// when some row of the wave moves.
// Precision: fp16 operands with fp32 accumulation; window-range keys
// (whose per-channel scales make logits large) are split as Khat = hi + lo,
// both fp16, and multiplied twice; centroid keys use one fp16 copy.  PSAC
// ([QWM] 2) adds (U^T q) . a as one more MFMA k-step (k 0..7).  Rotated
// values ([OKV]) are rotated back in registers at the end.
// When the row blocks alone would not fill the device, the cached tokens
// are split over blocks and a merge kernel combines the partial (o, m, l).
#include <type_traits>

#include "code_operand.h"
#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
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
  const uint16_t* q;
  void* out;
  float* lse;
  float* ws;          // split partials [S][B][Lq][Hq][D + 2] when S > 1
  int H, Hq, Tcap, C, n_tokens, Lq, out_bf16, S, tiles_per_split, n_rb, psac_int8;
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

template <int D, int KM, bool HAD, int R>
__global__ __launch_bounds__(kThreads) void chunk_kernel(const ChunkArgs a) {
  constexpr int NKS = D / 32;        // QK k-steps
  constexpr int NDT = D / 16;        // PV output dim tiles
  // KM: 0 window keys, 1 centroid keys as one fp16 copy, 2 centroid keys
  // split hi + lo like window keys
  constexpr bool LO = (KM != 1);     // hi/lo split keys
  // Tile pitches of 2 (mod 4) 16-byte units let the sixteen rows one operand
  // read touches fall on distinct banks; odd key rows and every other pair
  // of value rows swap neighbouring 16-byte units, which spreads the tile
  // stores over all banks as well.
  constexpr int KP = D + 16;         // key tile pitch (halfs)
  constexpr int VP = 64 + 16;        // value tile pitch (halfs)
  constexpr int NG = D / kGroup;     // parameter groups per row
  constexpr int KW = D / 16;         // key code words (16 channels) per token
  constexpr int NKT = 64 * KW;       // key words per tile
  constexpr int NVT = D * 4;         // value words per tile (16 tokens each)
  __shared__ __align__(16) _Float16 khi[64 * KP];
  __shared__ __align__(16) _Float16 klo[LO ? 64 * KP : 8];
  __shared__ __align__(16) _Float16 vt[D * VP];
  __shared__ __align__(16) _Float16 coef[R > 0 ? 64 * 16 : 8];
  // parameters, two sets: tile j's in set j & 1, stored one tile ahead
  __shared__ __align__(16) uint32_t kpar[2][KM == 0 ? D : 64 * NG];   // window: per channel; else per token group
  __shared__ __align__(16) uint32_t vpar[2][NG][64];                   // [group][token]

  const int rb = blockIdx.x % a.n_rb, split = blockIdx.x / a.n_rb;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.H, h = hq / G;
  const int64_t bh = (int64_t)b * a.H + h;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int row0 = rb * kBM + wave * kNT * 16;
  const bool live = row0 < a.Lq;   // wave-uniform
  const int n = a.n_tokens;
  const int n_tiles = (n + 63) / 64, n_full = n / 64;
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, n_tiles);

  CodeOr kor = {0x54005400u, 0x4C004C00u, 0x44004400u};
  asm volatile("" : "+v"(kor.b64), "+v"(kor.b16), "+v"(kor.b4));

  // ---- queries (B operand), fp16 (exact from bf16), resident for the whole loop
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
        for (int j = 0; j < 8; ++j) v[j] = (_Float16)x[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (_Float16)0.0f;
      }
      qreg[nt][ks] = v;
    }
  }
  // ---- PSAC: q' = U^T q, the B operand of one more 16x16x32 k-step: lanes
  // g == 0 supply q'[0 .. R-1] of their row, every other k is zero
  static_assert(R == 0 || R == 8, "PSAC rank 8 fills k 0..7 of one k-step");
  h8 qp[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
    for (int j = 0; j < 8; ++j) qp[nt][j] = (_Float16)0.0f;
    if (R > 0) {
      const int row = row0 + nt * 16 + c16;
      if (g == 0 && row < a.Lq) {
        const uint16_t* qr = a.q + (((int64_t)b * a.Lq + row) * a.Hq + hq) * D;
        const float* U = a.basis + bh * D * (R > 0 ? R : 1);
        float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        for (int d = 0; d < D; ++d) {
          const float qd = bf16_to_f32(qr[d]);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(U[d * R + j], qd, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) qp[nt][j] = (_Float16)acc[j];
      }
    }
  }

  // m_run: reference maximum (log2 units); thr: the raw score above which it
  // moves, (m_run + kLazyLog2) / scale_log2
  float m_run[kNT], thr[kNT];
  const float inv_scale_log2 = 1.0f / a.scale_log2;
  f4 o[kNT][NDT], ol[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    m_run[nt] = -__builtin_inff();
    thr[nt] = -__builtin_inff();
    ol[nt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[nt][dt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // all-ones operand row (row 0 of the 16-row A tile)
  h8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (_Float16)(c16 == 0 ? 1.0f : 0.0f);

  // ---- per-thread share of a tile: key word = token tk, channels
  // 16 kw .. 16 kw + 15 (each group of eight lanes holds two tokens);
  // value word = channel vc, tokens 16 vq .. 16 vq + 15
  const int tk = KW == 8 ? 2 * (tid >> 4) + ((tid >> 2) & 1) : tid / KW;
  const int kw = KW == 8 ? (tid & 3) + 4 * ((tid >> 3) & 1) : tid % KW;
  const int vc = tid >> 2, vq = tid & 3;
  const bool has_k = tid < NKT, has_v = tid < NVT;
  struct Pre {
    uint32_t kcw, vcw, kp, vp, cf, cs;   // cf/cs: PSAC words (INT8: two codes, scale)
    int ix;            // centroid index of token tk
    float cv[16];      // centroid channels 16 kw .. 16 kw + 15 of token tk
  };
  auto prefetch = [&](int tile, Pre& f) {
    const int t0 = tile * 64;
    const int64_t rowbase = bh * a.Tcap + t0;
    f.kcw = has_k ? reinterpret_cast<const uint32_t*>(a.kcodes + rowbase * (D / 4))[tk * KW + kw] : 0u;
    f.vcw = has_v ? reinterpret_cast<const uint32_t*>(
                        a.vcodes + (bh * (a.Tcap / 64) + tile) * (int64_t)D * 16)[tid]
                  : 0u;
    // value parameters [token][group], zero past the end
    f.vp = (tid < 64 * NG && t0 + tid / NG < n) ? a.vparams[rowbase * NG + tid] : 0u;
    if (KM == 0) {
      f.kp = (tid < D && tile < n_full) ? a.kparams[(bh * (a.Tcap / 64) + tile) * D + tid] : 0u;
    } else {
      f.kp = (tid < 64 * NG) ? a.kparams[rowbase * NG + tid] : 0u;
      // rows past the length hold no index: they read centroid 0
      f.ix = (has_k && t0 + tk < n) ? (int)a.kidx[rowbase + tk] : 0;
    }
    f.cf = 0u;
    f.cs = 0u;
    if (R > 0 && tid < 64 * 8) {   // PSAC coefficients: two per thread
      const int t = tid >> 3, m2 = (tid & 7) * 2;
      if (m2 < R && t0 + t < n) {
        if (a.psac_int8) {
          f.cf = reinterpret_cast<const uint16_t*>(
              reinterpret_cast<const uint8_t*>(a.kpsac) + (rowbase + t) * R)[m2 / 2];
          f.cs = a.kpsac_sc[rowbase + t];
        } else {
          f.cf = reinterpret_cast<const uint32_t*>(a.kpsac + (rowbase + t) * R)[m2 / 2];
        }
      }
    }
  };
  // centroid rows need the index, so they are requested one step later
  auto prefetch_cent = [&](Pre& f) {
    if (KM != 0 && has_k) {
      const float* cr = a.cent + (bh * a.C + f.ix) * D + 16 * kw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 c4 = *reinterpret_cast<const float4*>(cr + 4 * j);
        f.cv[4 * j] = c4.x;
        f.cv[4 * j + 1] = c4.y;
        f.cv[4 * j + 2] = c4.z;
        f.cv[4 * j + 3] = c4.w;
      }
    }
  };

  auto store_params = [&](int tile, const Pre& f) {
    const int ps = tile & 1;
    if (tid < 64 * NG) vpar[ps][tid % NG][tid / NG] = f.vp;
    if (KM == 0) {
      if (tid < D) kpar[ps][tid] = f.kp;
    } else {
      if (tid < 64 * NG) kpar[ps][tid] = f.kp;
    }
  };
  Pre pre;
  if (tile_begin < tile_end) {
    prefetch(tile_begin, pre);
    prefetch_cent(pre);
    store_params(tile_begin, pre);
  }

  // One 64-token tile; the ragged last tile (masking, key tail) is a
  // separate instantiation so that full tiles carry no masking code.
  auto tile_step = [&](int tile, auto ragged) {
    const int t0 = tile * 64;
    constexpr bool last = decltype(ragged)::value;    // the ragged last tile
    const bool full_keys = KM != 0 || !last;          // window keys: tail window
    // the previous tile's LDS tiles are consumed and this tile's parameters
    // (stored during the previous tile) are visible
    __syncthreads();
    const int ps = tile & 1;
    if (R > 0 && tid < 64 * 8) {
      uint32_t cw = pre.cf;
      if (a.psac_int8) {   // two INT8 codes times the token's scale, to fp16
        const float sc = f16_bits_to_f32(pre.cs);
        cw = pk_rne((float)(int8_t)(pre.cf & 0xFFu) * sc, (float)(int8_t)(pre.cf >> 8) * sc);
      }
      reinterpret_cast<uint32_t*>(coef)[(tid >> 3) * 8 + (tid & 7)] = cw;
    }
    const uint32_t kcw = pre.kcw, vcw = pre.vcw;
    float cv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) cv[c] = pre.cv[c];
    // ---- the next tile's packed data is in flight during this tile
    if (tile + 1 < tile_end) prefetch(tile + 1, pre);

    // ---- dequantise keys: token tk, channels 16 kw .. 16 kw + 15
    if (has_k) {
      float kv[16];
      if (full_keys) {
        uint32_t cw[8];
        code_word(kcw, kor, cw);
        if (KM == 0) {
          uint4 pw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) pw[j] = *reinterpret_cast<const uint4*>(&kpar[ps][16 * kw + 4 * j]);
          const uint32_t pv[16] = {pw[0].x, pw[0].y, pw[0].z, pw[0].w, pw[1].x, pw[1].y, pw[1].z, pw[1].w,
                                   pw[2].x, pw[2].y, pw[2].z, pw[2].w, pw[3].x, pw[3].y, pw[3].z, pw[3].w};
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const float s = f16_bits_to_f32(pv[c]), z = f16_bits_to_f32(pv[c] >> 16);
            kv[c] = fma_code(cw[c & 7], c >= 8, s, __builtin_fmaf(-code_base(c & 7), s, z));
          }
        } else {
          const uint32_t pw = kpar[ps][tk * NG + kw / 2];
          const float s = f16_bits_to_f32(pw), z = f16_bits_to_f32(pw >> 16);
          const float z16 = __builtin_fmaf(-16.0f, s, z), z4 = __builtin_fmaf(-4.0f, s, z),
                      z64 = __builtin_fmaf(-64.0f, s, z);
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const int i = c & 7;
            const float zb = (i == 2 || i == 5) ? z64 : ((i == 1 || i == 4 || i == 7) ? z4 : z16);
            // centroid + residual (the residual rounded to fp32 first)
            kv[c] = cv[c] + fma_code(cw[i], c >= 8, s, zb);
          }
        }
      } else {
        // the unfinished window: bf16 keys from the tail
        const uint16_t* kt = a.ktail + (bh * 64 + tk) * D + 16 * kw;
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(kt), kv);
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(kt + 8), kv + 8);
      }
      if (last && t0 + tk >= n) {
#pragma unroll
        for (int c = 0; c < 16; ++c) kv[c] = 0.0f;
      }
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        hw[m] = pk_rne(kv[2 * m], kv[2 * m + 1]);
        if (LO) {
          const h2 hh = __builtin_bit_cast(h2, hw[m]);
          lw[m] = pk_rne(kv[2 * m] - (float)hh[0], kv[2 * m + 1] - (float)hh[1]);
        }
      }
      // 16-byte units 2 kw, 2 kw + 1 of row tk, swapped in odd rows
      const int o0 = tk * KP + 8 * ((2 * kw) ^ (tk & 1)), o1 = tk * KP + 8 * ((2 * kw + 1) ^ (tk & 1));
      *reinterpret_cast<uint4*>(&khi[o0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&khi[o1]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      if (LO) {
        *reinterpret_cast<uint4*>(&klo[o0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint4*>(&klo[o1]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      }
    }
    // the next tile's centroid rows (its indices were requested above)
    if (tile + 1 < tile_end) prefetch_cent(pre);
    // ---- dequantise values: channel vc, tokens 16 vq .. 16 vq + 15, written
    // in operand order: position 32 kk + 8 g' + j holds token
    // 32 kk + 4 g' + j (j < 4) or 32 kk + 16 + 4 g' + j - 4 (j >= 4)
    if (has_v) {
      uint32_t cw[8];
      code_word(vcw, kor, cw);
      const uint4* pr = reinterpret_cast<const uint4*>(&vpar[ps][vc / kGroup][16 * vq]);
      const uint4 p4[4] = {pr[0], pr[1], pr[2], pr[3]};
      const uint32_t pv[16] = {p4[0].x, p4[0].y, p4[0].z, p4[0].w, p4[1].x, p4[1].y, p4[1].z, p4[1].w,
                               p4[2].x, p4[2].y, p4[2].z, p4[2].w, p4[3].x, p4[3].y, p4[3].z, p4[3].w};
      float vv[16];   // token 16 vq + u
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = u & 7;
        const float s = f16_bits_to_f32(pv[u]), z = f16_bits_to_f32(pv[u] >> 16);
        vv[u] = fma_code(cw[i], u >= 8, s, __builtin_fmaf(-code_base(i), s, z));
      }
      // tokens 16 vq + 4 gg + j: k-step vq / 2, positions 8 gg + 4 (vq & 1) + j
      // (16-byte units swapped in pairs when bit 1 of the row is set)
      _Float16* dst = &vt[vc * VP + 32 * (vq >> 1) + 4 * (vq & 1)];
      const int vs = (vc >> 1) & 1;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *reinterpret_cast<uint2*>(dst + 8 * (gg ^ vs)) =
            make_uint2(pk_rne(vv[4 * gg], vv[4 * gg + 1]), pk_rne(vv[4 * gg + 2], vv[4 * gg + 3]));
    }
    // the next tile's parameters into the other set (its last reader, the
    // previous tile's dequantisation, finished before this tile began)
    if (tile + 1 < tile_end) store_params(tile + 1, pre);
    __syncthreads();
    if (!live) return;   // every row of this wave is past the end: dequantise only

    // ---- S^T = Khat Q^T
    f4 s[kNT][4];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int ts = 0; ts < 4; ++ts) s[nt][ts] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      if (R > 0) {
        // PSAC first: k 0..7 are token ts*16 + c16's coefficients (lanes
        // g == 1 read the zero half of the row, g >= 2 meet a zero q')
        const h8 ca = *reinterpret_cast<const h8*>(&coef[(ts * 16 + c16) * 16 + 8 * (g & 1)]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca, qp[nt], s[nt][ts], 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const h8 ka = *reinterpret_cast<const h8*>(&khi[(ts * 16 + c16) * KP + ks * 32 + 8 * (g ^ (c16 & 1))]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qreg[nt][ks], s[nt][ts], 0, 0, 0);
        if (LO) {
          const h8 kl = *reinterpret_cast<const h8*>(&klo[(ts * 16 + c16) * KP + ks * 32 + 8 * (g ^ (c16 & 1))]);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            s[nt][ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, qreg[nt][ks], s[nt][ts], 0, 0, 0);
        }
      }
    }

    // ---- online softmax (base 2); lane owns row nt*16 + c16, tokens ts*16 + 4g + i.
    // A row's reference maximum m (the same in the four lanes of the row)
    // moves only when a score passes it by more than kLazyLog2, so p stays at
    // most 2^kLazyLog2 (well inside fp16) and O, l are rescaled rarely.  The
    // test needs only the lane's own scores; the row maximum across lanes is
    // formed only when some row of the wave moves.
    float lm[kNT];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      if (last) {
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + ts * 16 + 4 * g + i >= n) s[nt][ts][i] = -__builtin_inff();
      }
      float m = -__builtin_inff();
#pragma unroll
      for (int ts = 0; ts < 4; ++ts)
        m = fmaxf(fmaxf(m, fmaxf(s[nt][ts][0], s[nt][ts][1])), fmaxf(s[nt][ts][2], s[nt][ts][3]));
      lm[nt] = m;
      grow |= m > thr[nt];
    }
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float m = lm[nt];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const float mn = fmaxf(m_run[nt], m * a.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - mn);   // 0 on the first tile
        m_run[nt] = mn;
        thr[nt] = (mn + kLazyLog2) * inv_scale_log2;
        ol[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[nt][dt] *= alpha;
      }
    }
    h8 pb[kNT][2];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      uint32_t pw[8];
#pragma unroll
      for (int ts = 0; ts < 4; ++ts)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nt][ts][i], a.scale_log2, -m_run[nt]));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nt][ts][i + 1], a.scale_log2, -m_run[nt]));
          pw[ts * 2 + i / 2] = pk_rne(p0, p1);
        }
      // k-step kk takes slabs 2 kk and 2 kk + 1
      pb[nt][0] = as_h8(pw[0], pw[1], pw[2], pw[3]);
      pb[nt][1] = as_h8(pw[4], pw[5], pw[6], pw[7]);
    }

    // ---- O^T += Vhat^T P^T, l += 1^T P^T
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const h8 va = *reinterpret_cast<const h8*>(&vt[(dt * 16 + c16) * VP + kk * 32 + 8 * (g ^ ((c16 >> 1) & 1))]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[nt][kk], o[nt][dt], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        ol[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[nt][kk], ol[nt], 0, 0, 0);
    }
  };
  const bool has_ragged = (n & 63) != 0 && tile_end == n_tiles && tile_begin < tile_end;
  const int tile_stop = has_ragged ? tile_end - 1 : tile_end;
  for (int tile = tile_begin; tile < tile_stop; ++tile) tile_step(tile, std::false_type{});
  if (has_ragged) tile_step(tile_end - 1, std::true_type{});

  // ---- epilogue: l of row c16 sits in lane c16 (row 0 of the ones tile)
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const float l = __shfl(ol[nt][0], c16, 64);
    const int row = row0 + nt * 16 + c16;
    if (a.S > 1) {
      // partial (o, m, l) for the merge
      if (row < a.Lq) {
        float* dst = a.ws + ((((int64_t)split * gridDim.z + b) * a.Lq + row) * a.Hq + hq) * (D + 2);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<float4*>(dst + dt * 16 + 4 * g) =
              make_float4(o[nt][dt][0], o[nt][dt][1], o[nt][dt][2], o[nt][dt][3]);
        if (g == 0) {
          dst[D] = m_run[nt];
          dst[D + 1] = l;
        }
      }
      continue;
    }
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

template <int D, int KM, bool HAD, int R>
hipError_t launch_t(const ChunkArgs& a, int B, hipStream_t st) {
  const dim3 grid((unsigned)(a.n_rb * a.S), (unsigned)a.Hq, (unsigned)B);
  chunk_kernel<D, KM, HAD, R><<<grid, kThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S == 1) return e;
  chunk_merge_kernel<D, HAD><<<(unsigned)((int64_t)B * a.Lq * a.Hq), D, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int KM>
hipError_t launch_c(const ChunkArgs& a, bool had, int R, int B, hipStream_t st) {
  if (R == 8)
    return had ? launch_t<D, KM, true, 8>(a, B, st) : launch_t<D, KM, false, 8>(a, B, st);
  return had ? launch_t<D, KM, true, 0>(a, B, st) : launch_t<D, KM, false, 0>(a, B, st);
}

template <int D>
hipError_t launch_d(const ChunkArgs& a, int key_mode, bool split, bool had, int R, int B,
                    hipStream_t st) {
  if (key_mode == KVQ_KEY_WINDOW)
    return had ? launch_t<D, 0, true, 0>(a, B, st) : launch_t<D, 0, false, 0>(a, B, st);
  return split ? launch_c<D, 2>(a, had, R, B, st) : launch_c<D, 1>(a, had, R, B, st);
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
  const bool had = L.value_mode == KVQ_VAL_HADAMARD;
  const bool split = L.centroid_key_split != 0;
  return (L.head_dim == 128) ? launch_d<128>(a, L.key_mode, split, had, R, L.batch, stream)
                             : launch_d<64>(a, L.key_mode, split, had, R, L.batch, stream);
}

}  // namespace kvq
