// Chunk attention: a block of query rows (e.g. the frames being generated)
// against the packed INT2 cache, on the MFMA units.
//
// Block = 8 waves x 32 query rows (256 rows) of one (sequence, query head)
// and one range of cached tokens, which stream through in 64-token tiles.
// Each thread dequantises 16 keys and 16 values of a tile straight from its
// registers into fp16 LDS tiles (keys row-major, values transposed with the
// tokens in the order the PV operand reads them).  A 2-bit code enters the
// arithmetic as the exact fp16 value base + code (code_operand.h), so a
// dequantised element is one fma.
//   S^T = Khat Q^T    A = key tile from LDS, B = the wave's queries (kept in
//                     registers for the whole loop);
//   O^T += Vc^T P^T   A = the centred value tile, B = P straight from the
//                     score registers (the token order inside each 32-token
//                     k-step is permuted so that every lane already holds
//                     the eight P values it supplies);
//   L   += M^T P^T    A = a 16-row tile of row sums: row 0 all ones (the
//                     softmax denominator), the next rows each value
//                     group's level-1 point mu = z + s per (token, group)
//                     as fp16 hi and lo parts (per modality for
//                     per-modality rotations), so sum_t p_t mu_t comes out
//                     exact to fp32.
// Precision: every key enters as fp16 hi + lo (Khat = hi + lo, both fp16,
// multiplied twice), exact to fp32 whatever the key range.  A value enters
// as (code - 1) s in {-s, 0, s, 2s}, exact in fp16, and z + s comes from
// the row sums above, so the values carry no rounding at all.  The PSAC
// term uses k 0..23 of its k-step as a_hi q'_hi + a_hi q'_lo + a_lo q'_hi.
// Probabilities are fp16 (their rounding multiplies v - o, not v).
// Softmax is base 2 with a lazy reference maximum: a row's m moves only
// when a score passes it by more than 2^8; each lane tests its own scores,
// and the cross-lane row maximum and the rescale run in a wave-uniform
// branch that is rarely taken.
// PSAC ([QWM] 2) adds (U^T q) . a as one more MFMA k-step.
// Rotated values ([OKV]) are rotated back in registers at the end; with
// per-modality rotations each value takes its modality's signs first.
//
// Software pipeline, one barrier per tile: while a wave multiplies QK of
// tile j it dequantises its share of tile j + 1 into the other key buffer
// and the next of three value buffers, and while it multiplies PV of tile
// j - 1 it forms P of tile j; packed codes and parameters are requested
// two tiles ahead.  A ragged last tile runs unpipelined after the others.
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

// Position of tile token t (0..63) in the PV operand's k order: k-step
// t / 32; inside it, lane group g' supplies tokens 4g' .. 4g'+3 and
// 16 + 4g' .. 16 + 4g'+3 at positions 8g' .. 8g'+7.
KVQ_DEV int pv_pos(int t) {
  const int r = t & 31;
  return (t & 32) + 8 * ((r & 15) >> 2) + (r & 3) + ((r & 16) ? 4 : 0);
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
  constexpr int KBUF = 64 * KP;
  constexpr int VBUF = D * VP;
  constexpr int MBUF = NMU * 16 * VP;
  __shared__ __align__(16) _Float16 khi[2 * KBUF];
  __shared__ __align__(16) _Float16 klo[2 * KBUF];
  __shared__ __align__(16) _Float16 vt[3 * VBUF];
  __shared__ __align__(16) _Float16 mut[3 * MBUF];
  // PSAC operand rows, 32 halves per token: a_hi, a_hi, a_lo, 0 (8 each);
  // 16-byte units swizzled by bits 2-3 of the token so the 16 rows an
  // operand read touches spread over the banks
  __shared__ __align__(16) _Float16 coef[R > 0 ? 2 * 64 * 32 : 8];
  // parameters, two sets: tile t's in set t & 1, stored two tiles ahead
  __shared__ __align__(16) uint32_t kpar[2][KM == 0 ? D : 64 * NG];   // window: per channel; else per token group
  __shared__ __align__(16) uint32_t vpar[2][NG][64];                   // [group][token]
  __shared__ __align__(16) uint32_t vmod[2][VM == 2 ? 16 : 1];         // modality bytes of the tile

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
  const bool has_ragged = (n & 63) != 0 && tile_end == n_tiles && tile_begin < tile_end;
  const int full_end = has_ragged ? tile_end - 1 : tile_end;   // tiles [tile_begin, full_end) are full
  const int M = a.M;

  CodeOr kor = {0x54005400u, 0x4C004C00u, 0x44004400u};
  asm volatile("" : "+v"(kor.b64), "+v"(kor.b16), "+v"(kor.b4));

  // ---- LDS set-up: value and row-sum buffers zero (the first PV step
  // multiplies a zero P by buffer 2), row 0 of every row-sum tile all ones
  {
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (int e = tid; e < 3 * VBUF / 8; e += kThreads) reinterpret_cast<uint4*>(vt)[e] = z4;
    for (int e = tid; e < 3 * MBUF / 8; e += kThreads) reinterpret_cast<uint4*>(mut)[e] = z4;
    __syncthreads();
    if (tid < 3 * NMU * 64) {
      const int buf = tid / (NMU * 64), rest = tid % (NMU * 64), tile16 = rest / 64, t = rest % 64;
      if (tile16 == 0) mut[buf * MBUF + pv_pos(t)] = (_Float16)1.0f;   // row 0 swizzle: none
    }
  }

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
  // g = 0, 1, 2 supply q'_hi, q'_lo, q'_hi of their row (k 0..23), g = 3 zero
  static_assert(R == 0 || R == 8, "PSAC rank 8 fills k 0..23 of one k-step");
  h8 qp[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
    for (int j = 0; j < 8; ++j) qp[nt][j] = (_Float16)0.0f;
    if (R > 0) {
      const int row = row0 + nt * 16 + c16;
      if (g < 3 && row < a.Lq) {
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
          qp[nt][j] = (g == 1) ? (_Float16)(acc[j] - (float)hi) : hi;
        }
      }
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
    uint32_t kcw, vcw, kp, vp, cf, cs, md;   // cf/cs: PSAC words (INT8: two codes, scale)
    int ix;            // centroid index of token tk
    float cv[16];      // centroid channels 16 kw .. 16 kw + 15 of token tk
  };
  // packed data of a tile into registers.  RAG (the ragged last tile):
  // parameters and indices of rows past the length read as 0, so they
  // dequantise to finite values; full tiles load unconditionally.
  auto prefetch = [&](int tile, Pre& f, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    const int t0 = tile * 64;
    const int64_t rowbase = bh * a.Tcap + t0;
    const int pi = tid % (64 * NG);   // (token, group) parameter word
    f.kcw = has_k ? reinterpret_cast<const uint32_t*>(a.kcodes + rowbase * (D / 4))[tk * KW + kw] : 0u;
    f.vcw = has_v ? reinterpret_cast<const uint32_t*>(
                        a.vcodes + (bh * (a.Tcap / 64) + tile) * (int64_t)D * 16)[tid]
                  : 0u;
    f.vp = a.vparams[rowbase * NG + pi];
    if (RAG && t0 + pi / NG >= n) f.vp = 0u;
    if (KM == 0) {
      f.kp = (RAG && tile >= n_full) ? 0u : a.kparams[(bh * (a.Tcap / 64) + tile) * D + tid % D];
    } else {
      f.kp = a.kparams[rowbase * NG + pi];
      f.ix = has_k ? (int)a.kidx[rowbase + tk] : 0;
      if (RAG && t0 + pi / NG >= n) f.kp = 0u;
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
    f.md = 0u;
    if (VM == 2 && tid < 16)
      f.md = reinterpret_cast<const uint32_t*>(a.vmodal + (int64_t)b * a.Tcap + t0)[tid];
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
    vpar[ps][gm][tm] = f.vp;
    if (KM == 0) kpar[ps][tid % D] = f.kp;
    else kpar[ps][tid % (64 * NG)] = f.kp;
    if (VM == 2 && tid < 16) vmod[ps][tid] = f.md;
  };

  // Registers of the tile being dequantised (taken from Pre before the
  // next tile's loads are issued into it).
  struct Cur {
    uint32_t kcw, vcw, cf, cs;
    float cv[16];
  };
  auto take = [&](const Pre& f, Cur& c) {
    c.kcw = f.kcw;
    c.vcw = f.vcw;
    c.cf = f.cf;
    c.cs = f.cs;
#pragma unroll
    for (int i = 0; i < 16; ++i) c.cv[i] = KM != 0 ? f.cv[i] : 0.0f;
  };

  // ---- dequantise tile `tile` into key buffer kb, value / row-sum buffer
  // vbuf, coefficient buffer kb.  RAG: the ragged last tile (window keys of
  // the unfinished window come from the tail; keys past the length are 0).
  auto dequant = [&](int tile, const Cur& c, int kb, int vbuf, auto rag) {
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
    // keys: token tk, channels 16 kw .. 16 kw + 15, as hi + lo
    if (has_k) {
      float kv[16];
      const bool tail = RAG && KM == 0;   // the unfinished window
      if (!tail) {
        uint32_t cw[8];
        code_word(c.kcw, kor, cw);
        if (KM == 0) {
          uint4 pw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) pw[j] = *reinterpret_cast<const uint4*>(&kpar[ps][16 * kw + 4 * j]);
          const uint32_t pv[16] = {pw[0].x, pw[0].y, pw[0].z, pw[0].w, pw[1].x, pw[1].y, pw[1].z, pw[1].w,
                                   pw[2].x, pw[2].y, pw[2].z, pw[2].w, pw[3].x, pw[3].y, pw[3].z, pw[3].w};
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float s = f16_bits_to_f32(pv[i]), z = f16_bits_to_f32(pv[i] >> 16);
            kv[i] = fma_code(cw[i & 7], i >= 8, s, __builtin_fmaf(-code_base(i & 7), s, z));
          }
        } else {
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
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        hw[m] = pk_rne(kv[2 * m], kv[2 * m + 1]);
        const h2 hh = __builtin_bit_cast(h2, hw[m]);
        lw[m] = pk_rne(kv[2 * m] - (float)hh[0], kv[2 * m + 1] - (float)hh[1]);
      }
      // 16-byte units 2 kw, 2 kw + 1 of row tk, swapped in odd rows
      const int o0 = kb * KBUF + tk * KP + 8 * ((2 * kw) ^ (tk & 1));
      const int o1 = kb * KBUF + tk * KP + 8 * ((2 * kw + 1) ^ (tk & 1));
      *reinterpret_cast<uint4*>(&khi[o0]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&khi[o1]) = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      *reinterpret_cast<uint4*>(&klo[o0]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      *reinterpret_cast<uint4*>(&klo[o1]) = make_uint4(lw[4], lw[5], lw[6], lw[7]);
    }
    // values: channel vc, tokens 16 vq .. 16 vq + 15, centred on level 1,
    // (code - 1) s = (base + code) s - (base + 1) s, exact in fp32 and fp16,
    // written in operand order: position 32 kk + 8 g' + j holds token
    // 32 kk + 4 g' + j (j < 4) or 32 kk + 16 + 4 g' + j - 4 (j >= 4)
    if (has_v) {
      uint32_t cw[8];
      code_word(c.vcw, kor, cw);
      const uint4* pr = reinterpret_cast<const uint4*>(&vpar[ps][vc / kGroup][16 * vq]);
      const uint4 p4[4] = {pr[0], pr[1], pr[2], pr[3]};
      const uint32_t pv[16] = {p4[0].x, p4[0].y, p4[0].z, p4[0].w, p4[1].x, p4[1].y, p4[1].z, p4[1].w,
                               p4[2].x, p4[2].y, p4[2].z, p4[2].w, p4[3].x, p4[3].y, p4[3].z, p4[3].w};
      float vv[16];   // token 16 vq + u
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int p = u & 7;
        const float s = f16_bits_to_f32(pv[u]);
        vv[u] = fma_code(cw[p], u >= 8, s, -(code_base(p) + 1.0f) * s);
      }
      uint32_t pk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pk[j] = pk_rne(vv[2 * j], vv[2 * j + 1]);
      if (VM == 2) {
        // sign of (token, channel vc): bit m(t) of vsgn; negate those halves
        const uint32_t* mw = &vmod[ps][4 * vq];
        uint32_t neg = 0u;   // bit u: token 16 vq + u negated
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const uint32_t mb = mw[w4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t m = min((mb >> (8 * k)) & 0xFFu, (uint32_t)(M - 1));
            neg |= ((vsgn >> m) & 1u) << (4 * w4 + k);
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pk[j] ^= (((neg >> (2 * j)) & 1u) << 15) | (((neg >> (2 * j + 1)) & 1u) << 31);
      }
      // tokens 16 vq + 4 gg + j: k-step vq / 2, positions 8 gg + 4 (vq & 1) + j
      // (16-byte units swapped in pairs when bit 1 of the row is set)
      _Float16* dst = &vt[vbuf * VBUF + vc * VP + 32 * (vq >> 1) + 4 * (vq & 1)];
      const int vs = (vc >> 1) & 1;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *reinterpret_cast<uint2*>(dst + 8 * (gg ^ vs)) = make_uint2(pk[2 * gg], pk[2 * gg + 1]);
    }
    // row sums: level 1, z + s, of (token tm, group gm) as fp16 hi and lo,
    // in the rows of the token's modality (zero in the others)
    {
      const uint32_t pw = vpar[ps][gm][tm];
      const float s = f16_bits_to_f32(pw), z = f16_bits_to_f32(pw >> 16);
      const float mu = z + s;
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

  // ---- S^T = Khat Q^T for tokens 32 half .. 32 half + 31 of key buffer kb
  // (hi and lo, PSAC k-step first); s[nt][t] holds token slab 2 half + t
  auto qk = [&](int kb, int half, f4 (&s)[kNT][2]) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[nt][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    const _Float16* kh = khi + kb * KBUF;
    const _Float16* kl = klo + kb * KBUF;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ts = 2 * half + t;
      if (R > 0) {
        // PSAC first: row ts*16 + c16 of the coefficient tile (k 0..23)
        const int cr = ts * 16 + c16;
        const h8 ca = *reinterpret_cast<const h8*>(&coef[kb * 64 * 32 + cr * 32 + 8 * (g ^ ((cr >> 2) & 3))]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ca, qp[nt], s[nt][t], 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int off = (ts * 16 + c16) * KP + ks * 32 + 8 * (g ^ (c16 & 1));
        const h8 ka = *reinterpret_cast<const h8*>(&kh[off]);
        const h8 kl2 = *reinterpret_cast<const h8*>(&kl[off]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          s[nt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qreg[nt][ks], s[nt][t], 0, 0, 0);
          s[nt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl2, qreg[nt][ks], s[nt][t], 0, 0, 0);
        }
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

  // ---- online softmax (base 2) of one half tile's scores into P (fp16);
  // lane owns row nt*16 + c16, tokens 32 half + 16 t + 4g + i.  row_max
  // returns whether some row's reference maximum must move (then `grow`).
  auto row_max = [&](const f4 (&s)[kNT][2], float (&lm)[kNT]) {
    bool gr = false;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      float m = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 2; ++t)
        m = fmaxf(fmaxf(m, fmaxf(s[nt][t][0], s[nt][t][1])), fmaxf(s[nt][t][2], s[nt][t][3]));
      lm[nt] = m;
      gr |= m > thr[nt];
    }
    return gr;
  };
  auto grow = [&](const float (&lm)[kNT]) {
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
  // P of a half tile: the B operand of PV k-step `half` (slabs 2 half, 2 half + 1)
  auto probs = [&](const f4 (&s)[kNT][2], h8 (&pb)[kNT]) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      uint32_t pw[4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nt][t][i], a.scale_log2, -m_run[nt]));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nt][t][i + 1], a.scale_log2, -m_run[nt]));
          pw[t * 2 + i / 2] = pk_rne(p0, p1);
        }
      pb[nt] = as_h8(pw[0], pw[1], pw[2], pw[3]);
    }
  };
  // masks the scores of tokens at or past the length (ragged last tile)
  auto mask = [&](int t0, int half, f4 (&s)[kNT][2]) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 32 * half + 16 * t + 4 * g + i >= n) s[nt][t][i] = -__builtin_inff();
  };
  // QK and P of tile buffer kb: the second half's MFMAs run while the first
  // half's probabilities are formed; a rare move of the reference maximum
  // in the second half re-forms the first half's.
  auto qk_softmax = [&](int kb, h8 (&pb)[kNT][2], int t0, auto rag) {
    constexpr bool RAG = decltype(rag)::value;
    f4 sa[kNT][2], sb[kNT][2];
    float lm[kNT];
    qk(kb, 0, sa);
    if (RAG) mask(t0, 0, sa);
    if (__any(row_max(sa, lm))) grow(lm);
    h8 pa[kNT];
    qk(kb, 1, sb);
    probs(sa, pa);
    if (RAG) mask(t0, 1, sb);
    if (__any(row_max(sb, lm))) {
      grow(lm);
      probs(sa, pa);
    }
    h8 pc[kNT];
    probs(sb, pc);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      pb[nt][0] = pa[nt];
      pb[nt][1] = pc[nt];
    }
  };

  // P of the previous tile (zero before the first: its PV step adds nothing)
  h8 pprev[kNT][2];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) pprev[nt][kk][j] = (_Float16)0.0f;

  Pre pre;
  Cur cur;
  const int nfull = full_end - tile_begin;
  if (nfull > 0) {
    // ---- prologue: tile 0 of the split dequantised, tile 1's parameters stored
    prefetch(tile_begin, pre, std::false_type{});
    prefetch_cent(pre);
    store_params(tile_begin, pre);
    __syncthreads();
    take(pre, cur);
    if (nfull > 1) prefetch(tile_begin + 1, pre, std::false_type{});
    dequant(tile_begin, cur, 0, 0, std::false_type{});
    if (nfull > 1) {
      prefetch_cent(pre);
      store_params(tile_begin + 1, pre);
    }
  }

  // ---- one pipelined step: PV of tile j - 1 with the dequantisation of
  // tile j + 1, then QK and P of tile j.  DQ: tile j + 1 exists; PF: tile
  // j + 2 exists (its packed data is requested after the dequantisation).
  auto step = [&](int j, auto dq, auto pf) {
    constexpr bool DQ = decltype(dq)::value, PF = decltype(pf)::value;
    const int k = j - tile_begin;
    __syncthreads();
    if (DQ) take(pre, cur);
    // one straight-line block per kind of wave, so that the PV MFMAs and
    // the dequantisation can be interleaved
    if (live) {
      pv((k + 2) % 3, pprev);
      if (DQ) dequant(j + 1, cur, (k + 1) & 1, (k + 1) % 3, std::false_type{});
    } else {
      if (DQ) dequant(j + 1, cur, (k + 1) & 1, (k + 1) % 3, std::false_type{});
    }
    if (PF) prefetch(j + 2, pre, std::false_type{});
    if (live) qk_softmax(k & 1, pprev, j * 64, std::false_type{});
    if (PF) {
      prefetch_cent(pre);
      store_params(j + 2, pre);
    }
  };
  {
    int j = tile_begin;
    for (; j + 2 < full_end; ++j) step(j, std::true_type{}, std::true_type{});
    if (j + 1 < full_end) step(j++, std::true_type{}, std::false_type{});
    if (j < full_end) step(j++, std::false_type{}, std::false_type{});
  }
  // drain: PV of the last full tile
  if (nfull > 0 && live) pv((nfull - 1) % 3, pprev);

  // ---- the ragged last tile, unpipelined
  if (has_ragged) {
    const int tile = tile_end - 1;
    __syncthreads();   // every buffer is free
    prefetch(tile, pre, std::true_type{});
    prefetch_cent(pre);
    store_params(tile, pre);
    __syncthreads();
    take(pre, cur);
    dequant(tile, cur, 0, 0, std::true_type{});
    __syncthreads();
    if (live) {
      h8 pb[kNT][2];
      qk_softmax(0, pb, tile * 64, std::true_type{});
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
