// Quantise-append into the packed INT2 cache.
//
//  * values ([OKV] rotated values, optional, separately per modality) and
//    window keys ([OKV]
//    per-window key ranges): one block per (head, 64-token tile, sequence),
//    see tile_append_kernel.  A token row sits in D/8 lanes, 8 channels (16
//    bytes of bf16) per lane, so a 32-channel parameter group is one lane
//    quad and its min/max two xor-shuffles; the Walsh-Hadamard rotation runs
//    in registers (three in-lane butterfly stages, then one xor-shuffle
//    stage per remaining bit).
//  * centroid keys ([QWM] 1): the values here, the keys in assign.hip.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace kvq {
namespace {

// Fourth word of a raw buffer resource (32-bit data format), and the
// non-temporal cache policy of streamed input rows.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kStreamPolicy = 2;


// INT2 codes by sign bits.  The kernels hold each threshold negated,
// u_k = fma(-(k + 1/2), s, -z) = -t_k exactly, which is +0 (never -0) when
// t_k is zero and -inf for a zero step.  The sign of RN(x + u_k) is then the
// sign of the exact x - t_k, so bit 31 of x + u_k is (x < t_k), zeros
// included.  With s_k = (x < t_k) and t0 <= t1 <= t2, the code's high bit is
// not s1 and its low bit is not (s1 ? s0 : s2): the middle threshold picks
// the outer one.  acc collects the inverted bits from the top element down,
// one v_alignbit (acc << 1 | d >> 31) per bit, starting from all ones so
// that the inverted word has zeros above the bits collected.
struct NegThr {
  float u0, u1, u2;
};

KVQ_DEV NegThr neg_thresholds(const Q2& q) {
  NegThr n;
  const bool zero = (q.s == 0.0f);
  n.u0 = zero ? -__builtin_inff() : __builtin_fmaf(-0.5f, q.s, -q.z);
  n.u1 = zero ? -__builtin_inff() : __builtin_fmaf(-1.5f, q.s, -q.z);
  n.u2 = zero ? -__builtin_inff() : __builtin_fmaf(-2.5f, q.s, -q.z);
  return n;
}

KVQ_DEV uint32_t code_bits(uint32_t acc, float x, float u0, float u1, float u2) {
  const uint32_t d0 = __float_as_uint(x + u0), d1 = __float_as_uint(x + u1),
                 d2 = __float_as_uint(x + u2);
  acc = __builtin_amdgcn_alignbit(acc, d1, 31);
  return __builtin_amdgcn_alignbit(acc, (d1 & d0) | (~d1 & d2), 31);   // v_bfi_b32
}

// ---------------------------------------------------------------- values
// Walsh-Hadamard rotation of one token row spread over D/8 lanes (8
// elements per lane, element index = lane-in-row * 8 + k).  Stages run with
// h = 1, 2, 4 in-lane and then h = 8, 16, ... across lanes, each pair (i,
// i+h) becoming (a+b, a-b); finally every element is scaled by
// fp32(1/sqrt(D)).
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
  auto stage = [&](auto sc) {
    constexpr int S = decltype(sc)::value;
    const bool upper = (lane & S) != 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float o = lane_xor<S>(x[k]);
      x[k] = upper ? (o - x[k]) : (x[k] + o);
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  if constexpr (D / 8 > 8) stage(std::integral_constant<int, 8>{});
  static_assert(D / 8 <= 16, "wht_row: at most four cross-lane stages");
  const float c = __uint_as_float(D == 128 ? 0x3DB504F3u : 0x3E000000u);
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = x[k] * c;
}

// ---------------------------------------------------------------- append
// One block per (head, 64-token tile touched by the append, sequence).
// Thread (r0, j) owns the 8-channel slice j of rows r0, r0 + RPP, ... of
// the tile, for both keys and values, and issues all of its 16-byte loads
// before any arithmetic.
//  * values: quantised per row (lane quads); the codes are transposed into
//    the tile's channel-major layout through LDS words (one 32-bit word holds
//    16 tokens of one channel) and written back as whole tiles, keeping the
//    codes of tokens an earlier append already stored in this tile;
//  * keys (KEYS, window mode): when the append completes the window, each
//    channel's min/max is reduced in registers (xor shuffles across the rows
//    a wave holds, then one LDS exchange across the four waves), one thread
//    per channel derives the thresholds, and every thread packs the codes of
//    its own slices.  Block 0 also writes the tokens of the window left
//    unfinished into the tail, after every thread has read the old tail.
// VM: 0 plain values, 1 rotated, 2 rotated per modality (the rotated row
// with the channels whose sign is -1 in the token's modality negated).
// Cache words are stored non-temporally: interleaved with the input stream,
// ordinary stores cost the kernel ~6% (a probe of the same reads and
// writes: 477 against 449 us).
template <int D, int VM, bool KEYS>
__global__ __launch_bounds__(256) void tile_append_kernel(
    const uint16_t* __restrict__ kin, const uint16_t* __restrict__ vin,
    uint8_t* __restrict__ kcodes, uint32_t* __restrict__ kparams,
    uint16_t* __restrict__ ktail, uint8_t* __restrict__ vcodes,
    uint32_t* __restrict__ vparams, int H, int Tcap, int cur_len, int n_new,
    const uint32_t* __restrict__ vsigns, const uint8_t* __restrict__ vmodal, int M) {
  constexpr bool HAD = VM != 0;
  constexpr int LPR = D / 8, RPP = 256 / LPR, NP = kWindow / RPP;
  __shared__ float red_mn[4][D], red_mx[4][D];
  __shared__ float thr[3][D];   // negated key thresholds per channel
  __shared__ __align__(16) uint32_t vt[D][4];

  // windows vary fastest across blocks (consecutive blocks stream
  // consecutive windows of one head: 7% faster than heads fastest, whose
  // concurrent blocks together read whole token rows)
  const int job = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * H + h;
  const int end = cur_len + n_new;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = tid % LPR, r0 = tid / LPR;
  const int w = cur_len / kWindow + job;
  const int wb = w * kWindow;
  const int t_lo = max(wb, cur_len), t_hi = min(wb + kWindow, end);
  const bool full = KEYS && wb + kWindow <= end;
  const uint16_t* tail = ktail + bh * kWindow * D;
  uint32_t* vtile = reinterpret_cast<uint32_t*>(vcodes + (bh * (Tcap / kWindow) + w) * (int64_t)D * 16);

  // Every load is issued unconditionally from an in-bounds row (a guarded
  // load compiles to a branch around a wait, which would serialise them):
  // value rows clamp into the new tokens [t_lo, t_hi); key rows read the
  // window when it completes (earlier tokens from the tail) and otherwise
  // the same clamped rows, whose contents go unused.  Rows outside
  // [t_lo, t_hi) give codes in tile slots past the stream's end, which are
  // unspecified, or none at all.
  const int64_t row0 = ((int64_t)b * n_new - cur_len) * H + h;   // row index of token p: row0 + p * H
  uint4 vraw[NP], kraw[NP];
  uint32_t vneg[NP];   // per-modality rotations: sign bits of this row's 8 channels
  auto signs = [&](int tok) -> uint32_t {
    if (VM != 2) return 0u;
    const int m = min((int)vmodal[(int64_t)b * Tcap + tok], M - 1);
    return (vsigns[((int64_t)h * M + m) * (D / 32) + (8 * j) / 32] >> ((8 * j) & 31)) & 0xFFu;
  };
  if (cur_len <= wb && wb + kWindow <= end) {
    // every row of the window is new: buffer views from token wb's row,
    // a fixed per-lane offset and one scalar offset per row step
    const int64_t rw = (row0 + (int64_t)wb * H) * D;
    const int span = kWindow * H * D * 2;
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vin + rw), (short)0, span, kRsrcWord3);
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kin + rw), (short)0, span, kRsrcWord3);
    const int vo = (r0 * H * D + j * 8) * 2;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int so = k * RPP * H * D * 2;
      const auto vv = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, so, kStreamPolicy);
      const auto kv = __builtin_amdgcn_raw_buffer_load_b128(rk, vo, so, kStreamPolicy);
      vraw[k] = make_uint4(vv[0], vv[1], vv[2], vv[3]);
      kraw[k] = make_uint4(kv[0], kv[1], kv[2], kv[3]);
      vneg[k] = signs(wb + r0 + RPP * k);
    }
  } else {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int p = wb + r0 + RPP * k;
      const int pc = min(max(p, t_lo), t_hi - 1);
      vraw[k] = ld_stream(vin + (row0 + (int64_t)pc * H) * D + j * 8);
      vneg[k] = signs(pc);
      const int pk = full ? p : pc;
      const uint16_t* src = (pk < cur_len) ? tail + (int64_t)(pk & (kWindow - 1)) * D
                                           : kin + (row0 + (int64_t)pk * H) * D;
      kraw[k] = ld_stream(src + j * 8);
    }
  }
  // value tile words.  A tile that starts fresh (no earlier tokens in it) is
  // assembled from whole bytes; otherwise the words start from the codes of
  // the tokens an earlier append stored and new codes are OR-ed in.
  const int kept = t_lo - wb;   // tokens [wb, t_lo) are already in the tile
  const bool fresh = (kept == 0) && (D == 128);
  if (!fresh) {
    for (int e = tid; e < D * 4; e += 256) {
      const int wd = e & 3;
      const int keep = min(max(kept - 16 * wd, 0), 16);      // tokens of this word to keep
      const uint32_t mask = keep >= 16 ? 0xFFFFFFFFu : ((1u << (2 * keep)) - 1u);
      vt[e >> 2][wd] = keep > 0 ? (vtile[e] & mask) : 0u;
    }
  }
  __syncthreads();

  // ---- values
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int tt = r0 + RPP * k;                 // token within the tile
    const int p = wb + tt;
    const bool ok = p >= t_lo && p < t_hi;
    float x[8];
    bf16x8_to_f32(vraw[k], x);
    if (HAD) wht_row<D>(x);
    if (VM == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(__float_as_uint(x[e]) ^ (((vneg[k] >> e) & 1u) << 31));
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      mn = fminf(mn, x[e]);
      mx = fmaxf(mx, x[e]);
    }
    mn = fminf(mn, lane_xor<1>(mn));
    mx = fmaxf(mx, lane_xor<1>(mx));
    mn = fminf(mn, lane_xor<2>(mn));
    mx = fmaxf(mx, lane_xor<2>(mx));
    const Q2 q = q2_make(mn, mx);
    const NegThr u = neg_thresholds(q);
    uint32_t acc = ~0u;                      // channel 8j+e at bits [2e, 2e+1] of ~acc
#pragma unroll
    for (int e = 7; e >= 0; --e) acc = code_bits(acc, x[e], u.u0, u.u1, u.u2);
    const uint32_t bits = ~acc & 0xFFFFu;
    if (fresh) {
      // D = 128: lanes 16i + j (i = 0..3) of this wave hold tokens 4*wave + i
      // (+16k) of the same 8 channels.  Spread each lane's codes to one byte
      // per channel (bits 2i), OR the four lanes together, and let lane i
      // write the bytes of channels 8j + 2i, 8j + 2i + 1 (tokens 16k + 4w ..
      // 16k + 4w + 3 form byte w of word (channel, k)).
      const int i = lane >> 4;
      auto spread = [](uint32_t t) {          // 4 two-bit codes -> bytes 0..3
        t = (t | (t << 12)) & 0x000F000Fu;
        return (t | (t << 6)) & 0x03030303u;
      };
      uint32_t v0 = spread(bits & 0xFFu) << (2 * i), v1 = spread(bits >> 8) << (2 * i);
      v0 |= lane_xor<16>(v0);
      v1 |= lane_xor<16>(v1);
      v0 |= lane_xor<32>(v0);
      v1 |= lane_xor<32>(v1);
      uint8_t* vb = reinterpret_cast<uint8_t*>(&vt[0][0]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * i + u;
        const uint32_t src = (e < 4) ? v0 : v1;
        vb[((j * 8 + e) * 4 + (tt >> 4)) * 4 + wave] = (uint8_t)(src >> (8 * (e & 3)));
      }
    } else if (ok) {
      const int sh = 2 * (tt & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) atomicOr(&vt[j * 8 + e][tt >> 4], ((bits >> (2 * e)) & 3u) << sh);
    }
    if (ok && (j & 3) == 0) __builtin_nontemporal_store(q.word, &vparams[(bh * Tcap + p) * (D / kGroup) + (j >> 2)]);
  }
  __syncthreads();
  for (int e = tid; e < D * 4 / 2; e += 256)
    __builtin_nontemporal_store(reinterpret_cast<const v2u*>(&vt[0][0])[e], reinterpret_cast<v2u*>(vtile) + e);

  if (!KEYS) return;
  // ---- keys of a completed window
  if (full) {
    float kx[NP][8], mn[8], mx[8];
#pragma unroll
    for (int k = 0; k < NP; ++k) bf16x8_to_f32(kraw[k], kx[k]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = kx[0][e];
      mx[e] = kx[0][e];
#pragma unroll
      for (int k = 1; k < NP; ++k) {
        mn[e] = fminf(mn[e], kx[k][e]);
        mx[e] = fmaxf(mx[e], kx[k][e]);
      }
      // rows held by this wave: lanes with the same j differ in bits >= log2(LPR)
      if constexpr (LPR <= 8) {
        mn[e] = fminf(mn[e], lane_xor<8>(mn[e]));
        mx[e] = fmaxf(mx[e], lane_xor<8>(mx[e]));
      }
      mn[e] = fminf(mn[e], lane_xor<16>(mn[e]));
      mx[e] = fmaxf(mx[e], lane_xor<16>(mx[e]));
      mn[e] = fminf(mn[e], lane_xor<32>(mn[e]));
      mx[e] = fmaxf(mx[e], lane_xor<32>(mx[e]));
    }
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        red_mn[wave][j * 8 + e] = mn[e];
        red_mx[wave][j * 8 + e] = mx[e];
      }
    }
    __syncthreads();
    if (tid < D) {
      float a = red_mn[0][tid], c = red_mx[0][tid];
#pragma unroll
      for (int v = 1; v < 4; ++v) {
        a = fminf(a, red_mn[v][tid]);
        c = fmaxf(c, red_mx[v][tid]);
      }
      const Q2 q = q2_make(a, c);
      const NegThr u = neg_thresholds(q);
      thr[0][tid] = u.u0;
      thr[1][tid] = u.u1;
      thr[2][tid] = u.u2;
      __builtin_nontemporal_store(q.word, &kparams[(bh * (Tcap / kWindow) + w) * D + tid]);
    }
    __syncthreads();
    float u0[8], u1[8], u2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u0[e] = thr[0][j * 8 + e];
      u1[e] = thr[1][j * 8 + e];
      u2[e] = thr[2][j * 8 + e];
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      uint32_t acc = ~0u;
#pragma unroll
      for (int e = 7; e >= 0; --e) acc = code_bits(acc, kx[k][e], u0[e], u1[e], u2[e]);
      const uint32_t bits = ~acc;
      __builtin_nontemporal_store((uint16_t)bits,
                                  reinterpret_cast<uint16_t*>(kcodes + (bh * Tcap + wb + r0 + RPP * k) * (D / 4) + j * 2));
    }
  }
  if (job == 0) {
    __syncthreads();  // every thread has read the old tail
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

template <int D, bool KEYS>
hipError_t launch_tile_append(const kvq_cache* c, const void* k, const void* v, int cur_len,
                              int n_new, hipStream_t st) {
  const kvq_layout& L = c->layout;
  const int end = cur_len + n_new;
  const int jobs = (end - 1) / kWindow - cur_len / kWindow + 1;
  const dim3 grid((unsigned)jobs, (unsigned)L.kv_heads, (unsigned)L.batch);
  auto args = [&](auto kern) {
    kern<<<grid, 256, 0, st>>>((const uint16_t*)k, (const uint16_t*)v, (uint8_t*)c->k_codes,
                               (uint32_t*)c->k_params, (uint16_t*)c->k_tail,
                               (uint8_t*)c->v_codes, (uint32_t*)c->v_params, L.kv_heads,
                               L.capacity, cur_len, n_new, (const uint32_t*)c->v_signs,
                               (const uint8_t*)c->v_modality, L.n_modalities);
  };
  if (L.value_mode == KVQ_VAL_HADAMARD_MODAL) args(tile_append_kernel<D, 2, KEYS>);
  else if (L.value_mode == KVQ_VAL_HADAMARD) args(tile_append_kernel<D, 1, KEYS>);
  else args(tile_append_kernel<D, 0, KEYS>);
  return hipGetLastError();
}

template <int D>
hipError_t launch_append(const kvq_cache* c, const void* k, const void* v, int cur_len,
                         int n_new, hipStream_t st) {
  const kvq_layout& L = c->layout;
  if (L.key_mode == KVQ_KEY_WINDOW) return launch_tile_append<D, true>(c, k, v, cur_len, n_new, st);
  hipError_t e = launch_tile_append<D, false>(c, k, v, cur_len, n_new, st);
  if (e != hipSuccess) return e;
  return launch_centroid_append(c, k, cur_len, n_new, st);   // assign.hip
}

}  // namespace

hipError_t launch_quantize_append(const kvq_cache* c, const void* k_bf16,
                                  const void* v_bf16, int cur_len, int n_new,
                                  hipStream_t stream) {
  if (n_new == 0) return hipSuccess;
  return (c->layout.head_dim == 128) ? launch_append<128>(c, k_bf16, v_bf16, cur_len, n_new, stream)
                                     : launch_append<64>(c, k_bf16, v_bf16, cur_len, n_new, stream);
}

}  // namespace kvq
