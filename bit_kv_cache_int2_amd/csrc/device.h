// Device helpers shared by the kvint2 kernels (gfx950, wave64).
//
// Number formats follow the contract in include/kvint2.h: IEEE fp32 with
// round-to-nearest-even, no contraction (the library is built with
// -ffp-contract=off; every fused multiply-add is written as fmaf), fp16
// conversions by v_cvt_f16_f32 / v_cvt_f32_f16 in the default RNE mode with
// denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define KVQ_DEV __device__ __forceinline__

namespace kvq {

constexpr int kGroup = 32;
constexpr int kWindow = 64;
constexpr int kWave = 64;

KVQ_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Pins x as an fp32 value in a register.  Without it the backend may fuse
// the producing fma with a following fp16 conversion (v_fma_mix*_f16), which
// rounds once from the exact value instead of to fp32 and then to fp16.
KVQ_DEV float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

KVQ_DEV uint32_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)opaque(x);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

KVQ_DEV float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(b & 0xFFFFu));
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// 16-byte load of data read exactly once (streamed inputs): non-temporal, so
// it does not displace reusable lines from the caches.
KVQ_DEV uint4 ld_stream(const void* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Unpack 8 bf16 held in a uint4 into fp32 (exact; a -0 stays -0: the
// quantizers canonicalise the group minimum and maximum instead, which is
// all a zero's sign can reach, since comparisons treat the two zeros alike).
KVQ_DEV void bf16x8_to_f32(const uint4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// (mx - mn) / 3 correctly rounded in four operations: q0 = d * RN(1/3), the
// exact residual r = d - 3 q0 by fma, then q0 + r * RN(1/3) rounded once.
// Equal to the division for every non-negative fp32 d (checked over all of
// them); d = +inf gives NaN there, which the final min turns back into +inf.
KVQ_DEV float div3(float d) {
  const float y = 0x1.555556p-2f;
  const float q0 = d * y;
  const float r = __builtin_fmaf(-3.0f, q0, d);
  return fminf(__builtin_fmaf(r, y, q0), d);
}

// The INT2 group quantizer's parameters for a group with extrema mn, mx
// (canonical inputs).  t0..t2 are the three decision thresholds; when the
// stored scale is 0 they are +inf so that every code is 0.
struct Q2 {
  float s, z, t0, t1, t2;
  uint32_t word;  // fp16 scale bits | fp16 zero bits << 16
};

// Group parameters from the group's minimum and maximum (canonicalised
// here, so inputs may carry either zero sign).
KVQ_DEV Q2 q2_make(float mn, float mx) {
  Q2 q;
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  const float s32 = div3(mx - mn);
  const uint32_t sh = f32_to_f16_bits(s32), zh = f32_to_f16_bits(mn);
  q.s = f16_bits_to_f32(sh);
  q.z = f16_bits_to_f32(zh);
  q.word = sh | (zh << 16);
  const bool zero = (q.s == 0.0f);
  q.t0 = zero ? __builtin_inff() : __builtin_fmaf(0.5f, q.s, q.z);
  q.t1 = zero ? __builtin_inff() : __builtin_fmaf(1.5f, q.s, q.z);
  q.t2 = zero ? __builtin_inff() : __builtin_fmaf(2.5f, q.s, q.z);
  return q;
}

// Number of thresholds at or below x.  The thresholds are ordered (s >= 0),
// so the middle one picks which of the outer two decides the low bit.
KVQ_DEV uint32_t q2_code(float x, const Q2& q) {
  const bool up = x >= q.t1;
  return (up ? 2u : 0u) + (uint32_t)(x >= (up ? q.t2 : q.t0));
}

// Value of lane (lane ^ M) in a wave of 64, without the generic shuffle's
// per-call index arithmetic: xor 1 and 2 are DPP quad permutes, xor 4, 8
// and 16 swizzles inside each 32-lane half (bit mode: and 0x1F, xor M),
// xor 32 a bpermute.  Every lane must be active.
template <int M>
KVQ_DEV uint32_t lane_xor(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane_xor: power of two below 64");
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  } else if constexpr (M < 32) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (M << 10) | 0x1F);
  } else {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(((int)(threadIdx.x & 63) ^ 32) << 2, (int)v);
  }
}
template <int M>
KVQ_DEV float lane_xor(float v) {
  return __uint_as_float(lane_xor<M>(__float_as_uint(v)));
}

// Wave-level reductions (64 lanes) with butterfly shuffles.
KVQ_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
KVQ_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// fp32 value of byte b (0..3) of x, exact for 0..255 (v_cvt_f32_ubyteN).
template <int B>
KVQ_DEV float ubyte_f32(uint32_t x) {
  return (float)((x >> (8 * B)) & 0xFFu);
}

}  // namespace kvq
