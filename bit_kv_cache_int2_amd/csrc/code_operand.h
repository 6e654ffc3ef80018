// Exact fp16 MFMA operands made from packed 2-bit codes: a code placed at
// mantissa bits 8-9 under exponent 2 reads 4 + code, at bits 6-7 under
// exponent 4 16 + code, at bits 4-5 under exponent 6 64 + code.  The
// product of such an operand with any fp16 value is exact in the MFMA's
// fp32 accumulation; the base is removed separately.
#pragma once

#include "device.h"

namespace kvq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// (t & mask) | bits.  gfx9 VOP3 encodings take no literal constants and at
// most one scalar operand, so v_and_or_b32 needs one of the constants in a
// VGPR: callers pass the bits through an empty asm statement once, which
// hides their value and makes the compiler keep them in a register.
KVQ_DEV uint32_t and_or(uint32_t t, uint32_t mask, uint32_t bits) { return (t & mask) | bits; }

// Operand dwords for the 16 codes of word d: out[i] holds codes (i, i + 8)
// in its (low, high) half as base_i + code.  No bit of one half reaches the
// selected bits of the other: a left shift by 6 moves the low half to bits
// 6..21 (the high half's codes sit at 22 and up), a right shift by 6 moves
// the high half to bits 10..25 (the low half's codes end at bit 9).
struct CodeOr {
  uint32_t b64, b16, b4;   // exponent bits of 64, 16 and 4 in both halves
};
KVQ_DEV void code_word(uint32_t d, const CodeOr& k, uint32_t out[8]) {
  const uint32_t l6 = d << 6, r6 = d >> 6;
  out[0] = and_or(l6, 0x00C000C0u, k.b16);
  out[1] = and_or(l6, 0x03000300u, k.b4);
  out[2] = and_or(d, 0x00300030u, k.b64);
  out[3] = and_or(d, 0x00C000C0u, k.b16);
  out[4] = and_or(d, 0x03000300u, k.b4);
  out[5] = and_or(r6, 0x00300030u, k.b64);
  out[6] = and_or(r6, 0x00C000C0u, k.b16);
  out[7] = and_or(r6, 0x03000300u, k.b4);
}

// Base of code-word position i.
KVQ_DEV float code_base(int i) {
  return (i == 2 || i == 5) ? 64.0f : ((i == 1 || i == 4 || i == 7) ? 4.0f : 16.0f);
}

KVQ_DEV h8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(h8, make_uint4(a, b, c, d));
}

}  // namespace kvq
