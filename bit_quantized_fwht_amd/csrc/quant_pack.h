// Per-token int4 quantization of already rotated values, eight at a time
// (the 4-bit activations and KV cache of rotated W2A4/KV4 inference, Qift
// abstract): code = rint(x / s) with s = absmax / 7, IEEE float32 quotient,
// round half to even, packed as eight two's-complement nibbles in one word
// (element j at bits 4j..4j+3).
//
// Fast path: y = x * r with r = 1 / s (or y = v * fl(norm * r) for x =
// fl(v * norm)). For |x / s| <= 7.5, y is within 1.8e-6 of x / s (at most
// four roundings of 2^-24 relative each), so whenever y is more than 1e-5
// away from a half-integer, y, x / s and the correctly rounded quotient all
// round to the same integer. The caller tracks the largest |y - rint(y)| of a group
// and recomputes the group with the exact division when it exceeds 0.49999
// (or when r is not finite, i.e. s is so small that 1 / s overflows).
//
// Rounding uses the float adder: y + (1.5 * 2^23 + 8) rounds y to the nearest
// integer, ties to even (the constant is even), and leaves 8 + rint(y), a
// value in [1, 15] for |y| <= 7.5, in the low nibble of the sum's bits with
// nothing above it up to bit 22. Two such words combine into a byte with one
// shift-and-add, four bytes into a word with two byte permutes, and the
// offset of 8 turns into two's complement with one xor of 0x8 per nibble.
#pragma once

#include "qift_internal.h"

namespace qift {

constexpr float kRintMagic8 = 12582920.0f;  // 1.5 * 2^23 + 8

// codes of y[0..7] (already multiplied by 1 / s); dmax is raised to the
// largest |y[j] - rint(y[j])|
__device__ __forceinline__ uint32_t int4x8_rint(const float y[8], float& dmax) {
  uint32_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float ym = y[j] + kRintMagic8;
    const float t = ym - kRintMagic8;  // rint(y[j]), exact
    dmax = fmaxf(dmax, fabsf(y[j] - t));
    e[j] = __float_as_uint(ym);
  }
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = (e[2 * i + 1] << 4) + e[2 * i];  // byte: two offset nibbles
  const uint32_t lo = __builtin_amdgcn_perm(p[1], p[0], 0x0c0c0400u);  // bytes p0.b0, p1.b0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(p[3], p[2], 0x04000c0cu);  // bytes 0, 0, p2.b0, p3.b0
  return (lo | hi) ^ 0x88888888u;
}

// the same codes from the exact IEEE division (s == 0 gives 0)
__device__ __forceinline__ uint32_t int4x8_exact(const float x[8], float s) {
  uint32_t w = 0;
  if (s == 0.f) return 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= ((uint32_t)(int)rintf(__fdiv_rn(x[j], s)) & 0xFu) << (4 * j);
  return w;
}

// the fast path is valid for this row's reciprocal (finite, including r == 0
// for an all-zero row)
__device__ __forceinline__ bool rint_path_ok(float r) { return fabsf(r) <= 3.4e38f; }

}  // namespace qift
