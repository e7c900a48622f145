// Per-token int4 quantization of already rotated values, eight at a time
// (the 4-bit activations and KV cache of rotated W2A4/KV4 inference, Qift
// abstract): code = rint(x / s) with s = absmax / 7, IEEE float32 quotient,
// round half to even, packed as eight two's-complement nibbles in one word
// (element j at bits 4j..4j+3).
//
// Fast path: P = v * r exactly, with r = fl(norm * fl(1 / s)) for x =
// fl(v * norm) (norm = 1 for an unrotated x = v). For |x / s| <= 7.5, P is
// within 1.4e-6 of x / s (three roundings of 2^-24 relative each), so
// whenever P is more than 1e-5 away from a half-integer, P, x / s and the
// correctly rounded quotient all round to the same integer. The caller
// tracks the largest |P - rint(P)| of a group and recomputes the group with
// the exact division when it exceeds 0.49999 (or when r is not finite, i.e.
// s is so small that 1 / s overflows).
//
// Rounding uses the float adder inside a fused multiply-add: fl(v * r +
// (1.5 * 2^23 + 8)) rounds the exact product to the nearest integer, ties to
// even (the constant is even), and leaves 8 + rint(P), a value in [1, 15]
// for |P| <= 7.5, in the low nibble of the sum's bits with nothing above it
// up to bit 22; a second fused multiply-add gives P - rint(P). Two such words
// combine into a byte with one shift-and-add, four bytes into a word with two
// byte permutes, and the offset of 8 turns into two's complement with one xor
// of 0x8 per nibble.
#pragma once

#include "qift_internal.h"

namespace qift {

constexpr float kRintMagic8 = 12582920.0f;  // 1.5 * 2^23 + 8

// codes of v[0..7] * r (each product rounded once, inside the adder); dmax is
// raised to the largest |v r - rint(v r)|
__device__ __forceinline__ uint32_t int4x8_rint_fma(const float v[8], float r, float& dmax) {
  uint32_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float ym = __builtin_fmaf(v[j], r, kRintMagic8);
    const float t = ym - kRintMagic8;  // rint(v r), exact
    dmax = fmaxf(dmax, fabsf(__builtin_fmaf(v[j], r, -t)));
    e[j] = __float_as_uint(ym);
  }
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = (e[2 * i + 1] << 4) + e[2 * i];
  const uint32_t lo = __builtin_amdgcn_perm(p[1], p[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(p[3], p[2], 0x04000c0cu);
  return (lo | hi) ^ 0x88888888u;
}

// the same for four values: codes of v[0..3] * r in the low 16 bits
__device__ __forceinline__ uint32_t int4x4_rint_fma(const float v[4], float r, float& dmax) {
  uint32_t e[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float ym = __builtin_fmaf(v[j], r, kRintMagic8);
    const float t = ym - kRintMagic8;
    dmax = fmaxf(dmax, fabsf(__builtin_fmaf(v[j], r, -t)));
    e[j] = __float_as_uint(ym);
  }
  const uint32_t p0 = (e[1] << 4) + e[0], p1 = (e[3] << 4) + e[2];
  return __builtin_amdgcn_perm(p1, p0, 0x0c0c0400u) ^ 0x8888u;
}

// the same codes from the exact IEEE division, clamped to [-7, 7] (s == 0
// gives 0). The clamp binds only when s = fl(absmax / 7) is subnormal: its
// rounding can then make |x / s| exceed 7.5 (absmax = 8 * 2^-149 gives
// s = 2^-149 and x / s = 8).
__device__ __forceinline__ uint32_t int4x8_exact(const float x[8], float s) {
  uint32_t w = 0;
  if (s == 0.f) return 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = min(max((int)rintf(__fdiv_rn(x[j], s)), -7), 7);
    w |= ((uint32_t)q & 0xFu) << (4 * j);
  }
  return w;
}

// four values: int4x8_exact's codes in the low 16 bits
__device__ __forceinline__ uint32_t int4x4_exact(const float x[4], float s) {
  uint32_t w = 0;
  if (s == 0.f) return 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = min(max((int)rintf(__fdiv_rn(x[j], s)), -7), 7);
    w |= ((uint32_t)q & 0xFu) << (4 * j);
  }
  return w;
}

// the fast path is valid for this row's reciprocal (finite, including r == 0
// for an all-zero row)
__device__ __forceinline__ bool rint_path_ok(float r) { return fabsf(r) <= 3.4e38f; }

}  // namespace qift
