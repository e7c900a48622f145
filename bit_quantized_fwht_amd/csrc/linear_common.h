// Shared pieces of the rotated W2A4 linear kernels (decode and prefill):
// Y = (q . level^T) * s_a * s_w * kappa with an exact int32 accumulator (Qift
// abstract: decoded weight application of the no-zero two-bit level sets,
// per-channel scale, 4-bit activations).
//
// Both kernels run on v_mfma_i32_16x16x64_i8. Activations enter the matrix
// core as 16*q (int4 nibble moved to the top half of a byte), 2-bit MNZ codes
// as 32*(2t+1) (two's-complement code in the top two bits, bit 5 set), PoT
// codes as 16*level through a byte table, int4 weights as 16*w; the int32 sum
// is therefore 2^9 (MNZ) or 2^8 times the exact sum q*level and an arithmetic
// shift recovers it. |sum q*level| <= 7*7*65536 keeps every partial sum far
// inside int32.
#pragma once

#include "qift_internal.h"

namespace qift {

// features per lane segment: 64 for 2-bit codes (16 bytes = 4 code words),
// 32 for int4 weights (16 bytes = 4 words of 8)
template <int LV>
struct Fmt {
  static constexpr bool kInt4 = LV == QIFT_LEVELS_INT4;
  static constexpr int kLaneK = kInt4 ? 32 : 64;        // features per 16-byte code load
  static constexpr int kSteps = kLaneK / 16;            // MFMAs per code load
  static constexpr int kChunkK = 4 * kLaneK;            // features per wave step (4 lane groups)
  static constexpr int kShift = acc_shift(LV);
  // 32-bit code words per channel row
  __device__ static __forceinline__ int64_t code_words(int64_t K) { return kInt4 ? K / 8 : K / 16; }
};

template <int LV>
__device__ __forceinline__ v4i weight_operand(const uint4& c, int step, OpConsts k) {
  if constexpr (LV == QIFT_LEVELS_INT4) {
    const uint32_t w0 = step == 0 ? c.x : c.z;
    const uint32_t w1 = step == 0 ? c.y : c.w;
    return int4_operand(w0, w1);
  } else {
    const uint32_t w = step == 0 ? c.x : (step == 1 ? c.y : (step == 2 ? c.z : c.w));
    if constexpr (LV == QIFT_LEVELS_MNZ) return mnz_operand(w, k);
    else if constexpr (LV == QIFT_LEVELS_LUT) return lut_operand(w, k.lut);
    else return pot_operand(w);
  }
}

// activation operand for MFMA step `step` of a lane segment: 2-bit segments
// carry 64 features = 32 bytes (a0, a1), int4-weight segments 32 features =
// 16 bytes (a0 only).
__device__ __forceinline__ v4i act_operand(const uint4& a0, const uint4& a1, int step) {
  switch (step) {
    case 0: return int4_operand(a0.x, a0.y);
    case 1: return int4_operand(a0.z, a0.w);
    case 2: return int4_operand(a1.x, a1.y);
    default: return int4_operand(a1.z, a1.w);
  }
}

__device__ __forceinline__ void store_y(void* Y, int y_dtype, int64_t idx, int acc, float scale) {
  if (y_dtype == QIFT_I32) {
    reinterpret_cast<int*>(Y)[idx] = acc;
  } else {
    const float y = (float)acc * scale;
    if (y_dtype == QIFT_BF16) reinterpret_cast<uint16_t*>(Y)[idx] = float_to_bf16_bits(y);
    else reinterpret_cast<float*>(Y)[idx] = y;
  }
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace qift
