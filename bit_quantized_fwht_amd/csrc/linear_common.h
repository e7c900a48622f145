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

// lut: the byte table of the lane's channel (level-table kernels only)
template <int LV>
__device__ __forceinline__ v4i weight_operand(const uint4& c, int step, OpConsts k, uint32_t lut) {
  if constexpr (LV == QIFT_LEVELS_INT4) {
    const uint32_t w0 = step == 0 ? c.x : c.z;
    const uint32_t w1 = step == 0 ? c.y : c.w;
    return int4_operand(w0, w1);
  } else {
    const uint32_t w = step == 0 ? c.x : (step == 1 ? c.y : (step == 2 ? c.z : c.w));
    if constexpr (LV == QIFT_LEVELS_MNZ) return mnz_operand(w, k);
    else if constexpr (LV == QIFT_LEVELS_LUT) return lut_operand(w, lut);
    else return pot_operand(w);
  }
}

// Byte tables of the level-table kernels, one per 16-channel tile a lane
// decodes (T tiles, the lane's channel of tile i being chan(i)): the call's
// table for QIFT_LEVELS_LUT; for QIFT_LEVELS_ASYM the table of the lane's
// channel, from its zero point, which follows the N steps in the scales
// (channels past N read channel N - 1). Other kernels ignore them.
template <int LV, int T, typename Chan>
__device__ __forceinline__ void tile_tables(const qift_linear_desc& d, OpConsts k, int scale_f16,
                                            Chan chan, uint32_t (&lut)[T]) {
#pragma unroll
  for (int i = 0; i < T; ++i) lut[i] = k.lut;
  if constexpr (LV == QIFT_LEVELS_LUT) {
    if (d.levels == QIFT_LEVELS_ASYM) {
#pragma unroll
      for (int i = 0; i < T; ++i) {
        const int64_t n = chan(i) < d.N ? chan(i) : d.N - 1;
        lut[i] = asym_table(load_scale_nb(d.scales, d.N + n, scale_f16));
      }
    }
  }
}

// activation operand for MFMA step `step` of a lane segment: 2-bit segments
// carry 64 features = 32 bytes (a0, a1), int4-weight segments 32 features =
// 16 bytes (a0 only). am is the nibble mask: 0xF0F0F0F0 keeps the codes, 0
// zeroes the operand (a segment past K, whose loads read a clamped address).
__device__ __forceinline__ v4i act_operand(const uint4& a0, const uint4& a1, int step,
                                           uint32_t am) {
  const uint32_t x0 = step == 0 ? a0.x : step == 1 ? a0.z : step == 2 ? a1.x : a1.z;
  const uint32_t x1 = step == 0 ? a0.y : step == 1 ? a0.w : step == 2 ? a1.y : a1.w;
  v4i a;
  a[0] = (int)((x0 << 4) & am);
  a[1] = (int)(x0 & am);
  a[2] = (int)((x1 << 4) & am);
  a[3] = (int)(x1 & am);
  return a;
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

// 16- and 8-byte stores through a global pointer (see as_global)
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t e) {
  *as_global_out(reinterpret_cast<v4u*>(p)) = v4u{a, b, c, e};
}
__device__ __forceinline__ void st8(void* p, uint32_t a, uint32_t b) {
  *as_global_out(reinterpret_cast<v2u*>(p)) = v2u{a, b};
}
// the same, non-temporal (written once, not read back by the kernel)
__device__ __forceinline__ void st16_nt(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t e) {
  __builtin_nontemporal_store(v4u{a, b, c, e}, as_global_out(reinterpret_cast<v4u*>(p)));
}
__device__ __forceinline__ void st8_nt(void* p, uint32_t a, uint32_t b) {
  __builtin_nontemporal_store(v2u{a, b}, as_global_out(reinterpret_cast<v2u*>(p)));
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  const v4u v = *as_global(reinterpret_cast<const v4u*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}

}  // namespace qift
