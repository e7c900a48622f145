// Walsh-Hadamard butterflies between lanes of a wave, for the stages whose
// partner element sits in another lane (partner lane = lane ^ M, M in
// {1, 2, 7, 8}, always inside one 16-lane DPP row).
//
// The plain butterfly gives the lower element a + b and the upper a - b (a
// the lower element's value, b the upper's). Here a lane keeps its values up
// to a sign sigma (true value = sigma * stored); partners always share sigma
// because it only depends on index bits of stages already done. Then the
// lower lane's new stored value is stored + partner and the upper lane's is
// partner - stored = -(stored - partner), so every lane computes
//     stored' = partner * c + stored,   c = +1 (lower) or -1 (upper),
// and the upper lane flips its sigma. The products are exact, so the stored
// values are the float32 butterfly results up to sign. One v_fmac_f32 whose
// first source is read from the partner lane through DPP does a value:
//   M = 1, 2: quad_perm [1,0,3,2] / [2,3,0,1]; M = 7: row_half_mirror (lane
//   7 - i of each 8-lane half, i.e. i ^ 7); M = 8: row_ror:8 (rotating a
//   16-lane row by 8 is lane ^ 8). A caller whose partner would sit at
//   lane ^ 4 lays its data out so that it sits at lane ^ 7 instead (a change
//   of basis of the lane index bits; see row_group_of in rotate_row.h),
//   which DPP reads in one step.
// The compiler does not fold a v_mov_b32_dpp into a three-operand fma, hence
// the inline assembly. Each block starts with s_nop 1: a DPP source needs
// two wait states after the VALU instruction that wrote it; inside a block
// no instruction reads a register another instruction of the block wrote.
#pragma once

#include "qift_internal.h"

namespace qift {

#define QIFT_FMAC_SELF(i, CTRL) \
  "v_fmac_f32_dpp %" #i ", %" #i ", %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define QIFT_FMAC_SELF8(CTRL)                                                               \
  asm("s_nop 1\n\t" QIFT_FMAC_SELF(0, CTRL) QIFT_FMAC_SELF(1, CTRL) QIFT_FMAC_SELF(2, CTRL) \
          QIFT_FMAC_SELF(3, CTRL) QIFT_FMAC_SELF(4, CTRL) QIFT_FMAC_SELF(5, CTRL)           \
              QIFT_FMAC_SELF(6, CTRL) QIFT_FMAC_SELF(7, CTRL)                               \
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), \
        "+v"(v[7])                                                                          \
      : "v"(c))

// v[j] = (value of v[j] in lane ^ M) * c + v[j], j = 0..7
template <int M>
__device__ __forceinline__ void lane_butterfly8(float* v, float c) {
  static_assert(M == 1 || M == 2 || M == 7 || M == 8, "partner inside a 16-lane row");
  if constexpr (M == 1) {
    QIFT_FMAC_SELF8("quad_perm:[1,0,3,2]");
  } else if constexpr (M == 2) {
    QIFT_FMAC_SELF8("quad_perm:[2,3,0,1]");
  } else if constexpr (M == 7) {
    QIFT_FMAC_SELF8("row_half_mirror");
  } else {
    QIFT_FMAC_SELF8("row_ror:8");
  }
}

#undef QIFT_FMAC_SELF
#undef QIFT_FMAC_SELF8

// value of x in lane (lane ^ H) of the same quad, H in {1, 2}
template <int H>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int kCtrl = H == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] or [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// Largest of the 64 lanes' values, returned to every lane, for non-negative
// floats (whose bit patterns order like the values, so the max is exact):
// DPP steps within each 16-lane row (quad permutes, half-row and row
// mirrors), row broadcasts across rows (lane 15 into the next row, lane 31
// into the upper two), then lane 63 read back. Replaces six shuffle rounds
// through the LDS crossbar.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  int v = __float_as_int(x);
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

}  // namespace qift
