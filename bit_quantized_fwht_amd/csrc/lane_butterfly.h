// Walsh-Hadamard butterflies between lanes of a wave, for the stages whose
// partner element sits in another lane (partner lane = lane ^ H, H in
// {1, 2, 4, 8}, always inside one 16-lane DPP row).
//
// The plain butterfly gives the lower lane a + b and the upper lane a - b
// (a the lower lane's value, b the upper's). Here a lane keeps its values up
// to a sign sigma (true value = sigma * stored); partners always share sigma
// because it only depends on lane bits of stages already done. Then the lower
// lane's new stored value is stored + partner and the upper lane's is
// partner - stored = -(stored - partner), so every lane computes
//     stored' = partner * c + stored,   c = +1 (lower) or -1 (upper),
// and the upper lane flips its sigma. The products are exact, so the stored
// values are the float32 butterfly results up to sign. One v_fmac_f32 whose
// first source is read from the partner lane through DPP does a value:
//   H = 1, 2: quad_perm [1,0,3,2] / [2,3,0,1]; H = 8: row_ror:8 (rotating a
//   16-lane row by 8 is lane ^ 8); H = 4: row_half_mirror (lane 7 - i of each
//   8-lane half, i.e. i ^ 7) into a temporary, then quad_perm [3,2,1,0]
//   (i ^ 3) in the fmac, which together read lane i ^ 4.
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

// t = value of v in lane (i ^ 7) of its 8-lane half
#define QIFT_MIRROR(t, i) "v_mov_b32_dpp %" #t ", %" #i " row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
#define QIFT_FMAC_SRC(i, s, CTRL) \
  "v_fmac_f32_dpp %" #i ", %" #s ", %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"

// v[j] = (value of v[j] in lane ^ H) * c + v[j], j = 0..7
template <int H>
__device__ __forceinline__ void lane_butterfly8(float* v, float c) {
  static_assert(H == 1 || H == 2 || H == 4 || H == 8, "partner inside a 16-lane row");
  if constexpr (H == 1) {
    QIFT_FMAC_SELF8("quad_perm:[1,0,3,2]");
  } else if constexpr (H == 2) {
    QIFT_FMAC_SELF8("quad_perm:[2,3,0,1]");
  } else if constexpr (H == 8) {
    QIFT_FMAC_SELF8("row_ror:8");
  } else {
    float t[8];
    // operands: v = %0..%7, t = %8..%15, c = %16
    asm("s_nop 1\n\t" QIFT_MIRROR(8, 0) QIFT_MIRROR(9, 1) QIFT_MIRROR(10, 2) QIFT_MIRROR(11, 3)
            QIFT_MIRROR(12, 4) QIFT_MIRROR(13, 5) QIFT_MIRROR(14, 6) QIFT_MIRROR(15, 7)
        "s_nop 1\n\t" QIFT_FMAC_SRC(0, 8, "quad_perm:[3,2,1,0]")
            QIFT_FMAC_SRC(1, 9, "quad_perm:[3,2,1,0]") QIFT_FMAC_SRC(2, 10, "quad_perm:[3,2,1,0]")
                QIFT_FMAC_SRC(3, 11, "quad_perm:[3,2,1,0]") QIFT_FMAC_SRC(4, 12, "quad_perm:[3,2,1,0]")
                    QIFT_FMAC_SRC(5, 13, "quad_perm:[3,2,1,0]")
                        QIFT_FMAC_SRC(6, 14, "quad_perm:[3,2,1,0]")
                            QIFT_FMAC_SRC(7, 15, "quad_perm:[3,2,1,0]")
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
          "+v"(v[7]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]),
          "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(c));
  }
}

#undef QIFT_FMAC_SELF
#undef QIFT_FMAC_SELF8
#undef QIFT_FMAC_SRC
#undef QIFT_MIRROR

// value of x in lane (lane ^ H) of the same quad, H in {1, 2}
template <int H>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int kCtrl = H == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] or [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

}  // namespace qift
