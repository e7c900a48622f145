// Internal declarations of libqift: device helpers shared by the kernels,
// the grouped-linear plan layout, and the launchers called by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "qift.h"

namespace qift {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// workgroup barrier for LDS exchanges
// ---------------------------------------------------------------------------

// A workgroup barrier that orders LDS accesses only. __syncthreads() also
// orders global memory, which on gfx9 means waiting for every outstanding
// global load (one counter covers loads and stores): a barrier inside a
// kernel that keeps a weight stream in flight would drain that stream.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// element loads / stores
// ---------------------------------------------------------------------------

// A pointer the kernels know to point into device global memory. A pointer
// read from memory (the descriptors of a grouped plan) is otherwise generic:
// its accesses become flat instructions, which count against the LDS counter
// as well, so a wait for any of them waits for every outstanding load, store
// and LDS access.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* as_global(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* as_global_out(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float32 -> bfloat16, round to nearest even: gfx950's v_cvt_pk_bf16_f32
// (one instruction for two values; NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The 4-bit two's-complement code of clamp(rint(x / s), -7, 7), x / s the
// IEEE float32 quotient, for |x| <= absmax and s = fl(absmax / 7), computed
// as rint(x * r) with r = 1 / s except near a rounding tie:
//  - for |x / s| <= 7.5, x * r is within 1.3e-6 of the correctly rounded
//    quotient (two roundings of 2^-24 relative each), so when x * r is more
//    than 1e-5 from a half-integer both round to the same integer;
//  - within that window, or when x * r is not finite (1/s overflowing for a
//    tiny s), the exact division decides, clamped: a subnormal s can be
//    rounded far enough below absmax / 7 that |x / s| > 7.5 (the clamp cannot
//    bind while 1/s is finite, since s > 2^-128 keeps that rounding below
//    2^-22 relative);
//  - rint uses the float adder: y + 1.5*2^23 rounds to nearest even and
//    leaves rint(y) in the low mantissa bits in two's complement.
// s == 0 gives code 0.
__device__ __forceinline__ uint32_t code_int4_recip(float x, float s, float r) {
  const float kMagic = 12582912.0f;  // 1.5 * 2^23
  const float y = x * r;
  const float ym = y + kMagic;
  const float t = ym - kMagic;       // rint(y), exact
  uint32_t code = __float_as_uint(ym) & 0xFu;
  if (!(fabsf(y - t) <= 0.49999f))
    code = (uint32_t)min(max((int)rintf(__fdiv_rn(x, s)), -7), 7) & 0xFu;
  return s == 0.f ? 0u : code;
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard operands for v_mfma_f32_16x16x32_bf16 (KV4)
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Eight bfloat16 entries +-1 of a Walsh-Hadamard operand (two per word, the
// lower index in the low half): row r of H_8 (r < 8), all signs flipped when
// popcount(hi) is odd. Entry j is negative when popcount(r & j) is odd: for
// j = 2 m + 1 that is the sign of j = 2 m times (-1)^(r & 1), and for j = 2 m
// the sign is (-1)^(bit 1 of r * bit 0 of m + bit 2 of r * bit 1 of m).
//
// Operand A of H_32 for lane (slot p = lane % 16, k group q = lane / 16), the
// rows permuted so that half h of the outputs puts output 8 (p / 4) + 4 h +
// p % 4 in slot p: h32_operand_bf16(4 h + p % 4, (p / 4) & q), since
// popcount(i & k) splits over bits 0-2 and 3-4 of i and k. With it, the four
// results of slot rows 4 q' .. 4 q' + 3 that the MFMA leaves in lane
// (column, q') are, over both halves, the eight consecutive outputs 8 q' ..
// 8 q' + 7. The entries are exact, the products with bfloat16 inputs are
// exact, and the MFMA sums them in float32.
__device__ __forceinline__ v4u h32_operand_bf16(int r, int hi) {
  const uint32_t c = 0x3F803F80u ^ ((__builtin_popcount(hi) & 1) ? 0x80008000u : 0u) ^
                     ((r & 1) ? 0x80000000u : 0u);
  const uint32_t b1 = (r & 2) ? 0x80008000u : 0u, b2 = (r & 4) ? 0x80008000u : 0u;
  return v4u{c, c ^ b1, c ^ b2, c ^ b1 ^ b2};
}

__device__ __forceinline__ float load_scale(const void* p, int64_t i, int is_f16) {
  if (is_f16) return __half2float(reinterpret_cast<const __half*>(p)[i]);
  return reinterpret_cast<const float*>(p)[i];
}

// The same value without a branch on the dtype: two 16-bit loads (element i
// of a float16 array twice, or the two halves of element i of a float32
// array), both always issued. A load under a branch makes the compiler wait
// for it where the branch ends, which serializes loads meant to overlap.
__device__ __forceinline__ float load_scale_nb(const void* p, int64_t i, int is_f16) {
  const auto h = as_global(reinterpret_cast<const uint16_t*>(p));
  const int64_t j = is_f16 ? i : 2 * i;
  const uint32_t lo = h[j];
  const uint32_t hi = h[is_f16 ? j : j + 1];
  const float f16v = __half2float(__ushort_as_half((unsigned short)lo));
  return is_f16 ? f16v : __uint_as_float(lo | (hi << 16));
}

// ---------------------------------------------------------------------------
// matrix-core operands for v_mfma_i32_16x16x64_i8
//
// One lane supplies 16 int8 values (4 dwords) for 16 consecutive features
// k0..k0+15. The order of those 16 values inside the dwords is free as long
// as the activation (A) and weight (B) operands use the same one; the order
// used everywhere is
//   dword 0: k0+0, k0+2, k0+4, k0+6      dword 1: k0+1, k0+3, k0+5, k0+7
//   dword 2: k0+8, k0+10, k0+12, k0+14   dword 3: k0+9, k0+11, k0+13, k0+15
// which is what masks of the int4 and 2-bit packed layouts give directly.
// ---------------------------------------------------------------------------

// int4 pairs (two words, 16 features) -> 16*q per byte, exact.
__device__ __forceinline__ v4i int4_operand(uint32_t x0, uint32_t x1) {
  v4i a;
  a[0] = (int)((x0 << 4) & 0xF0F0F0F0u);
  a[1] = (int)(x0 & 0xF0F0F0F0u);
  a[2] = (int)((x1 << 4) & 0xF0F0F0F0u);
  a[3] = (int)(x1 & 0xF0F0F0F0u);
  return a;
}

// Per-call operand constants, derived from the descriptor's table word (the
// level table for QIFT_LEVELS_LUT, always 0 for the other levels):
// - the two masks of the MNZ operand, held in vector registers. gfx9 VOP3
//   encodings take no literal constants, and the compiler only forms
//   v_and_or_b32 from (a & m) | o when m and o live in VGPRs; with literal or
//   scalar masks it emits v_and + v_or. The masks are therefore derived from
//   a per-lane value it cannot fold: word * lane, with word 0 for MNZ;
// - the byte table of a level table: byte c = 8 * L[c] (|L| <= 15, so the
//   byte is the exact signed value).
struct OpConsts {
  uint32_t m, o, lut;
};
__device__ __forceinline__ OpConsts op_consts(int32_t word, int lane) {
  const uint32_t z = (uint32_t)word * (uint32_t)lane;
  return OpConsts{0xC0C0C0C0u | z, 0x20202020u | z, ((uint32_t)word << 3) & 0xF8F8F8F8u};
}

// 2-bit MNZ codes (one word, 16 features) -> 32*(2t+1) per byte: the code t
// lands in the two top bits of its byte (64t as a signed byte) and bit 5 adds
// 32. Seven VALU instructions per 16 codes.
__device__ __forceinline__ v4i mnz_operand(uint32_t c, OpConsts k) {
  v4i b;
  b[0] = (int)(((c << 6) & k.m) | k.o);
  b[1] = (int)(((c << 4) & k.m) | k.o);
  b[2] = (int)(((c << 2) & k.m) | k.o);
  b[3] = (int)((c & k.m) | k.o);
  return b;
}

// 2-bit PoT codes -> 16*level per byte through a 4-entry byte table
// (+1, +4, -1, -4) * 16 selected by v_perm_b32.
__device__ __forceinline__ v4i pot_operand(uint32_t c) {
  const uint32_t lut = 0xC0F04010u;  // bytes: 0x10, 0x40, 0xF0, 0xC0
  v4i b;
  b[0] = (int)__builtin_amdgcn_perm(0u, lut, c & 0x03030303u);
  b[1] = (int)__builtin_amdgcn_perm(0u, lut, (c >> 2) & 0x03030303u);
  b[2] = (int)__builtin_amdgcn_perm(0u, lut, (c >> 4) & 0x03030303u);
  b[3] = (int)__builtin_amdgcn_perm(0u, lut, (c >> 6) & 0x03030303u);
  return b;
}

// 2-bit codes of a level table -> 8 * L[code] per byte through the per-call
// byte table (the PoT decode with a run-time table).
__device__ __forceinline__ v4i lut_operand(uint32_t c, uint32_t lut) {
  v4i b;
  b[0] = (int)__builtin_amdgcn_perm(0u, lut, c & 0x03030303u);
  b[1] = (int)__builtin_amdgcn_perm(0u, lut, (c >> 2) & 0x03030303u);
  b[2] = (int)__builtin_amdgcn_perm(0u, lut, (c >> 4) & 0x03030303u);
  b[3] = (int)__builtin_amdgcn_perm(0u, lut, (c >> 6) & 0x03030303u);
  return b;
}

// Byte table of one channel of the asymmetric grid (QIFT_LEVELS_ASYM):
// byte c = 8 * (c - z), z the channel's zero point (an integer in [0, 3],
// stored as a scale value; anything else is clamped, NaN reads as 0). The
// four bytes are the window of the sequence 8 * (-3, -2, ..., 3) that starts
// at 3 - z. The table then drives the level-table decode, lut_operand, so the
// grid costs the matrix-core loop nothing: the zero point is folded into the
// decoded levels instead of a correction z * sum q after the sum.
__device__ __forceinline__ uint32_t asym_table(float zf) {
  const int z = zf >= 3.f ? 3 : zf >= 2.f ? 2 : zf >= 1.f ? 1 : 0;
  return (uint32_t)(0x0018100800F8F0E8ull >> (8 * (3 - z)));
}

// Right shift that turns the matrix-core sum back into sum q * level:
// MNZ 16 * 32 = 2^9, PoT 16 * 16 = 2^8, INT4 16 * 16 = 2^8, level table
// 16 * 8 = 2^7.
__host__ __device__ constexpr int acc_shift(int levels) {
  return levels == QIFT_LEVELS_MNZ ? 9 : (levels == QIFT_LEVELS_LUT ? 7 : 8);
}
__host__ __device__ constexpr float level_kappa(int levels) {
  return levels == QIFT_LEVELS_MNZ ? 0.5f : 1.0f;
}

__device__ __forceinline__ v4i mfma16(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// grouped linear plan (device copy lives in the caller's workspace)
// ---------------------------------------------------------------------------

struct PlanEntry {          // one linear
  qift_linear_desc d;       // 72 bytes
  int64_t tile_begin;       // first workgroup tile of this linear
  int64_t n_tiles;
};
static_assert(sizeof(qift_linear_desc) == 72, "descriptor layout");
static_assert(sizeof(PlanEntry) == 88, "plan entry layout");

struct PlanHeader {
  uint64_t magic;
  int32_t count;
  int32_t scale_f16;
  int32_t y_dtype;
  int32_t pad0;
  int64_t total_tiles;
  int64_t entries_offset;   // bytes from the workspace start
  int64_t tile_map_offset;  // int32 per tile: index of its linear
  int64_t pad1[2];
};
static_assert(sizeof(PlanHeader) == 64, "plan header layout");
constexpr uint64_t kPlanMagic = 0x5146545f504c414eull;  // "QFT_PLAN"

// decode kernel geometry: 256 threads = 4 waves, each wave QIFT_DECODE_TILES
// x 16 output channels
#ifndef QIFT_DECODE_TILES
#define QIFT_DECODE_TILES 4
#endif
#ifndef QIFT_DECODE_NT
#define QIFT_DECODE_NT 1
#endif
constexpr int kDecodeRowsPerWave = 16 * QIFT_DECODE_TILES;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeRowsPerTile = kDecodeRowsPerWave * kDecodeWaves;

// ---------------------------------------------------------------------------
// launchers (implemented in the .hip files; return a hipError_t)
// ---------------------------------------------------------------------------

// one activation matrix of a batched rotate launch (row-kernel fast path)
struct RotJob {
  const void* X;
  uint8_t* xq;
  float* s_a;
  float* x_rot;
  int K;
  int had_block;  // set by the caller; the launcher derives log2b and norm
  int log2b;
  float norm;
  int bf16;
};
bool rotate_fast_ok(const void* X, int64_t K, int had_block, const uint8_t* xq,
                    const float* x_rot);
hipError_t launch_rotate_quant_act_batched(const RotJob* jobs, const int64_t* rows, int count,
                                           hipStream_t s);
hipError_t launch_rotate_quant_act(const void* X, int x_bf16, int64_t M, int64_t K, int had_block,
                                   uint8_t* xq, float* s_a, float* x_rot, hipStream_t s);
hipError_t launch_quantize_weights(const void* W, int w_bf16, int64_t N, int64_t K, int had_block,
                                   int levels, uint32_t table, int mse_rule, uint32_t* codes,
                                   void* scales, int scale_f16, hipStream_t s);
hipError_t launch_kv4(const void* KV, int bf16, int64_t rows, int D, int had_block, uint8_t* kvq,
                      float* scales, hipStream_t s);
hipError_t launch_kv4_pair(const void* K, const void* V, int bf16, int64_t rows, int D,
                           int had_block, uint8_t* kq, float* ks, uint8_t* vq, float* vs,
                           hipStream_t s);
int64_t kv4_attn_tokens_per_run(int64_t S, int64_t T, int H);
size_t kv4_attn_workspace_bytes(int64_t S, int64_t T, int H);
hipError_t kv4_attn_scratch(float** ptr);
size_t gptq_hessian_workspace_bytes(int64_t S, int64_t K);
hipError_t launch_gptq_hessian(const void* X, int x_bf16, int64_t S, int64_t K, int had_block,
                               int accumulate, double* H, void* workspace, hipStream_t s);
size_t gptq_workspace_bytes(int64_t N, int64_t K);
hipError_t launch_gptq_quantize(const void* W, int w_bf16, int64_t N, int64_t K,
                                const double* H, int had_block, int levels, uint32_t table,
                                int mse_rule, double damp, uint32_t* codes, void* scales,
                                int scale_f16, void* workspace, hipStream_t s);
hipError_t launch_kv4_attention(const void* q, int q_bf16, int64_t S, int64_t T, int H,
                                int had_block, const uint8_t* kq, const float* ks,
                                const uint8_t* vq, const float* vs, float softmax_scale,
                                void* out, int out_bf16, float* part, hipStream_t s);
hipError_t launch_linear_decode(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                hipStream_t s);
hipError_t launch_linear_prefill(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                 hipStream_t s);
hipError_t launch_rotate_linear_decode(const qift_linear_desc& d, const void* X, int x_bf16,
                                       int had_block, int scale_f16, int y_dtype, hipStream_t s);
hipError_t launch_measure_stream(const void* src, void* dst, int64_t bytes, int mode,
                                 uint32_t* sink, hipStream_t s);
hipError_t launch_measure_mfma_i8(int64_t iters, int64_t workgroups, uint32_t* sink,
                                  uint64_t* clk, hipStream_t s);
hipError_t launch_linear_grouped(const void* workspace, int64_t total_tiles, int scale_f16,
                                 int y_dtype, hipStream_t s);

}  // namespace qift
