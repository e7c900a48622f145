// Rotation + per-token int4 quantization of one activation row by a
// workgroup of 256 threads, the fast path of the online activation path
// (rotated W2A4 inference, Qift abstract): the block Walsh-Hadamard rotation
// along K followed by the absmax scale and the int4 codes.
#pragma once

#include "lane_butterfly.h"
#include "quant_pack.h"

namespace qift {

constexpr int kRowThreads = 256;

// --- K1 fast path: K % 16 == 0 and block >= 16 ---------------------------------
//
// Each thread owns groups of 16 consecutive elements, loaded straight into
// registers (32 bytes bf16 / 64 bytes float). Butterfly stages 0-3 run inside
// a group and stages 4-7 between the lanes holding the partner groups
// (rotate_row_fast below), so rows with blocks up to 256 never touch LDS.
// For larger blocks the row is staged in LDS with one pad word per 16 floats
// (element e at e + e / 16): the 16 stores of a thread hit 16 consecutive
// banks and neighbouring threads are 17 words apart, so a wave's stores, the
// stride-256 pass of stages 8-11 and the final consecutive reads are all
// conflict-free.

__device__ __forceinline__ int pad16(int e) { return e + (e >> 4); }

// kMax: also raise m to the largest |value| the pass writes; NT threads
template <int NS, bool kMax = false, int NT = kRowThreads>
__device__ __forceinline__ void fwht_pass_padded(float* row, int K, int p, int tid,
                                                 float* m = nullptr) {
  constexpr int R = 1 << NS;
  const int sh = 4 * p;
  const int S = 1 << sh;
  const int groups = K >> NS;
  // for S >= 16 the padded index is affine in j: low + j S stays below
  // 2^(sh + NS) and j S is a multiple of 16, so pad16(base + j S) =
  // pad16(base) + j (S + S / 16), one base address and immediate offsets
  const int pstride = S >= 16 ? S + (S >> 4) : 0;
  for (int grp = tid; grp < groups; grp += NT) {
    const int low = grp & (S - 1);
    const int high = grp >> sh;
    const int base = (high << (sh + NS)) | low;
    float* const rb = row + pad16(base);
    auto at = [&](int j) -> float& { return S >= 16 ? rb[j * pstride] : row[pad16(base + j * S)]; };
    float v[R];
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = at(j);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int h = 1 << st;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if (!(j & h)) {
          const float a = v[j], b = v[j + h];
          v[j] = a + b;
          v[j + h] = a - b;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) at(j) = v[j];
    if constexpr (kMax) {
#pragma unroll
      for (int j = 0; j < R; ++j) *m = fmaxf(*m, fabsf(v[j]));
    }
  }
}

// 16 consecutive elements as raw words (bfloat16: 8 words of two, float32: 16
// words); widen16 turns them into floats. Keeping the two apart lets a caller
// issue other loads between them without the compiler waiting for these.
template <typename T>
__device__ __forceinline__ void load16_raw(const T* __restrict__ src, uint32_t w[16]);

template <>
__device__ __forceinline__ void load16_raw<uint16_t>(const uint16_t* __restrict__ src,
                                                     uint32_t w[16]) {
  const uint4 a = reinterpret_cast<const uint4*>(src)[0];
  const uint4 b = reinterpret_cast<const uint4*>(src)[1];
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

template <>
__device__ __forceinline__ void load16_raw<float>(const float* __restrict__ src, uint32_t w[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 f = reinterpret_cast<const uint4*>(src)[i];
    w[4 * i] = f.x; w[4 * i + 1] = f.y; w[4 * i + 2] = f.z; w[4 * i + 3] = f.w;
  }
}

template <typename T>
__device__ __forceinline__ void widen16(const uint32_t w[16], float v[16]);

template <>
__device__ __forceinline__ void widen16<uint16_t>(const uint32_t w[16], float v[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void widen16<float>(const uint32_t w[16], float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(w[i]);
}

// One row on the fast path, by a workgroup of NT threads (256 for the
// rotation kernels; 512 or 1024 inside a fused decode linear). A thread owns
// the groups row_group_of(tid) + q NT, q = 0, 1, ..., of 16 consecutive
// elements (at most
// kFastMaxGroups of them, K <= 16384); all of its global loads are issued
// before any group is transformed, so a long row costs one memory latency
// rather than one per group.
//  - stages 0..3 (strides 1..8) inside a group, in registers;
//  - stages 4..7 (strides 16..128 = groups 1, 2, 4, 8 apart = lanes 1, 2,
//    7, 8 apart with the layout of row_group_of) between lanes with DPP
//    (lane_butterfly8; values kept up to a per-lane sign sigma);
//  - blocks up to 256: the row never goes through LDS; absmax and
//    quantization work on the registers;
//  - larger blocks: the values (up to sigma) go to a padded LDS row, stages
//    8..11 run in one pass through it, and the quantization reads the row
//    back.
constexpr int kFastMaxGroups = 4;
static_assert(kFastMaxGroups * 16 * kRowThreads >= QIFT_MAX_ROW, "fast path covers QIFT_MAX_ROW");

// rows with log2(block) <= kRegLog2B need no LDS row buffer
constexpr int kRegLog2B = 8;

// The group of 16 elements that lane position t of a row holds (q = 0):
// within each run of 16 lanes, lanes with bit 2 set hold the groups with
// their two low index bits inverted (g = t ^ 3 there, else t; a change of
// basis of the index bits over GF(2), its own inverse). The partner groups
// of the lane stages, g ^ 1, g ^ 2, g ^ 4 and g ^ 8, then sit in lanes t ^ 1,
// t ^ 2, t ^ 7 and t ^ 8, each of which one DPP operand reads (with the
// plain layout, g ^ 4 in lane t ^ 4 took two DPP moves).
__device__ __forceinline__ int row_group_of(int t) { return t ^ (((t >> 2) & 1) * 3); }

// groups of 16 elements a thread holds for a workgroup of NT threads: enough
// for the longest row (QIFT_MAX_ROW), or Q when the caller knows its rows
// are shorter (K <= 16 Q NT). The registers are sized by it: at
// K = 4096 one group per thread keeps a 256-thread rotation at about 40
// VGPRs, so all eight of its workgroups per CU are resident at once (four
// groups need about 110 and allow half of them).
template <int NT>
struct RowGroups {
  static constexpr int kQ = (kFastMaxGroups * kRowThreads + NT - 1) / NT;
};

// 1. loads (a group past the row end reads group 0 and is discarded), as raw
// words; rotate_row_finish widens and transforms them
template <typename T, int NT, int Q = RowGroups<NT>::kQ>
__device__ __forceinline__ void rotate_row_load(const T* __restrict__ src, int K,
                                                uint32_t raw[Q][16]) {
  const int tg = row_group_of(threadIdx.x);
  const int groups = K >> 4;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int grp = tg + q * NT;
    load16_raw<T>(src + 16 * (grp < groups ? grp : 0), raw[q]);
  }
}

template <typename T, int NT, int Q = RowGroups<NT>::kQ>
__device__ __forceinline__ void rotate_row_finish(const uint32_t raw[Q][16],
                                                  int K, int log2b, float norm,
                                                  uint8_t* __restrict__ xq_row,
                                                  float* __restrict__ s_out,
                                                  float* __restrict__ xrot_row, float* row,
                                                  float* red) {
  constexpr int kQ = Q;  // groups per thread
  float v[kQ][16];
#pragma unroll
  for (int q = 0; q < kQ; ++q) widen16<T>(raw[q], v[q]);
  const bool in_regs = log2b <= kRegLog2B;
  const int tid = threadIdx.x;
  const int tg = row_group_of(tid);  // this thread's group for q = 0
  const int groups = K >> 4;
  const int wave_g0 = tid & ~63;  // the wave's first group (q = 0)
  // 2. stages 0..3 in registers (rounds with no group of this wave skipped;
  //    a partner group of a valid group is always valid, since K is a
  //    multiple of the block)
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (wave_g0 + q * NT < groups) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int h = 1 << st;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (!(j & h)) {
            const float a = v[q][j], b = v[q][j + h];
            v[q][j] = a + b;
            v[q][j + h] = a - b;
          }
        }
      }
    }
  }
  // 3. stages 4..7 between lanes: group index bit H, partner in lane ^ M
  //    (row_group_of); the upper group of a pair (bit H set) flips its sign
  float sigma = 1.f;
  const int lane_stages = min(log2b, kRegLog2B) - 4;
#define QIFT_LANE_STAGE(H, M)                                              \
  {                                                                        \
    const float c = (tg & (H)) ? -1.f : 1.f;                               \
    _Pragma("unroll") for (int q = 0; q < kQ; ++q) {                      \
      if (wave_g0 + q * NT < groups) {                                     \
        lane_butterfly8<M>(v[q], c);                                       \
        lane_butterfly8<M>(v[q] + 8, c);                                   \
      }                                                                    \
    }                                                                      \
    sigma *= c;                                                            \
  }
  if (lane_stages >= 1) QIFT_LANE_STAGE(1, 1)
  if (lane_stages >= 2) QIFT_LANE_STAGE(2, 2)
  if (lane_stages >= 3) QIFT_LANE_STAGE(4, 7)
  if (lane_stages >= 4) QIFT_LANE_STAGE(8, 8)
#undef QIFT_LANE_STAGE
  float mloc = 0.f;  // largest |value| of the row's last stage seen by this thread
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (tg + q * NT < groups) {
#pragma unroll
        for (int j = 0; j < 16; ++j) mloc = fmaxf(mloc, fabsf(v[q][j]));
      }
    }
  } else {
    // 4. stages 8.. in one pass through the padded LDS row. The values go in
    //    up to their sign sigma, which depends only on the low four bits of
    //    the group index (the lane bits of stages 4-7; NT is a multiple of
    //    16). A thread of the pass combines elements 256 apart, i.e. groups
    //    16 apart, which share those bits and so sigma: the pass's sums are
    //    the true ones times that common sigma, and every group comes back
    //    with the sigma it went in with, which the quantizer folds into its
    //    reciprocal as in the register path (16 fewer multiplies a group).
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int grp = tg + q * NT;
      if (grp < groups) {
        float* dst = row + 17 * grp;
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[j] = v[q][j];
      }
    }
    lds_barrier();
    switch (log2b - 8) {
      case 1: fwht_pass_padded<1, true, NT>(row, K, 2, tid, &mloc); break;
      case 2: fwht_pass_padded<2, true, NT>(row, K, 2, tid, &mloc); break;
      case 3: fwht_pass_padded<3, true, NT>(row, K, 2, tid, &mloc); break;
      default: fwht_pass_padded<4, true, NT>(row, K, 2, tid, &mloc); break;
    }
  }
  // 5. row absmax (for the LDS path the barrier also completes the pass)
  mloc *= norm;  // rounding is monotonic: max(|v|)*norm == max(|v*norm|)
  mloc = wave_max_nonneg(mloc);
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  lds_barrier();
  float amax = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) amax = fmaxf(amax, red[w]);
  const float s = __fdiv_rn(amax, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  const bool fast = rint_path_ok(rs);
  if (tid == 0) *s_out = s;
  // 6. quantize 16 consecutive elements per group: x = the rotated value up
  //    to sigma (on both paths), y = x * sigma / s
  const float sg = sigma;
  // v * sg * (norm / s) is within three roundings of x' / s with
  // x' = fl(v * norm) the rotated value (int4x8_rint_fma's margin covers it)
  const float rl = sg * (norm * rs);
  uint2* xrow = reinterpret_cast<uint2*>(xq_row);
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int grp = tg + q * NT;
    if (grp >= groups) continue;
    float x[16];  // x: the stored values (up to sg), then the rotated ones
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = v[q][j];
    } else {
      const float* s16 = row + 17 * grp;
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = s16[j];
    }
    // codes of x * rl, each product rounded once inside the adder
    float dmax = 0.f;
    uint32_t w0 = int4x8_rint_fma(x, rl, dmax);
    uint32_t w1 = int4x8_rint_fma(x + 8, rl, dmax);
    if (!(dmax <= 0.49999f) || !fast || xrot_row) {
      // the true rotated values fl(v * norm); fma(., sg, +0) also writes
      // every zero as +0 (an upper lane's x - x comes back as -0 through its
      // sign)
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(x[j] * norm, sg, 0.0f);
      if (!(dmax <= 0.49999f) || !fast) {  // a value near a rounding tie: exact division
        w0 = int4x8_exact(x, s);
        w1 = int4x8_exact(x + 8, s);
      }
      if (xrot_row) {
        float4* xr = reinterpret_cast<float4*>(xrot_row + 16 * grp);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xr[i] = float4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
      }
    }
    xrow[grp] = uint2{w0, w1};
  }
}

template <typename T, int NT = kRowThreads, int Q = RowGroups<NT>::kQ>
__device__ __forceinline__ void rotate_row_fast(const T* __restrict__ src, int K, int log2b,
                                                float norm, uint8_t* __restrict__ xq_row,
                                                float* __restrict__ s_out,
                                                float* __restrict__ xrot_row, float* row,
                                                float* red) {
  uint32_t raw[Q][16];
  rotate_row_load<T, NT, Q>(src, K, raw);
  rotate_row_finish<T, NT, Q>(raw, K, log2b, norm, xq_row, s_out, xrot_row, row, red);
}

}  // namespace qift
