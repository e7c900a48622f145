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
// a group and stages 4-7 between the lanes holding neighbouring groups
// (rotate_row_fast below), so rows with blocks up to 256 never touch LDS.
// For larger blocks the row is staged in LDS with one pad word per 16 floats
// (element e at e + e / 16): the 16 stores of a thread hit 16 consecutive
// banks and neighbouring threads are 17 words apart, so a wave's stores, the
// stride-256 pass of stages 8-11 and the final consecutive reads are all
// conflict-free.

__device__ __forceinline__ int pad16(int e) { return e + (e >> 4); }

// kMax: also raise m to the largest |value| the pass writes
template <int NS, bool kMax = false>
__device__ __forceinline__ void fwht_pass_padded(float* row, int K, int p, int tid,
                                                 float* m = nullptr) {
  constexpr int R = 1 << NS;
  const int sh = 4 * p;
  const int S = 1 << sh;
  const int groups = K >> NS;
  for (int grp = tid; grp < groups; grp += kRowThreads) {
    const int low = grp & (S - 1);
    const int high = grp >> sh;
    const int base = (high << (sh + NS)) | low;
    float v[R];
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = row[pad16(base + j * S)];
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
    for (int j = 0; j < R; ++j) row[pad16(base + j * S)] = v[j];
    if constexpr (kMax) {
#pragma unroll
      for (int j = 0; j < R; ++j) *m = fmaxf(*m, fabsf(v[j]));
    }
  }
}

template <typename T>
__device__ __forceinline__ void load16(const T* __restrict__ src, float v[16]);

template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t* __restrict__ src, float v[16]) {
  const uint4 a = reinterpret_cast<const uint4*>(src)[0];
  const uint4 b = reinterpret_cast<const uint4*>(src)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load16<float>(const float* __restrict__ src, float v[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = reinterpret_cast<const float4*>(src)[i];
    v[4 * i] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
}

// One row on the fast path. A thread owns the groups tid, tid + 256, ... of
// 16 consecutive elements (at most kFastMaxGroups of them, K <= 16384); all
// of its global loads are issued before any group is transformed, so a long
// row costs one memory latency rather than one per group.
//  - stages 0..3 (strides 1..8) inside a group, in registers;
//  - stages 4..7 (strides 16..128 = groups 1..8 apart = lanes 1..8 apart)
//    between lanes with DPP (lane_butterfly8; values kept up to a per-lane
//    sign sigma);
//  - blocks up to 256: the row never goes through LDS; absmax and
//    quantization work on the registers;
//  - larger blocks: the true values go to a padded LDS row, stages 8..11 run
//    in one pass through it, and the quantization reads the row back.
constexpr int kFastMaxGroups = 4;
static_assert(kFastMaxGroups * 16 * kRowThreads >= QIFT_MAX_ROW, "fast path covers QIFT_MAX_ROW");

// rows with log2(block) <= kRegLog2B need no LDS row buffer
constexpr int kRegLog2B = 8;

template <typename T>
__device__ __forceinline__ void rotate_row_fast(const T* __restrict__ src, int K, int log2b,
                                                float norm, uint8_t* __restrict__ xq_row,
                                                float* __restrict__ s_out,
                                                float* __restrict__ xrot_row, float* row,
                                                float* red) {
  const bool in_regs = log2b <= kRegLog2B;
  const int tid = threadIdx.x;
  const int groups = K >> 4;
  const int wave_g0 = tid & ~63;  // the wave's first group (q = 0)
  // 1. loads (a group past the row end reads group 0 and is discarded)
  float v[kFastMaxGroups][16];
#pragma unroll
  for (int q = 0; q < kFastMaxGroups; ++q) {
    const int grp = tid + q * kRowThreads;
    load16<T>(src + 16 * (grp < groups ? grp : 0), v[q]);
  }
  // 2. stages 0..3 in registers (rounds with no group of this wave skipped;
  //    a partner group of a valid group is always valid, since K is a
  //    multiple of the block)
#pragma unroll
  for (int q = 0; q < kFastMaxGroups; ++q) {
    if (wave_g0 + q * kRowThreads < groups) {
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
  // 3. stages 4..7 between lanes
  float sigma = 1.f;
  const int lane_stages = min(log2b, kRegLog2B) - 4;
#define QIFT_LANE_STAGE(H)                                                 \
  {                                                                        \
    const float c = (tid & (H)) ? -1.f : 1.f;                              \
    _Pragma("unroll") for (int q = 0; q < kFastMaxGroups; ++q) {           \
      if (wave_g0 + q * kRowThreads < groups) {                            \
        lane_butterfly8<H>(v[q], c);                                       \
        lane_butterfly8<H>(v[q] + 8, c);                                   \
      }                                                                    \
    }                                                                      \
    sigma *= c;                                                            \
  }
  if (lane_stages >= 1) QIFT_LANE_STAGE(1)
  if (lane_stages >= 2) QIFT_LANE_STAGE(2)
  if (lane_stages >= 3) QIFT_LANE_STAGE(4)
  if (lane_stages >= 4) QIFT_LANE_STAGE(8)
#undef QIFT_LANE_STAGE
  float mloc = 0.f;  // largest |value| of the row's last stage seen by this thread
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < kFastMaxGroups; ++q) {
      if (tid + q * kRowThreads < groups) {
#pragma unroll
        for (int j = 0; j < 16; ++j) mloc = fmaxf(mloc, fabsf(v[q][j]));
      }
    }
  } else {
    // 4. stages 8.. in one pass through the padded LDS row
#pragma unroll
    for (int q = 0; q < kFastMaxGroups; ++q) {
      const int grp = tid + q * kRowThreads;
      if (grp < groups) {
        float* dst = row + 17 * grp;
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[j] = sigma * v[q][j];
      }
    }
    __syncthreads();
    switch (log2b - 8) {
      case 1: fwht_pass_padded<1, true>(row, K, 2, tid, &mloc); break;
      case 2: fwht_pass_padded<2, true>(row, K, 2, tid, &mloc); break;
      case 3: fwht_pass_padded<3, true>(row, K, 2, tid, &mloc); break;
      default: fwht_pass_padded<4, true>(row, K, 2, tid, &mloc); break;
    }
  }
  // 5. row absmax (for the LDS path the barrier also completes the pass)
  mloc *= norm;  // rounding is monotonic: max(|v|)*norm == max(|v*norm|)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mloc;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) amax = fmaxf(amax, red[w]);
  const float s = __fdiv_rn(amax, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  const bool fast = rint_path_ok(rs);
  if (tid == 0) *s_out = s;
  // 6. quantize 16 consecutive elements per group: x = the rotated value up
  //    to sigma (sigma = 1 on the LDS path), y = x * sigma / s
  const float sg = in_regs ? sigma : 1.f;
  // y = v * sg * (norm / s): within four roundings of x' / s with
  // x' = fl(v * norm) the rotated value (int4x8_rint's margin covers it)
  const float rl = sg * (norm * rs);
  uint2* xrow = reinterpret_cast<uint2*>(xq_row);
#pragma unroll
  for (int q = 0; q < kFastMaxGroups; ++q) {
    const int grp = tid + q * kRowThreads;
    if (grp >= groups) continue;
    float x[16], y[16];  // x: the stored values (up to sg), then the rotated ones
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = v[q][j];
    } else {
      const float* s16 = row + 17 * grp;
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = s16[j];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = x[j] * rl;
    float dmax = 0.f;
    uint32_t w0 = int4x8_rint(y, dmax);
    uint32_t w1 = int4x8_rint(y + 8, dmax);
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

}  // namespace qift
