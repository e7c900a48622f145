// Row kernels of the rotated quantization pipeline:
//  - rotate_quant_act: online activation path (block Walsh-Hadamard rotation
//    along K, per-token absmax, symmetric int4, packed);
//  - quantize_weights: offline weight path (same rotation, per-channel absmax
//    scale, nearest no-zero level, packed 2-bit codes; or int4 weights).
// Source of the method: "Qift: Shift-Friendly No-Zero W2 Post-Training
// Quantization for Rotated W2A4/KV4 LLM Inference", abstract.
//
// One workgroup handles one row. The general kernels stage the row in LDS as
// float32 and run the butterflies in passes of up to four stages, each pass
// keeping 16 (or fewer) elements in registers; the activation fast path keeps
// the row in registers for the first eight stages (see below).
#include "weight_codes.h"

namespace qift {


// --- staged row load: X[row] -> LDS float32 --------------------------------

template <typename T>
__device__ __forceinline__ void load_row(const T* __restrict__ src, float* row, int K, int tid);

template <>
__device__ __forceinline__ void load_row<float>(const float* __restrict__ src, float* row, int K,
                                                int tid) {
  if ((K & 3) == 0 && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
    float4* r4 = reinterpret_cast<float4*>(row);
    for (int i = tid; i < (K >> 2); i += kRowThreads) r4[i] = s4[i];
  } else {
    for (int i = tid; i < K; i += kRowThreads) row[i] = src[i];
  }
}

template <>
__device__ __forceinline__ void load_row<uint16_t>(const uint16_t* __restrict__ src, float* row,
                                                   int K, int tid) {
  if ((K & 7) == 0 && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
    const uint4* s8 = reinterpret_cast<const uint4*>(src);
    for (int i = tid; i < (K >> 3); i += kRowThreads) {
      uint4 u = s8[i];
      float4 lo, hi;
      lo.x = __uint_as_float(u.x << 16);
      lo.y = __uint_as_float(u.x & 0xffff0000u);
      lo.z = __uint_as_float(u.y << 16);
      lo.w = __uint_as_float(u.y & 0xffff0000u);
      hi.x = __uint_as_float(u.z << 16);
      hi.y = __uint_as_float(u.z & 0xffff0000u);
      hi.z = __uint_as_float(u.w << 16);
      hi.w = __uint_as_float(u.w & 0xffff0000u);
      reinterpret_cast<float4*>(row)[2 * i] = lo;
      reinterpret_cast<float4*>(row)[2 * i + 1] = hi;
    }
  } else {
    for (int i = tid; i < K; i += kRowThreads) row[i] = bf16_bits_to_float(src[i]);
  }
}

// --- butterflies --------------------------------------------------------------

// One pass: stages 4p .. 4p+NS-1 of every Hadamard block of the row. Element
// index bits [4p, 4p+NS) select the 2^NS elements a thread holds; they all
// lie in the same block because 4p+NS <= log2(block).
template <int NS>
__device__ __forceinline__ void fwht_pass(float* row, int K, int p, int tid) {
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
    for (int j = 0; j < R; ++j) v[j] = row[base + j * S];
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
    for (int j = 0; j < R; ++j) row[base + j * S] = v[j];
  }
}

// Unnormalized block transform of the LDS row; log2b = log2(block).
__device__ __forceinline__ void fwht_row(float* row, int K, int log2b, int tid) {
  for (int p = 0; 4 * p < log2b; ++p) {
    const int ns = min(4, log2b - 4 * p);
    switch (ns) {
      case 1: fwht_pass<1>(row, K, p, tid); break;
      case 2: fwht_pass<2>(row, K, p, tid); break;
      case 3: fwht_pass<3>(row, K, p, tid); break;
      default: fwht_pass<4>(row, K, p, tid); break;
    }
    __syncthreads();
  }
}

// --- K1: rotate + per-token int4 ---------------------------------------------

template <typename T>
__global__ __launch_bounds__(kRowThreads) void rotate_quant_act_kernel(
    const T* __restrict__ X, int K, int log2b, float norm, uint8_t* __restrict__ xq,
    float* __restrict__ s_a, float* __restrict__ x_rot) {
  extern __shared__ float row[];
  __shared__ float red[kRowThreads / 64];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  load_row<T>(X + m * K, row, K, tid);
  __syncthreads();
  fwht_row(row, K, log2b, tid);
  const float amax = row_absmax(row, K, norm, tid, red);
  const float s = __fdiv_rn(amax, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  if (tid == 0) s_a[m] = s;
  uint8_t* xq_row = xq + m * (int64_t)(K / 2);
  if ((K & 7) == 0) {
    uint32_t* w_row = reinterpret_cast<uint32_t*>(xq_row);
    for (int g = tid; g < (K >> 3); g += kRowThreads) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = row[8 * g + i] * norm;
        word |= code_int4_recip(x, s, rs) << (4 * i);
        if (x_rot) x_rot[m * K + 8 * g + i] = x;
      }
      w_row[g] = word;
    }
  } else {
    for (int j = tid; j < (K >> 1); j += kRowThreads) {
      const float x0 = row[2 * j] * norm, x1 = row[2 * j + 1] * norm;
      xq_row[j] = (uint8_t)(code_int4_recip(x0, s, rs) | (code_int4_recip(x1, s, rs) << 4));
      if (x_rot) {
        x_rot[m * K + 2 * j] = x0;
        x_rot[m * K + 2 * j + 1] = x1;
      }
    }
  }
}

// The fast path (rotate_row_fast) lives in rotate_row.h.

template <typename T>
__global__ __launch_bounds__(kRowThreads) void rotate_quant_act_fast_kernel(
    const T* __restrict__ X, int K, int log2b, float norm, uint8_t* __restrict__ xq,
    float* __restrict__ s_a, float* __restrict__ x_rot) {
  extern __shared__ float row[];
  __shared__ float red[kRowThreads / 64];
  const int64_t m = blockIdx.x;
  rotate_row_fast<T>(X + m * K, K, log2b, norm, xq + m * (int64_t)(K / 2), s_a + m,
                     x_rot ? x_rot + m * K : nullptr, row, red);
}

// Several activation matrices in one launch (workgroup b covers row b of the
// concatenation of their rows), e.g. the inputs of all linears of a decode
// step, which are too small to fill the chip one at a time.
struct RotBatch {
  RotJob job[QIFT_MAX_ROTATE_BATCH];
  int64_t row_begin[QIFT_MAX_ROTATE_BATCH + 1];
  int count;
};

__global__ __launch_bounds__(kRowThreads) void rotate_quant_act_batched_kernel(RotBatch bt) {
  extern __shared__ float row[];
  __shared__ float red[kRowThreads / 64];
  const int64_t b = blockIdx.x;
  int j = 0;
#pragma unroll
  for (int k = 1; k < QIFT_MAX_ROTATE_BATCH; ++k)
    if (k < bt.count && b >= bt.row_begin[k]) j = k;
  const RotJob& jb = bt.job[j];
  const int64_t m = b - bt.row_begin[j];
  const int K = jb.K;
  uint8_t* xq_row = jb.xq + m * (int64_t)(K / 2);
  float* xr = jb.x_rot ? jb.x_rot + m * K : nullptr;
  if (jb.bf16)
    rotate_row_fast<uint16_t>(reinterpret_cast<const uint16_t*>(jb.X) + m * K, K, jb.log2b,
                              jb.norm, xq_row, jb.s_a + m, xr, row, red);
  else
    rotate_row_fast<float>(reinterpret_cast<const float*>(jb.X) + m * K, K, jb.log2b, jb.norm,
                           xq_row, jb.s_a + m, xr, row, red);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void quantize_weights_kernel(
    const T* __restrict__ W, int64_t N, int K, int log2b, float norm, int levels, uint32_t table,
    uint32_t pref, float outer, int mse_rule, uint32_t* __restrict__ codes,
    void* __restrict__ scales, int scale_f16) {
  extern __shared__ float row[];
  __shared__ float red[kRowThreads / 64];
  __shared__ double red64[kRowThreads / 64];
  const int tid = threadIdx.x;
  const int64_t n = blockIdx.x;
  const bool int4 = levels == QIFT_LEVELS_INT4;
  const int64_t words = int4 ? K / 8 : K / 16;
  const int64_t tiles = (N + 15) >> 4;
  if (n >= N) {  // zero codes for the padding channels of the last tile
    for (int w = tid; w < words; w += kRowThreads) codes[tiled_word(n, w, words, tiles)] = 0u;
    return;
  }
  load_row<T>(W + n * K, row, K, tid);
  __syncthreads();
  fwht_row(row, K, log2b, tid);
  const float s32 =
      choose_scale(row, K, norm, levels, table, pref, outer, mse_rule, scale_f16, red, red64);
  const float s = stored_scale(s32, scale_f16);
  if (tid == 0) {
    if (scale_f16)
      reinterpret_cast<__half*>(scales)[n] = __float2half_rn(s32);
    else
      reinterpret_cast<float*>(scales)[n] = s32;
  }
  if (int4) {
    for (int g = tid; g < (K >> 3); g += kRowThreads) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        word |= ((uint32_t)quant_int4(row[8 * g + i] * norm, s) & 0xFu) << (4 * i);
      codes[tiled_word(n, g, words, tiles)] = word;
    }
  } else {
    for (int g = tid; g < (K >> 4); g += kRowThreads) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float w = row[16 * g + i] * norm;
        word |= code2(levels, w, s, table, pref) << code_bit_offset(i);
      }
      codes[tiled_word(n, g, words, tiles)] = word;
    }
  }
}

// --- launchers -----------------------------------------------------------------

static int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

// 1/sqrt(B) rounded once to float32 (exact for even log2 B).
static float had_norm(int B) { return (float)(1.0 / __builtin_sqrt((double)B)); }

hipError_t launch_rotate_quant_act(const void* X, int x_bf16, int64_t M, int64_t K, int had_block,
                                   uint8_t* xq, float* s_a, float* x_rot, hipStream_t s) {
  const int lb = ilog2(had_block);
  const float nrm = had_norm(had_block);
  if (rotate_fast_ok(X, K, had_block, xq, x_rot)) {
    const size_t lds = lb > kRegLog2B ? (size_t)(K + K / 16) * sizeof(float) : 0;
    if (x_bf16)
      hipLaunchKernelGGL(rotate_quant_act_fast_kernel<uint16_t>, dim3((unsigned)M),
                         dim3(kRowThreads), lds, s, reinterpret_cast<const uint16_t*>(X), (int)K,
                         lb, nrm, xq, s_a, x_rot);
    else
      hipLaunchKernelGGL(rotate_quant_act_fast_kernel<float>, dim3((unsigned)M), dim3(kRowThreads),
                         lds, s, reinterpret_cast<const float*>(X), (int)K, lb, nrm, xq, s_a, x_rot);
    return hipGetLastError();
  }
  const size_t lds = (size_t)K * sizeof(float);
  if (x_bf16)
    hipLaunchKernelGGL(rotate_quant_act_kernel<uint16_t>, dim3((unsigned)M), dim3(kRowThreads),
                       lds, s, reinterpret_cast<const uint16_t*>(X), (int)K, lb, nrm, xq, s_a,
                       x_rot);
  else
    hipLaunchKernelGGL(rotate_quant_act_kernel<float>, dim3((unsigned)M), dim3(kRowThreads), lds,
                       s, reinterpret_cast<const float*>(X), (int)K, lb, nrm, xq, s_a, x_rot);
  return hipGetLastError();
}

bool rotate_fast_ok(const void* X, int64_t K, int had_block, const uint8_t* xq,
                    const float* x_rot) {
  const uintptr_t align = reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(xq) |
                          reinterpret_cast<uintptr_t>(x_rot);
  return K % 16 == 0 && had_block >= 16 && (align & 15) == 0;
}

hipError_t launch_rotate_quant_act_batched(const RotJob* jobs, const int64_t* rows, int count,
                                           hipStream_t s) {
  RotBatch bt{};
  bt.count = count;
  int64_t total = 0;
  int64_t kmax = 0;
  for (int j = 0; j < count; ++j) {
    bt.job[j] = jobs[j];
    bt.job[j].log2b = ilog2(jobs[j].had_block);
    bt.job[j].norm = had_norm(jobs[j].had_block);
    bt.row_begin[j] = total;
    total += rows[j];
    if (bt.job[j].log2b > kRegLog2B && rows[j] > 0) kmax = jobs[j].K > kmax ? jobs[j].K : kmax;
  }
  for (int j = count; j <= QIFT_MAX_ROTATE_BATCH; ++j) bt.row_begin[j] = total;
  if (total == 0) return hipSuccess;
  const size_t lds = (size_t)(kmax + kmax / 16) * sizeof(float);
  hipLaunchKernelGGL(rotate_quant_act_batched_kernel, dim3((unsigned)total), dim3(kRowThreads),
                     lds, s, bt);
  return hipGetLastError();
}

hipError_t launch_quantize_weights(const void* W, int w_bf16, int64_t N, int64_t K, int had_block,
                                   int levels, uint32_t table, int mse_rule, uint32_t* codes,
                                   void* scales, int scale_f16, hipStream_t s) {
  const size_t lds = (size_t)K * sizeof(float);
  const int lb = ilog2(had_block);
  const float nrm = had_norm(had_block);
  const unsigned grid = (unsigned)((N + 15) / 16 * 16);  // padded to whole 16-channel tiles
  uint32_t pref = 0;
  const float outer = level_outer_and_pref(levels, table, &pref);
  if (w_bf16)
    hipLaunchKernelGGL(quantize_weights_kernel<uint16_t>, dim3(grid), dim3(kRowThreads), lds, s,
                       reinterpret_cast<const uint16_t*>(W), N, (int)K, lb, nrm, levels, table,
                       pref, outer, mse_rule, codes, scales, scale_f16);
  else
    hipLaunchKernelGGL(quantize_weights_kernel<float>, dim3(grid), dim3(kRowThreads), lds, s,
                       reinterpret_cast<const float*>(W), N, (int)K, lb, nrm, levels, table, pref,
                       outer, mse_rule, codes, scales, scale_f16);
  return hipGetLastError();
}

}  // namespace qift
