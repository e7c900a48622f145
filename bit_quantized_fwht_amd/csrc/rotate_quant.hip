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

// The fast path (rotate_row_fast) lives in rotate_row.h. Q: groups of 16
// elements per thread, the fewest that cover the row (K <= 4096 Q), which
// sizes the registers and so the number of resident workgroups.

template <typename T, int Q>
__global__ __launch_bounds__(kRowThreads) void rotate_quant_act_fast_kernel(
    const T* __restrict__ X, int K, int log2b, float norm, uint8_t* __restrict__ xq,
    float* __restrict__ s_a, float* __restrict__ x_rot) {
  extern __shared__ float row[];
  __shared__ float red[kRowThreads / 64];
  const int64_t m = blockIdx.x;
  rotate_row_fast<T, kRowThreads, Q>(X + m * K, K, log2b, norm, xq + m * (int64_t)(K / 2),
                                     s_a + m, x_rot ? x_rot + m * K : nullptr, row, red);
}

// Rows of K = 4096 bfloat16 values with one block of 4096: the first five
// butterfly stages on the matrix cores. For element e = 32 c + k (chunk c,
// k < 32) the Hadamard sign (-1)^popcount(i & e) splits over (c, k), so H_4096
// = H_128 (x) H_32: one v_mfma_f32_16x16x32_bf16 applies H_32 to 16 chunks at
// once, straight from the loaded bfloat16 words (entries +-1: exact products,
// summed in float32), which replaces the widening and the five stages of
// strides 1 .. 16 (six of about 24 vector instructions per element). The
// operand A rows are permuted as for the KV4 matrix-core kernel
// (h32_operand_bf16), so lane (t = lane % 16, g = lane / 16) receives the
// outputs 8 g .. 8 g + 7 of the chunk in column t. The seven stages across
// chunks follow:
//  - chunk bits 0-3 between the lanes of a 16-lane row with DPP
//    (lane_butterfly8, values kept up to a sign sigma); the chunk of column t
//    is 32 w + 16 a + row_group_of(t) (wave w, tile a), so the partners sit at
//    lane ^ 1, ^ 2, ^ 7, ^ 8;
//  - chunk bit 4 (the wave's two tiles) in registers;
//  - chunk bits 5, 6 (the four waves) in one pass through a padded LDS row
//    (element e at e + 4 (e / 32)): thread T combines the runs of four
//    elements at 4 T + 1024 j, j = 0..3, whose chunks share bits 0-3 and so
//    sigma = (-1)^popcount(chunk & 15).
// Each thread then quantizes its four runs (16 bits of codes each); absmax,
// scale, codes and the near-tie fallback are the arithmetic of the other
// rotation kernels.
constexpr int kMfmaRowK = 4096;
constexpr int kMfmaRowLds = kMfmaRowK + kMfmaRowK / 8;  // floats, with the pad

__global__ __launch_bounds__(kRowThreads) void rotate_quant_act_mfma4096_kernel(
    const uint16_t* __restrict__ X, float norm, uint8_t* __restrict__ xq,
    float* __restrict__ s_a, float* __restrict__ x_rot) {
  __shared__ __attribute__((aligned(16))) float row[kMfmaRowLds];
  __shared__ float red[kRowThreads / 64];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int t = lane & 15, g = lane >> 4;
  const uint16_t* __restrict__ src = X + m * kMfmaRowK;
  // operand B of tile a: elements 8 g .. 8 g + 7 of chunk c[a] (16 bytes)
  const int rg = row_group_of(t);
  int c[2];
  v4u xb[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    c[a] = 32 * w + 16 * a + rg;
    xb[a] = *reinterpret_cast<const v4u*>(src + 32 * c[a] + 8 * g);
  }
  v4u ha[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) ha[h] = h32_operand_bf16(4 * h + (t & 3), (t >> 2) & g);
  // v[a][j]: output 32 c[a] + 8 g + j, unnormalized
  float v[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xb[a]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4f y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, ha[h]), b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[a][4 * h + i] = y[i];
    }
  }
  // chunk bits 0-3 between lanes (upper lane of a pair: c = -1)
#define QIFT_MFMA_ROW_STAGE(H, M)                         {                                                         const float cs = (rg & (H)) ? -1.f : 1.f;               lane_butterfly8<M>(v[0], cs);                           lane_butterfly8<M>(v[1], cs);                         }
  QIFT_MFMA_ROW_STAGE(1, 1)
  QIFT_MFMA_ROW_STAGE(2, 2)
  QIFT_MFMA_ROW_STAGE(4, 7)
  QIFT_MFMA_ROW_STAGE(8, 8)
#undef QIFT_MFMA_ROW_STAGE
  // chunk bit 4: the two tiles
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = v[0][j], q = v[1][j];
    v[0][j] = p + q;
    v[1][j] = p - q;
  }
  // chunk bits 5, 6 through LDS
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float* dst = row + 36 * c[a] + 8 * g;
    *reinterpret_cast<float4*>(dst) = float4{v[a][0], v[a][1], v[a][2], v[a][3]};
    *reinterpret_cast<float4*>(dst + 4) = float4{v[a][4], v[a][5], v[a][6], v[a][7]};
  }
  lds_barrier();
  float x[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + 1024 * j;
    const float4 f = *reinterpret_cast<const float4*>(row + e + 4 * (e >> 5));
    x[j][0] = f.x; x[j][1] = f.y; x[j][2] = f.z; x[j][3] = f.w;
  }
#pragma unroll
  for (int h = 1; h < 4; h <<= 1)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (!(j & h)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = x[j][i], q = x[j + h][i];
          x[j][i] = p + q;
          x[j + h][i] = p - q;
        }
      }
  float mloc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, fabsf(x[j][i]));
  mloc *= norm;  // rounding is monotonic: max(|v|)*norm == max(|v*norm|)
  mloc = wave_max_nonneg(mloc);
  if (lane == 0) red[w] = mloc;
  lds_barrier();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  const bool fast = rint_path_ok(rs);
  if (tid == 0) s_a[m] = s;
  // sigma of this thread's chunks (tid / 8 + 32 j: bits 0-3 = (tid / 8) & 15)
  const float sg = (__builtin_popcount((tid >> 3) & 15) & 1) ? -1.f : 1.f;
  const float rl = sg * (norm * rs);
  uint16_t* xrow = reinterpret_cast<uint16_t*>(xq + m * (kMfmaRowK / 2));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float dmax = 0.f;
    uint32_t code = int4x4_rint_fma(x[j], rl, dmax);
    const int e = 4 * tid + 1024 * j;
    if (!(dmax <= 0.49999f) || !fast || x_rot) {
      float xr[4];  // the true rotated values; fma(., sg, +0) writes zeros as +0
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = __builtin_fmaf(x[j][i] * norm, sg, 0.0f);
      if (!(dmax <= 0.49999f) || !fast) code = int4x4_exact(xr, s);
      if (x_rot)
        *reinterpret_cast<float4*>(x_rot + m * kMfmaRowK + e) = float4{xr[0], xr[1], xr[2], xr[3]};
    }
    xrow[e / 4] = (uint16_t)code;
  }
}

// Rows of bfloat16 values with a block of 2^LB = 256, 512 or 1024 elements
// (any K that is a multiple of the block, up to QIFT_MAX_ROW): the same
// matrix-core split, with the whole block inside one wave's two tiles of 16
// chunks, so no stage goes through LDS. The row is cut into groups of 32
// chunks (1024 elements); wave w takes groups w, w + 4, ... (at most P).
// Lane (t, g) holds, for group p and tile a, the outputs 8 g .. 8 g + 7 of
// chunk 32 p + 16 a + row_group_of(t): after H_32 on the matrix cores, chunk
// bits 0 .. LB - 6 (at most 3) run between lanes by DPP and, for a block of
// 1024, chunk bit 4 between the tiles in registers. The eight consecutive
// outputs a lane holds per chunk are one word of codes, stored as they are.
// Chunks past the row end (K % 1024 != 0: blocks of 256 or 512) are loaded
// from chunk 0 and never mix with valid ones: a row ends on a block
// boundary, and the stages of a 256-block stay inside a tile half (chunk
// bit 3 fixed), those of a 512-block inside a tile. They are neither counted
// in the absmax nor stored.
template <int LB, int P>
__global__ __launch_bounds__(kRowThreads) void rotate_quant_act_mfma_groups_kernel(
    const uint16_t* __restrict__ X, int K, float norm, uint8_t* __restrict__ xq,
    float* __restrict__ s_a, float* __restrict__ x_rot) {
  static_assert(LB >= 8 && LB <= 10, "blocks of 256, 512 or 1024 elements");
  __shared__ float red[kRowThreads / 64];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int t = lane & 15, g = lane >> 4;
  const int rg = row_group_of(t);
  const int nchunks = K >> 5;
  const uint16_t* __restrict__ src = X + m * K;
  int c[P][2];
  bool ok[P][2];
  v4u xb[P][2];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      c[p][a] = 32 * (w + 4 * p) + 16 * a + rg;
      ok[p][a] = c[p][a] < nchunks;
      xb[p][a] = *reinterpret_cast<const v4u*>(src + 32 * (ok[p][a] ? c[p][a] : 0) + 8 * g);
    }
  v4u ha[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) ha[h] = h32_operand_bf16(4 * h + (t & 3), (t >> 2) & g);
  // every group is transformed, past the row end too (on chunk 0's values,
  // never counted or stored): without a branch per group the compiler keeps
  // all loads at the top, one memory latency per row instead of one per group
  float v[P][2][8];
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xb[p][a]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4f y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, ha[h]), b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[p][a][4 * h + i] = y[i];
      }
    }
  }
  float sigma = 1.f;
#define QIFT_MFMA_GROUP_STAGE(H, MM)                     \
  {                                                      \
    const float cs = (rg & (H)) ? -1.f : 1.f;            \
    _Pragma("unroll") for (int p = 0; p < P; ++p) {      \
      lane_butterfly8<MM>(v[p][0], cs);                  \
      lane_butterfly8<MM>(v[p][1], cs);                  \
    }                                                    \
    sigma *= cs;                                         \
  }
  QIFT_MFMA_GROUP_STAGE(1, 1)
  QIFT_MFMA_GROUP_STAGE(2, 2)
  QIFT_MFMA_GROUP_STAGE(4, 7)
  if constexpr (LB >= 9) QIFT_MFMA_GROUP_STAGE(8, 8)
#undef QIFT_MFMA_GROUP_STAGE
  if constexpr (LB == 10) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x0 = v[p][0][j], x1 = v[p][1][j];
        v[p][0][j] = x0 + x1;
        v[p][1][j] = x0 - x1;
      }
    }
  }
  float mloc = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
      if (ok[p][a]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) mloc = fmaxf(mloc, fabsf(v[p][a][j]));
      }
  }
  mloc *= norm;  // rounding is monotonic: max(|v|)*norm == max(|v*norm|)
  mloc = wave_max_nonneg(mloc);
  if (lane == 0) red[w] = mloc;
  lds_barrier();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = __fdiv_rn(amax, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  const bool fast = rint_path_ok(rs);
  if (tid == 0) s_a[m] = s;
  const float rl = sigma * (norm * rs);
  uint32_t* xrow = reinterpret_cast<uint32_t*>(xq + m * (int64_t)(K / 2));
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      if (!ok[p][a]) continue;
      float dmax = 0.f;
      uint32_t code = int4x8_rint_fma(v[p][a], rl, dmax);
      const int e = 32 * c[p][a] + 8 * g;
      if (!(dmax <= 0.49999f) || !fast || x_rot) {
        float xr[8];  // the true rotated values; fma(., sigma, +0) writes zeros as +0
#pragma unroll
        for (int i = 0; i < 8; ++i) xr[i] = __builtin_fmaf(v[p][a][i] * norm, sigma, 0.0f);
        if (!(dmax <= 0.49999f) || !fast) code = int4x8_exact(xr, s);
        if (x_rot) {
          float4* xo = reinterpret_cast<float4*>(x_rot + m * K + e);
          xo[0] = float4{xr[0], xr[1], xr[2], xr[3]};
          xo[1] = float4{xr[4], xr[5], xr[6], xr[7]};
        }
      }
      xrow[e / 8] = code;
    }
  }
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
  if (levels == QIFT_LEVELS_ASYM) {
    // the conventional min-max grid with a zero point: step (hi - lo) / 3 of
    // the range widened to contain 0, zero point rint(-lo / s) in [0, 3]
    // (both with the stored step), stored after the N steps
    float lo, hi;
    row_range0(row, K, norm, tid, red, lo, hi);
    const float s32 = __fdiv_rn(__fsub_rn(hi, lo), 3.f);
    const float s = stored_scale(s32, scale_f16);
    const float z = s == 0.f ? 0.f : fminf(fmaxf(rintf(__fdiv_rn(-lo, s)), 0.f), 3.f);
    if (tid == 0) {
      if (scale_f16) {
        reinterpret_cast<__half*>(scales)[n] = __float2half_rn(s32);
        reinterpret_cast<__half*>(scales)[N + n] = __float2half_rn(z);
      } else {
        reinterpret_cast<float*>(scales)[n] = s32;
        reinterpret_cast<float*>(scales)[N + n] = z;
      }
    }
    for (int g = tid; g < (K >> 4); g += kRowThreads) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) word |= code_asym(row[16 * g + i] * norm, s, z) << code_bit_offset(i);
      codes[tiled_word(n, g, words, tiles)] = word;
    }
    return;
  }
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
  if (x_bf16 && K == kMfmaRowK && had_block == kMfmaRowK && rotate_fast_ok(X, K, had_block, xq, x_rot)) {
    hipLaunchKernelGGL(rotate_quant_act_mfma4096_kernel, dim3((unsigned)M), dim3(kRowThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(X), nrm, xq, s_a, x_rot);
    return hipGetLastError();
  }
  // bfloat16 rows with blocks of 256, 512 or 1024: the group kernel, with
  // ceil(K / 4096) groups of 1024 elements per wave (one memory latency per
  // row: every load is issued before the first transform). Against the
  // register-path kernel: 4096 x 14336 (block 1024) 28.8 against 51.6 us,
  // 2048 x 11008 (block 256) 13.1 against 14.5 us, 2048 x 4096 (block 1024)
  // 6.4 against 7.7 us.
  if (x_bf16 && lb >= 8 && lb <= 10 && K <= QIFT_MAX_ROW &&
      rotate_fast_ok(X, K, had_block, xq, x_rot)) {
    const int P = (int)((K + 4095) / 4096);  // 1 .. 4
#define QIFT_ROT_GROUPS(LBB, PP)                                                          \
  hipLaunchKernelGGL((rotate_quant_act_mfma_groups_kernel<LBB, PP>), dim3((unsigned)M),  \
                     dim3(kRowThreads), 0, s, reinterpret_cast<const uint16_t*>(X), (int)K, \
                     nrm, xq, s_a, x_rot)
#define QIFT_ROT_GROUPS_P(LBB)            \
  if (P == 1) QIFT_ROT_GROUPS(LBB, 1);    \
  else if (P == 2) QIFT_ROT_GROUPS(LBB, 2); \
  else if (P == 3) QIFT_ROT_GROUPS(LBB, 3); \
  else QIFT_ROT_GROUPS(LBB, 4);
    if (lb == 8) {
      QIFT_ROT_GROUPS_P(8)
    } else if (lb == 9) {
      QIFT_ROT_GROUPS_P(9)
    } else {
      QIFT_ROT_GROUPS_P(10)
    }
#undef QIFT_ROT_GROUPS_P
#undef QIFT_ROT_GROUPS
    return hipGetLastError();
  }
  if (rotate_fast_ok(X, K, had_block, xq, x_rot)) {
    const size_t lds = lb > kRegLog2B ? (size_t)(K + K / 16) * sizeof(float) : 0;
    const int groups = (int)((K / 16 + kRowThreads - 1) / kRowThreads);  // per thread, 1..4
#define QIFT_ROT_FAST(TT, QQ)                                                                \
  hipLaunchKernelGGL((rotate_quant_act_fast_kernel<TT, QQ>), dim3((unsigned)M),             \
                     dim3(kRowThreads), lds, s, reinterpret_cast<const TT*>(X), (int)K, lb, nrm, \
                     xq, s_a, x_rot)
    if (x_bf16) {
      if (groups == 1) QIFT_ROT_FAST(uint16_t, 1);
      else if (groups == 2) QIFT_ROT_FAST(uint16_t, 2);
      else if (groups == 3) QIFT_ROT_FAST(uint16_t, 3);
      else QIFT_ROT_FAST(uint16_t, 4);
    } else {
      if (groups == 1) QIFT_ROT_FAST(float, 1);
      else if (groups == 2) QIFT_ROT_FAST(float, 2);
      else if (groups == 3) QIFT_ROT_FAST(float, 3);
      else QIFT_ROT_FAST(float, 4);
    }
#undef QIFT_ROT_FAST
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
