// Measurement kernels for the benchmark: the chip's achievable HBM stream
// rate and int8 matrix-core rate, against which the kernels of the method are
// reported. Not a step of the method.
#include "linear_common.h"

namespace qift {

// MODE 0: read-only stream (every 16-byte unit loaded once and folded into
// one value per thread, stored only if it equals an impossible pattern);
// MODE 1: copy src -> dst. Workgroup b owns the contiguous units
// [b * kUnitsPerGroup, (b + 1) * kUnitsPerGroup) (64 KB), its threads four
// loads in flight each, non-temporal loads and stores; the rounds where all
// four are in range run without bounds checks. (Measured on MI355X: this
// blocked order reads about 15% faster than a grid-stride walk of the same
// loads, and non-temporal loads about 10% faster than plain ones.)
constexpr int64_t kUnitsPerGroup = 4096;

template <int MODE>
__global__ __launch_bounds__(256) void measure_stream_kernel(const v4u* __restrict__ src,
                                                             v4u* __restrict__ dst, int64_t n16,
                                                             uint32_t* __restrict__ sink) {
  const int64_t lo = (int64_t)blockIdx.x * kUnitsPerGroup;
  const int64_t hi = lo + kUnitsPerGroup < n16 ? lo + kUnitsPerGroup : n16;
  int64_t i = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * 256 < hi; i += 4 * 256) {
    v4u v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(as_global(src + i + 256 * u));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (MODE == 1) {
        __builtin_nontemporal_store(v[u], as_global_out(dst + i + 256 * u));
      } else {
        acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
      }
    }
  }
  for (; i < hi; i += 256) {
    const v4u v = __builtin_nontemporal_load(as_global(src + i));
    if constexpr (MODE == 1) {
      __builtin_nontemporal_store(v, as_global_out(dst + i));
    } else {
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x9e3779b9u) *as_global_out(sink + (blockIdx.x & 8191u)) = acc;
}

// Each wave runs `iters` rounds of 8 independent v_mfma_i32_16x16x64_i8 on
// register operands (the bit patterns of the linear's operands), then folds
// its accumulators into one value. Wave 0 of workgroup 0 also reads the
// shader clock and the constant 100 MHz clock at its start and end
// (clk[0..3]), from which the clock under this load follows.
__global__ __launch_bounds__(256) void measure_mfma_i8_kernel(int iters, uint32_t seed,
                                                              uint32_t* __restrict__ sink,
                                                              uint64_t* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  uint64_t c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  const uint32_t x = seed * (uint32_t)(lane + 1);
  v4i a = v4i{(int)(x & 0xF0F0F0F0u), (int)((x << 4) & 0xF0F0F0F0u), (int)(x ^ 0x30303030u),
              (int)(x & 0x70707070u)};
  v4i b = v4i{(int)(x | 0x20202020u), (int)((x >> 2) | 0x20202020u), (int)(0xE0E0E0E0u | x),
              (int)(0x60606060u ^ x)};
  v4i acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = mfma16(a, b, v4i{i, 0, 0, 0});
  for (int it = 1; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = mfma16(a, b, acc[i]);
  }
  int fold = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) fold ^= acc[i][0] ^ acc[i][1] ^ acc[i][2] ^ acc[i][3];
  if (fold == 0x12345678) *as_global_out(sink + (blockIdx.x & 8191u)) = (uint32_t)fold;
  if (timer) {
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    v4u w = v4u{(uint32_t)c0, (uint32_t)(c0 >> 32), (uint32_t)r0, (uint32_t)(r0 >> 32)};
    *as_global_out(reinterpret_cast<v4u*>(clk)) = w;
    w = v4u{(uint32_t)c1, (uint32_t)(c1 >> 32), (uint32_t)r1, (uint32_t)(r1 >> 32)};
    *as_global_out(reinterpret_cast<v4u*>(clk) + 1) = w;
  }
}

hipError_t launch_measure_stream(const void* src, void* dst, int64_t bytes, int mode,
                                 uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const unsigned grid = (unsigned)((n16 + kUnitsPerGroup - 1) / kUnitsPerGroup);
  if (mode == 1) {
    hipLaunchKernelGGL(measure_stream_kernel<1>, dim3(grid), dim3(256), 0, s,
                       reinterpret_cast<const v4u*>(src), reinterpret_cast<v4u*>(dst), n16, sink);
  } else {
    hipLaunchKernelGGL(measure_stream_kernel<0>, dim3(grid), dim3(256), 0, s,
                       reinterpret_cast<const v4u*>(src), nullptr, n16, sink);
  }
  return hipGetLastError();
}

hipError_t launch_measure_mfma_i8(int64_t iters, int64_t workgroups, uint32_t* sink,
                                  uint64_t* clk, hipStream_t s) {
  hipLaunchKernelGGL(measure_mfma_i8_kernel, dim3((unsigned)workgroups), dim3(256), 0, s, (int)iters,
                     0x9e3779b9u, sink, clk);
  return hipGetLastError();
}

}  // namespace qift
