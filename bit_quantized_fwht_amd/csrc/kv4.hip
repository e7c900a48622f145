// KV4 quantizer: every head vector of a [T, H, D] key or value tensor is
// rotated by a block Hadamard transform along D and quantized to int4 with
// its own absmax scale (the "KV4" of rotated W2A4/KV4 inference, Qift
// abstract).
//
// Layout on the GPU: a head vector of D elements is held by L = D/E lanes
// with E = min(D, 32) consecutive elements each, so five butterfly stages run
// inside a lane's registers and only log2(L) stages (xor 1 and 2 for
// D = 128, quad permutes) cross lanes. A lane loads E*2 contiguous bytes
// (bf16) and stores E/2 bytes of codes; the kernel is bound by HBM bandwidth.
#include "qift_internal.h"

namespace qift {

constexpr int kKvThreads = 256;

template <int E, typename T>
__device__ __forceinline__ void kv4_load(const T* __restrict__ src, float v[E]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const uint4 u = reinterpret_cast<const uint4*>(src)[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 f = reinterpret_cast<const float4*>(src)[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  }
}

template <int E, int L, typename T>
__global__ __launch_bounds__(kKvThreads) void kv4_kernel(const T* __restrict__ KV, int64_t rows,
                                                         int log2b, float norm,
                                                         uint8_t* __restrict__ kvq,
                                                         float* __restrict__ scales) {
  constexpr int D = E * L;
  constexpr int kLogE = E == 32 ? 5 : 4;
  const int lane = threadIdx.x & (L - 1);
  const int64_t r = (int64_t)blockIdx.x * (kKvThreads / L) + threadIdx.x / L;
  const bool live = r < rows;
  float v[E];
  if (live) {
    kv4_load<E, T>(KV + r * D + lane * E, v);
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = 0.f;
  }
  // in-lane stages (strides 1 .. E/2)
#pragma unroll
  for (int st = 0; st < kLogE; ++st) {
    if (st < log2b) {
      const int h = 1 << st;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if (!(j & h)) {
          const float a = v[j], b = v[j + h];
          v[j] = a + b;
          v[j + h] = a - b;
        }
      }
    }
  }
  // cross-lane stages (strides E .. B/2): partner lane = lane ^ h
#pragma unroll
  for (int h = 1; h < L; h <<= 1) {
    if ((E * h) < (1 << log2b)) {
      const bool upper = (lane & h) != 0;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float o = __shfl_xor(v[j], h, 64);
        v[j] = upper ? (o - v[j]) : (v[j] + o);
      }
    }
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    v[j] *= norm;
    m = fmaxf(m, fabsf(v[j]));
  }
#pragma unroll
  for (int off = 1; off < L; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float s = __fdiv_rn(m, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  uint32_t words[E / 8];
#pragma unroll
  for (int w = 0; w < E / 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      word |= code_int4_recip(v[8 * w + j], s, rs) << (4 * j);
    words[w] = word;
  }
  if (live) {
    uint8_t* dst = kvq + r * (D / 2) + lane * (E / 2);
    if constexpr (E == 32)
      *reinterpret_cast<uint4*>(dst) = uint4{words[0], words[1], words[2], words[3]};
    else
      *reinterpret_cast<uint2*>(dst) = uint2{words[0], words[1]};
    if (lane == 0) scales[r] = s;
  }
}

template <int E, int L>
static void launch_kv4_l(const void* KV, int bf16, int64_t rows, int log2b, float norm,
                         uint8_t* kvq, float* scales, hipStream_t s) {
  const int per_block = kKvThreads / L;
  const unsigned grid = (unsigned)((rows + per_block - 1) / per_block);
  if (bf16)
    hipLaunchKernelGGL((kv4_kernel<E, L, uint16_t>), dim3(grid), dim3(kKvThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(KV), rows, log2b, norm, kvq, scales);
  else
    hipLaunchKernelGGL((kv4_kernel<E, L, float>), dim3(grid), dim3(kKvThreads), 0, s,
                       reinterpret_cast<const float*>(KV), rows, log2b, norm, kvq, scales);
}

hipError_t launch_kv4(const void* KV, int bf16, int64_t rows, int D, int had_block, uint8_t* kvq,
                      float* scales, hipStream_t s) {
  int log2b = 0;
  while ((1 << log2b) < had_block) ++log2b;
  const float norm = (float)(1.0 / __builtin_sqrt((double)had_block));
  switch (D) {
    case 16: launch_kv4_l<16, 1>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 32: launch_kv4_l<32, 1>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 64: launch_kv4_l<32, 2>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 128: launch_kv4_l<32, 4>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 256: launch_kv4_l<32, 8>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qift
