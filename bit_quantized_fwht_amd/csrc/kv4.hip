// KV4 quantizer: every head vector of a [T, H, D] key or value tensor is
// rotated by a block Hadamard transform along D and quantized to int4 with
// its own absmax scale (the "KV4" of rotated W2A4/KV4 inference, Qift
// abstract).
//
// Layout on the GPU: a head vector of D elements is held by L = D/8 lanes,
// 8 consecutive elements per lane, so one wave holds 64/L vectors. The first
// three butterfly stages run inside a lane's registers, the remaining
// log2(B)-3 stages between lanes with xor shuffles. Loads are 16 bytes per
// lane (bf16) and the packed output is one 32-bit word per lane, both fully
// coalesced; the kernel is bound by HBM bandwidth.
#include "qift_internal.h"

namespace qift {

constexpr int kKvThreads = 256;

template <int L, typename T>
__global__ __launch_bounds__(kKvThreads) void kv4_kernel(const T* __restrict__ KV, int64_t rows,
                                                         int log2b, float norm,
                                                         uint8_t* __restrict__ kvq,
                                                         float* __restrict__ scales) {
  constexpr int D = 8 * L;
  const int lane = threadIdx.x & (L - 1);
  const int64_t r = (int64_t)blockIdx.x * (kKvThreads / L) + (threadIdx.x / L);
  const bool live = r < rows;
  float v[8];
  if (live) {
    if constexpr (sizeof(T) == 2) {
      const uint4 u = reinterpret_cast<const uint4*>(KV + r * D)[lane];
      v[0] = __uint_as_float(u.x << 16);
      v[1] = __uint_as_float(u.x & 0xffff0000u);
      v[2] = __uint_as_float(u.y << 16);
      v[3] = __uint_as_float(u.y & 0xffff0000u);
      v[4] = __uint_as_float(u.z << 16);
      v[5] = __uint_as_float(u.z & 0xffff0000u);
      v[6] = __uint_as_float(u.w << 16);
      v[7] = __uint_as_float(u.w & 0xffff0000u);
    } else {
      const float4* p = reinterpret_cast<const float4*>(KV + r * D) + 2 * lane;
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  // in-lane stages (strides 1, 2, 4)
  const int in_lane = log2b < 3 ? log2b : 3;
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    if (st < in_lane) {
      const int h = 1 << st;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!(j & h)) {
          const float a = v[j], b = v[j + h];
          v[j] = a + b;
          v[j + h] = a - b;
        }
      }
    }
  }
  // cross-lane stages (strides 8 .. B/2): partner lane = lane ^ h
  for (int h = 1; (8 * h) < (1 << log2b); h <<= 1) {
    const bool upper = (lane & h) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float o = __shfl_xor(v[j], h, 64);
      v[j] = upper ? (o - v[j]) : (v[j] + o);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] *= norm;
    m = fmaxf(m, fabsf(v[j]));
  }
#pragma unroll
  for (int off = 1; off < L; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float s = __fdiv_rn(m, 7.0f);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int q = 0;
    if (s != 0.f) {
      float t = rintf(__fdiv_rn(v[j], s));
      t = fminf(fmaxf(t, -7.f), 7.f);
      q = (int)t;
    }
    word |= ((uint32_t)q & 0xFu) << (4 * j);
  }
  if (live) {
    reinterpret_cast<uint32_t*>(kvq + r * (D / 2))[lane] = word;
    if (lane == 0) scales[r] = s;
  }
}

template <int L>
static void launch_kv4_l(const void* KV, int bf16, int64_t rows, int log2b, float norm,
                         uint8_t* kvq, float* scales, hipStream_t s) {
  const int per_block = kKvThreads / L;
  const unsigned grid = (unsigned)((rows + per_block - 1) / per_block);
  if (bf16)
    hipLaunchKernelGGL((kv4_kernel<L, uint16_t>), dim3(grid), dim3(kKvThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(KV), rows, log2b, norm, kvq, scales);
  else
    hipLaunchKernelGGL((kv4_kernel<L, float>), dim3(grid), dim3(kKvThreads), 0, s,
                       reinterpret_cast<const float*>(KV), rows, log2b, norm, kvq, scales);
}

hipError_t launch_kv4(const void* KV, int bf16, int64_t rows, int D, int had_block, uint8_t* kvq,
                      float* scales, hipStream_t s) {
  int log2b = 0;
  while ((1 << log2b) < had_block) ++log2b;
  const float norm = (float)(1.0 / __builtin_sqrt((double)had_block));
  switch (D) {
    case 16: launch_kv4_l<2>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 32: launch_kv4_l<4>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 64: launch_kv4_l<8>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 128: launch_kv4_l<16>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    case 256: launch_kv4_l<32>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qift
