// KV4 quantizer: every head vector of a [T, H, D] key or value tensor is
// rotated by a block Hadamard transform along D and quantized to int4 with
// its own absmax scale (the "KV4" of rotated W2A4/KV4 inference, Qift
// abstract).
//
// Layout on the GPU: a head vector of D elements is held by L = D/E lanes of
// one quad with E consecutive elements each (E = min(D, 32); 64 for
// D = 256), so log2(E) butterfly stages run inside a lane's registers and at
// most two (partners at lane xor 1 and xor 2) cross lanes, through DPP quad
// permutations. (64 elements per lane for D = 128 saves 12% of the
// instructions but runs 25% slower: half the waves, each with twice the
// serial work and loads spread over twice the span.) A lane loads 2E (bf16) or 4E bytes and stores E/2 bytes of
// codes. The kernel is bound by HBM bandwidth in principle and by VALU issue
// in practice, so every step is written for the fewest instructions per
// element:
//  - a cross-lane butterfly costs one DPP-fed fused multiply-add per element
//    (lane_butterfly8: each lane keeps its values up to a sign sigma);
//  - the absmax ignores the sign; the quantizer folds sigma into 1 / s;
//  - rounding and packing use the float adder and byte permutes
//    (int4x8_rint), with the exact division only for near-tie groups.
#include "lane_butterfly.h"
#include "quant_pack.h"

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

// kFull: the Hadamard block is the whole head vector (every stage runs; the
// common case), so the stage conditions are compile-time constants.
template <int E, int L, bool kFull, typename T>
__global__ __launch_bounds__(kKvThreads) void kv4_kernel(const T* __restrict__ KV, int64_t rows,
                                                         int log2b, float norm,
                                                         uint8_t* __restrict__ kvq,
                                                         float* __restrict__ scales) {
  static_assert(L == 1 || L == 2 || L == 4, "a head vector stays inside one quad");
  constexpr int D = E * L;
  constexpr int kLogE = E == 64 ? 6 : (E == 32 ? 5 : 4);
  const int lane = threadIdx.x & (L - 1);
  const int64_t r = (int64_t)blockIdx.x * (kKvThreads / L) + threadIdx.x / L;
  const bool live = r < rows;  // uniform over the quad
  // a row past the end reads the last row; its results are not stored
  float v[E];
  kv4_load<E, T>(KV + (live ? r : rows - 1) * D + lane * E, v);
  // in-lane stages (strides 1 .. E/2)
#pragma unroll
  for (int st = 0; st < kLogE; ++st) {
    if (kFull || st < log2b) {
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
  // cross-lane stages (strides E, 2E), values kept up to the sign sigma
  float sigma = 1.f;
  if constexpr (L >= 2) {
    if (kFull || E < (1 << log2b)) {
      const float c = (lane & 1) ? -1.f : 1.f;
#pragma unroll
      for (int j = 0; j < E; j += 8) lane_butterfly8<1>(v + j, c);
      sigma = c;
    }
  }
  if constexpr (L == 4) {
    if (kFull || 2 * E < (1 << log2b)) {
      const float c = (lane & 2) ? -1.f : 1.f;
#pragma unroll
      for (int j = 0; j < E; j += 8) lane_butterfly8<2>(v + j, c);
      sigma *= c;
    }
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) m = fmaxf(m, fabsf(v[j]));
  if constexpr (L >= 2) m = fmaxf(m, quad_xor<1>(m));
  if constexpr (L == 4) m = fmaxf(m, quad_xor<2>(m));
  m *= norm;  // rounding is monotonic: max(|v|) * norm == max(|v * norm|)
  const float s = __fdiv_rn(m, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  // y = stored * sigma * (norm / s), within four roundings of x' / s with
  // x' = fl(v * norm) the rotated value (int4x8_rint's margin covers it)
  const float rl = sigma * (norm * rs);
  uint32_t words[E / 8];
  float dmax = 0.f;
#pragma unroll
  for (int w = 0; w < E / 8; ++w) {
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = v[8 * w + j] * rl;
    words[w] = int4x8_rint(y, dmax);
  }
  if (!(dmax <= 0.49999f) || !rint_path_ok(rs)) {
    // a value within 1e-5 of a rounding tie (rare): exact division
#pragma unroll
    for (int w = 0; w < E / 8; ++w) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = sigma * (v[8 * w + j] * norm);
      words[w] = int4x8_exact(x, s);
    }
  }
  if (live) {
    uint8_t* dst = kvq + r * (D / 2) + lane * (E / 2);
    if constexpr (E == 64) {
      reinterpret_cast<uint4*>(dst)[0] = uint4{words[0], words[1], words[2], words[3]};
      reinterpret_cast<uint4*>(dst)[1] = uint4{words[4], words[5], words[6], words[7]};
    } else if constexpr (E == 32) {
      *reinterpret_cast<uint4*>(dst) = uint4{words[0], words[1], words[2], words[3]};
    } else {
      *reinterpret_cast<uint2*>(dst) = uint2{words[0], words[1]};
    }
    if (lane == 0) scales[r] = s;
  }
}

template <int E, int L, bool kFull>
static void launch_kv4_f(const void* KV, int bf16, int64_t rows, int log2b, float norm,
                         uint8_t* kvq, float* scales, hipStream_t s) {
  const int per_block = kKvThreads / L;
  const unsigned grid = (unsigned)((rows + per_block - 1) / per_block);
  if (bf16)
    hipLaunchKernelGGL((kv4_kernel<E, L, kFull, uint16_t>), dim3(grid), dim3(kKvThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(KV), rows, log2b, norm, kvq, scales);
  else
    hipLaunchKernelGGL((kv4_kernel<E, L, kFull, float>), dim3(grid), dim3(kKvThreads), 0, s,
                       reinterpret_cast<const float*>(KV), rows, log2b, norm, kvq, scales);
}

template <int E, int L>
static void launch_kv4_l(const void* KV, int bf16, int64_t rows, int log2b, float norm,
                         uint8_t* kvq, float* scales, hipStream_t s) {
  if ((1 << log2b) == E * L)
    launch_kv4_f<E, L, true>(KV, bf16, rows, log2b, norm, kvq, scales, s);
  else
    launch_kv4_f<E, L, false>(KV, bf16, rows, log2b, norm, kvq, scales, s);
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
    case 256: launch_kv4_l<64, 4>(KV, bf16, rows, log2b, norm, kvq, scales, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qift
