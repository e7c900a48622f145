// Per-channel weight codes of the offline quantizers: the nearest-level
// decision for each level set, the level each code stands for, the stored
// scale, the scale rules and the chunk-major tiled word layout. Shared by the
// plain quantizer and the error-compensated one, so that both take the same
// decision for the same float32 weight (Qift abstract: fixed no-zero two-bit
// level sets with one scale per output channel and no zero point).
#pragma once

#include "rotate_row.h"

namespace qift {

// max |row[i]| * norm over the row (every thread gets the result).
__device__ __forceinline__ float row_absmax(const float* row, int K, float norm, int tid,
                                            float* red) {
  float m = 0.f;
  for (int i = tid; i < K; i += kRowThreads) m = fmaxf(m, fabsf(row[i]));
  m *= norm;  // rounding is monotonic: max(|v|)*norm == max(|v*norm|)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Largest v over the workgroup (every thread gets the result).
__device__ __forceinline__ float block_max(float v, int tid, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Range of the row (value i = row[i] * norm) widened to contain 0:
// lo = min(min v, 0), hi = max(max v, 0) (every thread gets both).
__device__ __forceinline__ void row_range0(const float* row, int K, float norm, int tid,
                                           float* red, float& lo, float& hi) {
  float mn = 0.f, mx = 0.f;
  for (int i = tid; i < K; i += kRowThreads) {
    mn = fminf(mn, row[i]);
    mx = fmaxf(mx, row[i]);
  }
  // rounding is monotonic: min(v) * norm == min(v * norm), likewise max
  hi = block_max(mx * norm, tid, red);
  lo = -block_max(-(mn * norm), tid, red);
}

// Code of the asymmetric min-max grid: clip(rint(w / s) + z, 0, 3) in
// float32 (z the zero point as a float); 0 when s = 0.
__device__ __forceinline__ uint32_t code_asym(float w, float s, float z) {
  if (s == 0.f) return 0u;
  return (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(w, s)) + z, 0.f), 3.f);
}

__device__ __forceinline__ int quant_int4(float x, float s) {
  if (s == 0.f) return 0;
  float q = rintf(__fdiv_rn(x, s));
  q = fminf(fmaxf(q, -7.f), 7.f);
  return (int)q;
}

__device__ __forceinline__ uint32_t code_mnz(float w, float s) {
  // 2-bit two's complement t with half-scale level 2t+1: +inner 00, +outer 01,
  // -outer 10, -inner 11. |w| == s is a tie and goes to the inner level.
  if (s == 0.f) return 0u;
  const bool outer = fabsf(w) > s;
  const bool neg = w < 0.f;
  return neg ? (outer ? 2u : 3u) : (outer ? 1u : 0u);
}

__device__ __forceinline__ uint32_t code_pot(float w, float s) {
  // bit 1 = sign, bit 0 = shift by two; outer iff |w| > 2.5 s, compared
  // exactly in double (2|w| and 5s are exact there).
  if (s == 0.f) return 0u;
  const bool outer = 2.0 * (double)fabsf(w) > 5.0 * (double)s;
  const bool neg = w < 0.f;
  return ((neg ? 1u : 0u) << 1) | (outer ? 1u : 0u);
}

// Level table: code of the level nearest to w, distances |w - L[c] * s| in
// double (L[c] * s is exact there), the codes visited in the tie-break order
// `pref` (byte r = the code of rank r: smaller |L|, then the non-negative
// level, then the lower code) so that the first minimum wins.
__device__ __forceinline__ uint32_t code_lut(float w, float s, uint32_t table, uint32_t pref) {
  double best = __builtin_huge_val();
  uint32_t code = pref & 3u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t c = (pref >> (8 * r)) & 3u;
    const double L = (double)(int8_t)((table >> (8 * c)) & 0xFFu);
    const double dist = fabs((double)w - L * (double)s);
    if (dist < best) {
      best = dist;
      code = c;
    }
  }
  return code;
}

__device__ __forceinline__ uint32_t code2(int levels, float w, float s, uint32_t table,
                                          uint32_t pref) {
  return levels == QIFT_LEVELS_MNZ ? code_mnz(w, s)
         : levels == QIFT_LEVELS_POT ? code_pot(w, s)
                                     : code_lut(w, s, table, pref);
}

// The multiple of the scale that 2-bit code c stands for.
__device__ __forceinline__ double real_level(int levels, uint32_t c, uint32_t table) {
  if (levels == QIFT_LEVELS_MNZ) return 0.5 * (double)(2 * (c >= 2u ? (int)c - 4 : (int)c) + 1);
  if (levels == QIFT_LEVELS_POT) return ((c & 2u) ? -1.0 : 1.0) * ((c & 1u) ? 4.0 : 1.0);
  return (double)(int8_t)((table >> (8 * c)) & 0xFFu);
}

// Sum of v over the workgroup in a fixed order (every thread gets the same
// value).
__device__ __forceinline__ double block_sum(double v, double* red, int tid) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float stored_scale(float s32, int scale_f16) {
  return scale_f16 ? __half2float(__float2half_rn(s32)) : s32;
}

__device__ __forceinline__ int code_bit_offset(int i) {
  return 8 * ((i >> 1) & 3) + 4 * (i >> 3) + 2 * (i & 1);
}

// Word w of channel row n in the chunk-major tiled weight layout (W words per
// channel row, T tiles of 16 channels): chunk c = w / 16 of all tiles comes
// first, 256 T words for every full chunk; in chunk c (u_c = min(16, W - 16c)
// words per channel) tile r = n / 16 holds 16 u_c words, in which the 16-byte
// unit of lane (g, i) = ((w % 16) / 4, n % 16) sits at word 4 * (16 g + i),
// word j = w % 4 inside it.
__device__ __forceinline__ int64_t tiled_word(int64_t n, int64_t w, int64_t W, int64_t T) {
  const int64_t r = n >> 4, i = n & 15;
  const int64_t c = w >> 4, g = (w >> 2) & 3, j = w & 3;
  const int64_t uc = W - 16 * c < 16 ? W - 16 * c : 16;
  return c * 256 * T + r * 16 * uc + (16 * g + i) * 4 + j;
}

// Candidates of the searched scale: fractions (64 - j) / 64 of the absmax
// scale, j = 0 .. kScaleCandidates - 1.
constexpr int kScaleCandidates = 64;


// Scale of one channel row held in LDS as float32 (value i = row[i] * norm):
// the absmax rule s = fl32(absmax / outer), or with mse_rule the candidate
// fl32(s * (64 - j) / 64), j = 0..63, whose stored value gives the smallest
// float64 sum of squared errors (the first, i.e. largest, on ties). Returns
// the float32 scale before rounding to the stored dtype. Every thread of the
// workgroup gets the result.
__device__ __forceinline__ float choose_scale(const float* row, int K, float norm, int levels,
                                              uint32_t table, uint32_t pref, float outer,
                                              int mse_rule, int scale_f16, float* red,
                                              double* red64) {
  const int tid = threadIdx.x;
  const bool int4 = levels == QIFT_LEVELS_INT4;
  const float amax = row_absmax(row, K, norm, tid, red);
  float s32 = __fdiv_rn(amax, outer);
  if (mse_rule) {
    const float base = s32;
    double best = __builtin_huge_val();
    for (int j = 0; j < kScaleCandidates; ++j) {
      const float cand = base * ((float)(kScaleCandidates - j) / (float)kScaleCandidates);
      const float sj = stored_scale(cand, scale_f16);
      double e = 0.0;
      for (int i = tid; i < K; i += kRowThreads) {
        const float w = row[i] * norm;
        const double lv = int4 ? (double)quant_int4(w, sj)
                               : real_level(levels, code2(levels, w, sj, table, pref), table);
        const double d = (double)w - lv * (double)sj;
        e += d * d;
      }
      e = block_sum(e, red64, tid);
      if (e < best) {
        best = e;
        s32 = cand;
      }
    }
  }
  return s32;
}

// Host side: the outer level of the absmax rule and, for a level table, the
// codes in tie-break order (byte r = the code of rank r: smaller |L|, then the
// non-negative level, then the lower code).
inline float level_outer_and_pref(int levels, uint32_t table, uint32_t* pref) {
  *pref = 0;
  if (levels != QIFT_LEVELS_LUT)
    return levels == QIFT_LEVELS_MNZ ? 1.5f : levels == QIFT_LEVELS_POT ? 4.0f : 7.0f;
  int L[4], order[4] = {0, 1, 2, 3}, mx = 0;
  for (int c = 0; c < 4; ++c) {
    L[c] = (int)(int8_t)((table >> (8 * c)) & 0xFFu);
    mx = L[c] < 0 ? (-L[c] > mx ? -L[c] : mx) : (L[c] > mx ? L[c] : mx);
  }
  auto key = [&](int c) { return (L[c] < 0 ? -L[c] : L[c]) * 16 + (L[c] < 0 ? 8 : 0) + c; };
  for (int i = 1; i < 4; ++i)
    for (int j = i; j > 0 && key(order[j]) < key(order[j - 1]); --j) {
      const int tmp = order[j];
      order[j] = order[j - 1];
      order[j - 1] = tmp;
    }
  for (int r = 0; r < 4; ++r) *pref |= (uint32_t)order[r] << (8 * r);
  return (float)mx;
}

}  // namespace qift
