// The rotated W2A4 linear, decode side (M <= 16): Y = (q . level^T) * s_a *
// s_w * kappa with an exact int32 accumulator (Qift abstract: decoded weight
// application of the no-zero two-bit level sets, per-channel scale, 4-bit
// activations).
//
// A wave owns 64 output channels and walks K; every lane loads 16 bytes of
// codes per 16-channel tile per step straight into registers (no LDS),
// unpacks them into operands and issues one MFMA per 16 channels; the 16 rows
// of the MFMA's other side carry the (at most 16) tokens. The accumulation
// over K happens inside the matrix core, so no cross-lane reduction is needed.
// The grouped kernel runs the decode tiles of several linears (one plan in a
// caller-owned workspace) in one launch.
#include "linear_common.h"

namespace qift {

// ---------------------------------------------------------------------------
// decode: M <= 16
// ---------------------------------------------------------------------------

#ifndef QIFT_DECODE_MINBLOCKS
#define QIFT_DECODE_MINBLOCKS 2
#endif

constexpr int kDecodeTiles = kDecodeRowsPerWave / 16;  // 16-channel MFMA tiles per wave

// weight-stream load: 16 bytes, optionally marked non-temporal (streamed once)
__device__ __forceinline__ uint4 ld16_stream(const uint32_t* p) {
#if QIFT_DECODE_NT
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
#else
  return ld16(p);
#endif
}

// Output staging of one wave: 16 rows x 64 channels of int32, rows padded to
// 68 words.
constexpr int kDecEpiStride = 68;
constexpr int kDecEpiWords = 16 * kDecEpiStride;

template <int LV>
__device__ __forceinline__ void decode_wave(const qift_linear_desc& d, int64_t n0, int scale_f16,
                                            int y_dtype, int lane, int* epi) {
  using F = Fmt<LV>;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t M = d.M, K = d.K, N = d.N;
  const int64_t cw = F::code_words(K);
  const int64_t tiles = (N + 15) >> 4;
  const uint8_t* xq = d.xq;
  const uint32_t* codes = d.codes;
  const bool act_row = r16 < M;
  const OpConsts km = op_consts(d.reserved, lane);

  v4i acc[kDecodeTiles];
#pragma unroll
  for (int i = 0; i < kDecodeTiles; ++i) acc[i] = v4i{0, 0, 0, 0};

  const int64_t nchunks = (K + F::kChunkK - 1) / F::kChunkK;

  // one K chunk of this lane: its 16-byte code unit of each tile and the
  // matching 32 (or 16) bytes of its activation row
  struct Chunk {
    uint4 c[kDecodeTiles];
    uint4 a0, a1;
  };
  auto load = [&](Chunk& ch, int64_t t) {
    const int64_t kseg = t * F::kChunkK + (int64_t)g * F::kLaneK;
    const bool kval = t < nchunks && kseg < K;
    // chunk-major tiled layout: chunk t of all tiles at t * 256 * tiles;
    // in it, tile (n0 + 16 i) / 16 holds 16 * ut words with the lane's
    // 16-byte unit at word 4 * lane -- one contiguous 1 KB per full chunk,
    // and the wave's four tiles are adjacent
    const int64_t ut = cw - 16 * t < 16 ? cw - 16 * t : 16;
    const uint32_t* cbase = codes + t * 256 * tiles + 4 * lane;
#pragma unroll
    for (int i = 0; i < kDecodeTiles; ++i) {
      const int64_t tn = n0 + 16 * i;
      ch.c[i] = (kval && tn < N) ? ld16_stream(cbase + (tn >> 4) * 16 * ut) : uint4{0u, 0u, 0u, 0u};
    }
    ch.a0 = uint4{0u, 0u, 0u, 0u};
    ch.a1 = uint4{0u, 0u, 0u, 0u};
    if (kval && act_row) {
      const uint8_t* ap = xq + (int64_t)r16 * (K / 2) + kseg / 2;
      ch.a0 = ld16(ap);
      if constexpr (!F::kInt4) ch.a1 = ld16(ap + 16);
    }
  };
  auto compute = [&](const Chunk& ch) {
#pragma unroll
    for (int s = 0; s < F::kSteps; ++s) {
      const v4i A = act_operand(ch.a0, ch.a1, s);
#pragma unroll
      for (int i = 0; i < kDecodeTiles; ++i)
        acc[i] = mfma16(A, weight_operand<LV>(ch.c[i], s, km), acc[i]);
    }
  };
  // two chunks in flight: the loads of chunk t+1 are issued before chunk t
  // is consumed
  Chunk x, y;
  load(x, 0);
  for (int64_t t = 0; t < nchunks; t += 2) {
    load(y, t + 1);
    compute(x);
    load(x, t + 2);
    if (t + 1 < nchunks) compute(y);
  }

  // Epilogue. The lane holds rows m = 4g + r of channels n0 + 16 i + r16 (MFMA
  // order), so direct stores would write 64-byte halves of cache lines, four
  // rows apart (20% of the launch at M = 16). The wave's 16 x 64 block goes
  // through its own LDS region instead and is stored row-major: each lane then
  // owns 4 consecutive channels of one row and writes them as one piece.
  const float kappa = level_kappa(LV);
#pragma unroll
  for (int i = 0; i < kDecodeTiles; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      epi[(4 * g + r) * kDecEpiStride + 16 * i + r16] = acc[i][r] >> F::kShift;
  // one wave writes and reads its own region: its LDS operations complete in order
  const int c0 = 4 * (lane & 15);
  const int64_t n = n0 + c0;
  float sw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sw[e] = n + e < N ? load_scale(d.scales, n + e, scale_f16) * kappa : 0.f;
  const bool vec = (N & 3) == 0 && n + 4 <= N && (reinterpret_cast<uintptr_t>(d.Y) & 15) == 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int m = 4 * p + (lane >> 4);
    if (m >= M) continue;
    const int4 v = *reinterpret_cast<const int4*>(&epi[m * kDecEpiStride + c0]);
    const int a[4] = {v.x, v.y, v.z, v.w};
    const int64_t o = (int64_t)m * N + n;
    if (y_dtype == QIFT_I32) {
      int* y = reinterpret_cast<int*>(d.Y) + o;
      if (vec) {
        *reinterpret_cast<int4*>(y) = v;
      } else {
        for (int e = 0; e < 4; ++e)
          if (n + e < N) y[e] = a[e];
      }
    } else {
      const float sa = d.s_a[m];
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (float)a[e] * (sa * sw[e]);
      if (y_dtype == QIFT_BF16) {
        uint16_t* yo = reinterpret_cast<uint16_t*>(d.Y) + o;
        if (vec) {
          *reinterpret_cast<uint2*>(yo) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yo[e] = float_to_bf16_bits(y[e]);
        }
      } else {
        float* yo = reinterpret_cast<float*>(d.Y) + o;
        if (vec) {
          *reinterpret_cast<float4*>(yo) = float4{y[0], y[1], y[2], y[3]};
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yo[e] = y[e];
        }
      }
    }
  }
}

__device__ __forceinline__ void decode_dispatch(const qift_linear_desc& d, int64_t tile,
                                                int scale_f16, int y_dtype, int* epi_all) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n0 = tile * kDecodeRowsPerTile + (int64_t)wave * kDecodeRowsPerWave;
  if (n0 >= d.N) return;
  int* epi = epi_all + wave * kDecEpiWords;
  switch (d.levels) {
    case QIFT_LEVELS_MNZ: decode_wave<QIFT_LEVELS_MNZ>(d, n0, scale_f16, y_dtype, lane, epi); break;
    case QIFT_LEVELS_POT: decode_wave<QIFT_LEVELS_POT>(d, n0, scale_f16, y_dtype, lane, epi); break;
    case QIFT_LEVELS_LUT: decode_wave<QIFT_LEVELS_LUT>(d, n0, scale_f16, y_dtype, lane, epi); break;
    default: decode_wave<QIFT_LEVELS_INT4>(d, n0, scale_f16, y_dtype, lane, epi); break;
  }
}

__global__ __launch_bounds__(256, QIFT_DECODE_MINBLOCKS) void linear_decode_kernel(qift_linear_desc d, int scale_f16,
                                                            int y_dtype) {
  __shared__ __attribute__((aligned(16))) int epi[kDecodeWaves * kDecEpiWords];
  decode_dispatch(d, blockIdx.x, scale_f16, y_dtype, epi);
}

__global__ __launch_bounds__(256, QIFT_DECODE_MINBLOCKS) void linear_grouped_kernel(const uint8_t* __restrict__ ws) {
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(ws);
  const int64_t tile = blockIdx.x;
  if (tile >= h->total_tiles) return;
  const int32_t e = reinterpret_cast<const int32_t*>(ws + h->tile_map_offset)[tile];
  const PlanEntry* pe = reinterpret_cast<const PlanEntry*>(ws + h->entries_offset) + e;
  const qift_linear_desc d = pe->d;
  __shared__ __attribute__((aligned(16))) int epi[kDecodeWaves * kDecEpiWords];
  decode_dispatch(d, tile - pe->tile_begin, h->scale_f16, h->y_dtype, epi);
}

// ---------------------------------------------------------------------------
// decode of one linear with few channels: K split over the waves of a
// workgroup
// ---------------------------------------------------------------------------

// Split-K epilogue: the S waves' partial int32 blocks are summed through
// LDS (red, S * 256 ints); wave 0 applies the scales and stores.
template <int LV, int S>
__device__ __forceinline__ void splitk_epilogue(const qift_linear_desc& d, const float* s_a,
                                                const v4i& acc, int scale_f16, int y_dtype,
                                                int* red) {
  using F = Fmt<LV>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t M = d.M, N = d.N;
  const int64_t tn = blockIdx.x;
  // partial sums: the lane holds rows 4g + r of column r16
#pragma unroll
  for (int r = 0; r < 4; ++r) red[256 * wave + 16 * (4 * g + r) + r16] = acc[r];
  __syncthreads();
  if (wave != 0) return;
  // wave 0: lane -> row m = lane / 4, columns 4 (lane % 4) .. + 3
  const int m = lane >> 2;
  const int c0 = 4 * (lane & 3);
  if (m >= M) return;
  int a[4] = {0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < S; ++w) {
    const int4 v = *reinterpret_cast<const int4*>(&red[256 * w + 16 * m + c0]);
    a[0] += v.x;
    a[1] += v.y;
    a[2] += v.z;
    a[3] += v.w;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] >>= F::kShift;
  const int64_t n = tn * 16 + c0;
  const int64_t o = (int64_t)m * N + n;
  const bool vec = (N & 3) == 0 && n + 4 <= N && (reinterpret_cast<uintptr_t>(d.Y) & 15) == 0;
  if (y_dtype == QIFT_I32) {
    int* yo = reinterpret_cast<int*>(d.Y) + o;
    if (vec) {
      *reinterpret_cast<int4*>(yo) = int4{a[0], a[1], a[2], a[3]};
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) yo[e] = a[e];
    }
    return;
  }
  const float kappa = level_kappa(LV);
  const float sa = s_a[m];
  float yv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    yv[e] = n + e < N ? (float)a[e] * (sa * (load_scale(d.scales, n + e, scale_f16) * kappa)) : 0.f;
  if (y_dtype == QIFT_BF16) {
    uint16_t* yo = reinterpret_cast<uint16_t*>(d.Y) + o;
    if (vec) {
      *reinterpret_cast<uint2*>(yo) = uint2{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])};
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) yo[e] = float_to_bf16_bits(yv[e]);
    }
  } else {
    float* yo = reinterpret_cast<float*>(d.Y) + o;
    if (vec) {
      *reinterpret_cast<float4*>(yo) = float4{yv[0], yv[1], yv[2], yv[3]};
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) yo[e] = yv[e];
    }
  }
}


// A linear call on its own (not grouped) has N / 256 workgroups of 64-channel
// waves, 16 for N = 4096: 16 of 256 CUs would carry its whole weight stream.
// Here a workgroup owns one 16-channel tile and its S waves take every S-th
// K chunk (wave w: chunks w, w + S, ...), each with two chunks in flight; the
// S partial int32 blocks are summed through LDS (integer sums, so the result
// is the same as one wave walking all of K).
template <int LV, int S>
__device__ __forceinline__ void decode_splitk_tile(const qift_linear_desc& d, const uint8_t* xq,
                                                   const float* s_a, int scale_f16, int y_dtype,
                                                   int* red) {
  using F = Fmt<LV>;
  // red: wave w's partial block, rows m and columns c at 256 w + 16 m + c
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t M = d.M, K = d.K, N = d.N;
  const int64_t cw = F::code_words(K);
  const int64_t tiles = (N + 15) >> 4;
  const int64_t tn = blockIdx.x;  // 16-channel tile
  const int64_t nchunks = (K + F::kChunkK - 1) / F::kChunkK;
  const bool act_row = r16 < M;
  const OpConsts km = op_consts(d.reserved, lane);

  struct Chunk {
    uint4 c, a0, a1;
  };
  // chunk t of the tile: the lane's 16-byte code unit (chunk-major tiled
  // layout: chunk t of tile tn at t * 256 * tiles + tn * 16 * ut words) and
  // the matching 32 (or 16) bytes of its activation row
  auto load = [&](Chunk& ch, int64_t t) {
    const int64_t kseg = t * F::kChunkK + (int64_t)g * F::kLaneK;
    const bool kval = t < nchunks && kseg < K;
    const int64_t ut = cw - 16 * t < 16 ? cw - 16 * t : 16;
    ch.c = kval ? ld16_stream(d.codes + t * 256 * tiles + tn * 16 * ut + 4 * lane)
                : uint4{0u, 0u, 0u, 0u};
    ch.a0 = uint4{0u, 0u, 0u, 0u};
    ch.a1 = uint4{0u, 0u, 0u, 0u};
    if (kval && act_row) {
      const uint8_t* ap = xq + (int64_t)r16 * (K / 2) + kseg / 2;
      ch.a0 = ld16(ap);
      if constexpr (!F::kInt4) ch.a1 = ld16(ap + 16);
    }
  };
  v4i acc = v4i{0, 0, 0, 0};
  auto compute = [&](const Chunk& ch) {
#pragma unroll
    for (int s = 0; s < F::kSteps; ++s)
      acc = mfma16(act_operand(ch.a0, ch.a1, s), weight_operand<LV>(ch.c, s, km), acc);
  };
  Chunk x, y;
  load(x, wave);
  for (int64_t t = wave; t < nchunks; t += 2 * S) {
    load(y, t + S);
    compute(x);
    load(x, t + 2 * S);
    if (t + S < nchunks) compute(y);
  }

  splitk_epilogue<LV, S>(d, s_a, acc, scale_f16, y_dtype, red);
}

template <int LV, int S>
__global__ __launch_bounds__(64 * S) void linear_decode_splitk_kernel(qift_linear_desc d,
                                                                      int scale_f16,
                                                                      int y_dtype) {
  __shared__ __attribute__((aligned(16))) int red[S * 256];
  decode_splitk_tile<LV, S>(d, d.xq, d.s_a, scale_f16, y_dtype, red);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// 64-channel waves when they alone give at least two workgroups per CU
// (N >= 131072); else one 16-channel tile per workgroup with K split over
// S = 4, 8 or 16 waves by the number of K chunks, so that each wave has about
// two chunks: the whole weight stream of a LLaMA-sized call is in flight at
// once. Each call of a LLaMA-7B-shaped stack (weights from HBM) in one HIP
// graph: 4096 x 4096 4.3 us (S = 8), 4096 -> 11008 6.1 us (S = 8; 6.3 with
// S = 4), 11008 -> 4096 5.8 us (S = 16; 6.9 with S = 8).
constexpr int64_t kDecodeWideMinTiles = 512;

template <int LV>
hipError_t launch_decode_splitk(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                hipStream_t s) {
  using F = Fmt<LV>;
  const dim3 grid((unsigned)((d.N + 15) / 16));
  const int64_t nchunks = (d.K + F::kChunkK - 1) / F::kChunkK;
  const int S = nchunks <= 8 ? 4 : nchunks <= 16 ? 8 : 16;
  if (S == 4)
    hipLaunchKernelGGL((linear_decode_splitk_kernel<LV, 4>), grid, dim3(256), 0, s, d, scale_f16,
                       y_dtype);
  else if (S == 8)
    hipLaunchKernelGGL((linear_decode_splitk_kernel<LV, 8>), grid, dim3(512), 0, s, d, scale_f16,
                       y_dtype);
  else
    hipLaunchKernelGGL((linear_decode_splitk_kernel<LV, 16>), grid, dim3(1024), 0, s, d,
                       scale_f16, y_dtype);
  return hipGetLastError();
}

hipError_t launch_linear_decode(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                hipStream_t s) {
  const int64_t tiles = (d.N + kDecodeRowsPerTile - 1) / kDecodeRowsPerTile;
  if (tiles < kDecodeWideMinTiles) {
    switch (d.levels) {
      case QIFT_LEVELS_MNZ: return launch_decode_splitk<QIFT_LEVELS_MNZ>(d, scale_f16, y_dtype, s);
      case QIFT_LEVELS_POT: return launch_decode_splitk<QIFT_LEVELS_POT>(d, scale_f16, y_dtype, s);
      case QIFT_LEVELS_LUT: return launch_decode_splitk<QIFT_LEVELS_LUT>(d, scale_f16, y_dtype, s);
      default: return launch_decode_splitk<QIFT_LEVELS_INT4>(d, scale_f16, y_dtype, s);
    }
  }
  hipLaunchKernelGGL(linear_decode_kernel, dim3((unsigned)tiles), dim3(256), 0, s, d, scale_f16,
                     y_dtype);
  return hipGetLastError();
}

hipError_t launch_linear_grouped(const void* workspace, int64_t total_tiles, int, int,
                                 hipStream_t s) {
  hipLaunchKernelGGL(linear_grouped_kernel, dim3((unsigned)total_tiles), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(workspace));
  return hipGetLastError();
}

}  // namespace qift
