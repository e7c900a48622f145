// The rotated W2A4 linear: Y = (q . level^T) * s_a * s_w * kappa with an exact
// int32 accumulator (Qift abstract: decoded weight application of the no-zero
// two-bit level sets, per-channel scale, 4-bit activations).
//
// Both kernels run on v_mfma_i32_16x16x64_i8. Activations enter the matrix
// core as 16*q (int4 nibble moved to the top half of a byte), 2-bit MNZ codes
// as 32*(2t+1) (two's-complement code in the top two bits, bit 5 set), PoT
// codes as 16*level through a byte table, int4 weights as 16*w; the int32 sum
// is therefore 2^9 (MNZ) or 2^8 times the exact sum q*level and an arithmetic
// shift recovers it. |sum q*level| <= 7*7*65536 keeps every partial sum far
// inside int32.
//
//  decode (M <= 16): the weight stream. A wave owns 64 output channels and
//    walks K; every lane loads 16 bytes of codes per 16-channel tile per
//    step straight into registers (no LDS), unpacks them into operands and
//    issues one MFMA per 16 channels; the 16 rows of the MFMA's other side
//    carry the (at most 16) tokens. The accumulation over K happens inside
//    the matrix core, so no cross-lane reduction is needed.
//  prefill (M > 16): 128x128 output tiles, 4 waves of 64x64, packed operands
//    staged through LDS (padded rows, conflict-free 16-byte reads) with the
//    next K step prefetched into registers while the current one computes.
#include "qift_internal.h"

namespace qift {

// ---------------------------------------------------------------------------
// common pieces
// ---------------------------------------------------------------------------

// features per lane segment: 64 for 2-bit codes (16 bytes = 4 code words),
// 32 for int4 weights (16 bytes = 4 words of 8)
template <int LV>
struct Fmt {
  static constexpr bool kInt4 = LV == QIFT_LEVELS_INT4;
  static constexpr int kLaneK = kInt4 ? 32 : 64;        // features per 16-byte code load
  static constexpr int kSteps = kLaneK / 16;            // MFMAs per code load
  static constexpr int kChunkK = 4 * kLaneK;            // features per wave step (4 lane groups)
  static constexpr int kShift = acc_shift(LV);
  // 32-bit code words per channel row
  __device__ static __forceinline__ int64_t code_words(int64_t K) { return kInt4 ? K / 8 : K / 16; }
};

template <int LV>
__device__ __forceinline__ v4i weight_operand(const uint4& c, int step) {
  if constexpr (LV == QIFT_LEVELS_INT4) {
    const uint32_t w0 = step == 0 ? c.x : c.z;
    const uint32_t w1 = step == 0 ? c.y : c.w;
    return int4_operand(w0, w1);
  } else {
    const uint32_t w = step == 0 ? c.x : (step == 1 ? c.y : (step == 2 ? c.z : c.w));
    if constexpr (LV == QIFT_LEVELS_MNZ) return mnz_operand(w);
    else return pot_operand(w);
  }
}

// activation operand for MFMA step `step` of a lane segment: 2-bit segments
// carry 64 features = 32 bytes (a0, a1), int4-weight segments 32 features =
// 16 bytes (a0 only).
__device__ __forceinline__ v4i act_operand(const uint4& a0, const uint4& a1, int step) {
  switch (step) {
    case 0: return int4_operand(a0.x, a0.y);
    case 1: return int4_operand(a0.z, a0.w);
    case 2: return int4_operand(a1.x, a1.y);
    default: return int4_operand(a1.z, a1.w);
  }
}

__device__ __forceinline__ void store_y(void* Y, int y_dtype, int64_t idx, int acc, float scale) {
  if (y_dtype == QIFT_I32) {
    reinterpret_cast<int*>(Y)[idx] = acc;
  } else {
    const float y = (float)acc * scale;
    if (y_dtype == QIFT_BF16) reinterpret_cast<uint16_t*>(Y)[idx] = float_to_bf16_bits(y);
    else reinterpret_cast<float*>(Y)[idx] = y;
  }
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---------------------------------------------------------------------------
// decode: M <= 16
// ---------------------------------------------------------------------------

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

template <int LV>
__device__ __forceinline__ void decode_wave(const qift_linear_desc& d, int64_t n0, int scale_f16,
                                            int y_dtype, int lane) {
  using F = Fmt<LV>;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t M = d.M, K = d.K, N = d.N;
  const int64_t cw = F::code_words(K);
  const uint8_t* xq = d.xq;
  const uint32_t* codes = d.codes;
  const bool act_row = r16 < M;

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
    // tiled layout: 16-channel tile (n0 + 16 i) / 16, chunk t, the lane's
    // 16-byte unit at word 4 * lane -- one contiguous 1 KB per wave load
#pragma unroll
    for (int i = 0; i < kDecodeTiles; ++i) {
      const int64_t tn = n0 + 16 * i;
      ch.c[i] = (kval && tn < N) ? ld16_stream(codes + (tn >> 4) * 16 * cw + t * 256 + 4 * lane)
                                 : uint4{0u, 0u, 0u, 0u};
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
        acc[i] = mfma16(A, weight_operand<LV>(ch.c[i], s), acc[i]);
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

  // epilogue: lane holds rows m = 4g + r of channel n0 + 16 i + r16
  const float kappa = level_kappa(LV);
#pragma unroll
  for (int i = 0; i < kDecodeTiles; ++i) {
    const int64_t n = n0 + 16 * i + r16;
    if (n >= N) continue;
    const float sw = load_scale(d.scales, n, scale_f16) * kappa;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (m < M) {
        const int a = acc[i][r] >> F::kShift;
        store_y(d.Y, y_dtype, (int64_t)m * N + n, a, d.s_a[m] * sw);
      }
    }
  }
}

__device__ __forceinline__ void decode_dispatch(const qift_linear_desc& d, int64_t tile,
                                                int scale_f16, int y_dtype) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n0 = tile * kDecodeRowsPerTile + (int64_t)wave * kDecodeRowsPerWave;
  if (n0 >= d.N) return;
  switch (d.levels) {
    case QIFT_LEVELS_MNZ: decode_wave<QIFT_LEVELS_MNZ>(d, n0, scale_f16, y_dtype, lane); break;
    case QIFT_LEVELS_POT: decode_wave<QIFT_LEVELS_POT>(d, n0, scale_f16, y_dtype, lane); break;
    default: decode_wave<QIFT_LEVELS_INT4>(d, n0, scale_f16, y_dtype, lane); break;
  }
}

__global__ __launch_bounds__(256) void linear_decode_kernel(qift_linear_desc d, int scale_f16,
                                                            int y_dtype) {
  decode_dispatch(d, blockIdx.x, scale_f16, y_dtype);
}

__global__ __launch_bounds__(256) void linear_grouped_kernel(const uint8_t* __restrict__ ws) {
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(ws);
  const int64_t tile = blockIdx.x;
  if (tile >= h->total_tiles) return;
  const int32_t e = reinterpret_cast<const int32_t*>(ws + h->tile_map_offset)[tile];
  const PlanEntry* pe = reinterpret_cast<const PlanEntry*>(ws + h->entries_offset) + e;
  const qift_linear_desc d = pe->d;
  decode_dispatch(d, tile - pe->tile_begin, h->scale_f16, h->y_dtype);
}

// ---------------------------------------------------------------------------
// prefill: M > 16
// ---------------------------------------------------------------------------

constexpr int kBM = 128, kBN = 128;
constexpr int kWaveTM = 4, kWaveTN = 4;  // 16x16 fragments per wave (64 x 64)

template <int LV>
struct PrefillCfg {
  using F = Fmt<LV>;
  static constexpr int kBK = F::kChunkK;                  // features per LDS stage
  static constexpr int kARowBytes = kBK / 2;              // int4 activations
  static constexpr int kAStride = kARowBytes + 16;        // padded: conflict-free 16 B reads
  static constexpr int kALoads = kBM * kARowBytes / 16 / 256;  // 16-byte loads per thread
  // weights: one 1 KB tiled chunk per 16-channel tile, copied verbatim
  static constexpr int kBLoads = (kBN / 16) * 1024 / 16 / 256;
  static constexpr int kLds = kBM * kAStride + (kBN / 16) * 1024;
};

template <int LV>
__device__ __forceinline__ void prefill_tile(const qift_linear_desc& d, int64_t m0, int64_t nt0,
                                             int scale_f16, int y_dtype, uint8_t* lds) {
  using C = PrefillCfg<LV>;
  using F = typename C::F;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int wm = (wave >> 1) * 64;  // wave offset inside the tile, M side
  const int wn = (wave & 1) * 64;   // N side
  const int64_t M = d.M, K = d.K, N = d.N;
  const int64_t cw = F::code_words(K);
  const int64_t arow = K / 2;       // bytes per activation row
  uint8_t* As = lds;
  uint8_t* Bs = lds + kBM * C::kAStride;

  v4i acc[kWaveTM][kWaveTN];
#pragma unroll
  for (int i = 0; i < kWaveTM; ++i)
#pragma unroll
    for (int j = 0; j < kWaveTN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  uint4 ra[C::kALoads], rb[C::kBLoads];
  constexpr int kAChunks = C::kARowBytes / 16;  // 16-byte chunks per row

  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / kAChunks, ch = idx % kAChunks;
      const int64_t m = m0 + row;
      const int64_t kb = k0 / 2 + 16 * ch;  // byte offset in the row
      ra[i] = (m < M && 2 * kb < K) ? ld16(d.xq + m * arow + kb) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i) {
      const int u = tid + 256 * i;       // 16-byte unit: tile u / 64, lane u % 64
      const int64_t tn = nt0 + 16 * (u >> 6);
      const int ul = u & 63;
      const bool ok = tn < N && k0 + (int64_t)(ul >> 4) * F::kLaneK < K;
      rb[i] = ok ? ld16(d.codes + (tn >> 4) * 16 * cw + (k0 / C::kBK) * 256 + 4 * ul)
                 : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx / kAChunks, ch = idx % kAChunks;
      *reinterpret_cast<uint4*>(As + row * C::kAStride + 16 * ch) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i)
      *reinterpret_cast<uint4*>(Bs + 16 * (tid + 256 * i)) = rb[i];
  };

  const int64_t nstages = (K + C::kBK - 1) / C::kBK;
  gload(0);
  for (int64_t st = 0; st < nstages; ++st) {
    __syncthreads();  // previous stage's LDS reads are done
    lstore();
    __syncthreads();
    if (st + 1 < nstages) gload((st + 1) * C::kBK);
    // fragments of this lane: activations (segment g of each A row), codes
    uint4 fa0[kWaveTM], fa1[kWaveTM], fb[kWaveTN];
#pragma unroll
    for (int i = 0; i < kWaveTM; ++i) {
      const uint8_t* p = As + (wm + 16 * i + r16) * C::kAStride + g * (F::kLaneK / 2);
      fa0[i] = *reinterpret_cast<const uint4*>(p);
      if constexpr (!F::kInt4) fa1[i] = *reinterpret_cast<const uint4*>(p + 16);
      else fa1[i] = uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kWaveTN; ++j)
      fb[j] = *reinterpret_cast<const uint4*>(Bs + ((wn >> 4) + j) * 1024 + 16 * lane);
#pragma unroll
    for (int s = 0; s < F::kSteps; ++s) {
      v4i B[kWaveTN];
#pragma unroll
      for (int j = 0; j < kWaveTN; ++j) B[j] = weight_operand<LV>(fb[j], s);
#pragma unroll
      for (int i = 0; i < kWaveTM; ++i) {
        const v4i A = act_operand(fa0[i], fa1[i], s);
#pragma unroll
        for (int j = 0; j < kWaveTN; ++j) acc[i][j] = mfma16(A, B[j], acc[i][j]);
      }
    }
  }

  const float kappa = level_kappa(LV);
#pragma unroll
  for (int j = 0; j < kWaveTN; ++j) {
    const int64_t n = nt0 + wn + 16 * j + r16;
    if (n >= N) continue;
    const float sw = load_scale(d.scales, n, scale_f16) * kappa;
#pragma unroll
    for (int i = 0; i < kWaveTM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm + 16 * i + 4 * g + r;
        if (m < M) {
          const int a = acc[i][j][r] >> F::kShift;
          store_y(d.Y, y_dtype, m * N + n, a, d.s_a[m] * sw);
        }
      }
    }
  }
}

template <int LV>
__global__ __launch_bounds__(256) void linear_prefill_kernel(qift_linear_desc d, int scale_f16,
                                                             int y_dtype) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[PrefillCfg<LV>::kLds];
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  prefill_tile<LV>(d, m0, n0, scale_f16, y_dtype, lds);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_linear_decode(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                hipStream_t s) {
  const int64_t tiles = (d.N + kDecodeRowsPerTile - 1) / kDecodeRowsPerTile;
  hipLaunchKernelGGL(linear_decode_kernel, dim3((unsigned)tiles), dim3(256), 0, s, d, scale_f16,
                     y_dtype);
  return hipGetLastError();
}

hipError_t launch_linear_prefill(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                 hipStream_t s) {
  const dim3 grid((unsigned)((d.N + kBN - 1) / kBN), (unsigned)((d.M + kBM - 1) / kBM));
  switch (d.levels) {
    case QIFT_LEVELS_MNZ:
      hipLaunchKernelGGL(linear_prefill_kernel<QIFT_LEVELS_MNZ>, grid, dim3(256), 0, s, d,
                         scale_f16, y_dtype);
      break;
    case QIFT_LEVELS_POT:
      hipLaunchKernelGGL(linear_prefill_kernel<QIFT_LEVELS_POT>, grid, dim3(256), 0, s, d,
                         scale_f16, y_dtype);
      break;
    default:
      hipLaunchKernelGGL(linear_prefill_kernel<QIFT_LEVELS_INT4>, grid, dim3(256), 0, s, d,
                         scale_f16, y_dtype);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_linear_grouped(const void* workspace, int64_t total_tiles, int, int,
                                 hipStream_t s) {
  hipLaunchKernelGGL(linear_grouped_kernel, dim3((unsigned)total_tiles), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(workspace));
  return hipGetLastError();
}

}  // namespace qift
