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
#include <type_traits>

#include "linear_common.h"
#include "rotate_row.h"

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
  const v4u v = __builtin_nontemporal_load(as_global(reinterpret_cast<const v4u*>(p)));
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
  uint32_t lut[kDecodeTiles];
  tile_tables<LV>(d, km, scale_f16, [&](int i) { return n0 + 16 * i + r16; }, lut);

  v4i acc[kDecodeTiles];
#pragma unroll
  for (int i = 0; i < kDecodeTiles; ++i) acc[i] = v4i{0, 0, 0, 0};

  const int64_t nchunks = (K + F::kChunkK - 1) / F::kChunkK;

  // one K chunk of this lane: its 16-byte code unit of each tile and the
  // matching 32 (or 16) bytes of its activation row. Within a chunk every
  // load is issued for every lane (a slot outside the operands reads a
  // clamped valid address): a load under a per-lane branch makes the compiler
  // wait for it where the branch ends, which would serialize the chunks meant
  // to be in flight. What such a slot reads is never used: a tile past N and
  // an activation row past M only feed outputs that are not stored, and a
  // segment past K (a partial last chunk) has its activation operand zeroed
  // through am. Chunks past the last are skipped by wave-uniform branches
  // (clamping them would send every wave to one cache line).
  struct Chunk {
    uint4 c[kDecodeTiles];
    uint4 a0, a1;
    uint32_t am;
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
      // a tile past N reads the wave's first tile again
      const int64_t tn = n0 + 16 * i < N ? n0 + 16 * i : n0;
      ch.c[i] = ld16_stream(kval ? cbase + (tn >> 4) * 16 * ut : codes + 4 * lane);
    }
    const uint8_t* ap = xq + (act_row ? (int64_t)r16 * (K / 2) : 0) + (kval ? kseg / 2 : 0);
    ch.a0 = ld16(ap);
    ch.a1 = F::kInt4 ? ch.a0 : ld16(ap + 16);
    ch.am = kval ? 0xF0F0F0F0u : 0u;
  };
  auto compute = [&](const Chunk& ch) {
#pragma unroll
    for (int s = 0; s < F::kSteps; ++s) {
      const v4i A = act_operand(ch.a0, ch.a1, s, ch.am);
#pragma unroll
      for (int i = 0; i < kDecodeTiles; ++i)
        acc[i] = mfma16(A, weight_operand<LV>(ch.c[i], s, km, lut[i]), acc[i]);
    }
  };
  // two chunks in flight: the loads of chunk t+1 are issued before chunk t
  // is consumed
  Chunk x, y;
  load(x, 0);
  // epilogue operands (lane -> channels n0 + c0 .. + 3 of rows 4 p + lane / 16),
  // fetched now so their latency overlaps the stream; clamped indices
  const float kappa = level_kappa(LV);
  const int c0 = 4 * (lane & 15);
  const int64_t n = n0 + c0;
  float sw[4], sa[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    sw[e] = load_scale_nb(d.scales, n + e < N ? n + e : N - 1, scale_f16) * kappa;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int m = 4 * p + (lane >> 4);
    sa[p] = *as_global(d.s_a + (m < M ? m : M - 1));
  }
  // steady state: pairs of chunks with the next pair's first chunk in range,
  // no branch between a prefetch and the use of the chunk before it (so the
  // compiler can wait for exactly the older loads); then the last one or two
  int64_t t = 0;
  for (; t + 2 < nchunks; t += 2) {
    load(y, t + 1);
    compute(x);
    load(x, t + 2);
    compute(y);
  }
  // (one branch on the second chunk, so both loads are in flight before the
  // first is used; arms that both computed x would have that hoisted above
  // the second load)
  const bool two = t + 1 < nchunks;
  if (two) load(y, t + 1);
  compute(x);
  if (two) compute(y);

  // Epilogue. The lane holds rows m = 4g + r of channels n0 + 16 i + r16 (MFMA
  // order), so direct stores would write 64-byte halves of cache lines, four
  // rows apart (20% of the launch at M = 16). The wave's 16 x 64 block goes
  // through its own LDS region instead and is stored row-major: each lane then
  // owns 4 consecutive channels of one row and writes them as one piece,
  // non-temporal (the output is not read back by this launch: at M = 16, 44
  // MB of bfloat16 outputs interleaved with the weight stream; 5% faster
  // there, 2% at M = 8).
#pragma unroll
  for (int i = 0; i < kDecodeTiles; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      epi[(4 * g + r) * kDecEpiStride + 16 * i + r16] = acc[i][r] >> F::kShift;
  // one wave writes and reads its own region: its LDS operations complete in order
  const bool vec = (N & 3) == 0 && n + 4 <= N && (reinterpret_cast<uintptr_t>(d.Y) & 15) == 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int m = 4 * p + (lane >> 4);
    if (m >= M) continue;
    const int4 v = *reinterpret_cast<const int4*>(&epi[m * kDecEpiStride + c0]);
    const int a[4] = {v.x, v.y, v.z, v.w};
    const int64_t o = (int64_t)m * N + n;
    if (y_dtype == QIFT_I32) {
      auto y = as_global_out(reinterpret_cast<int*>(d.Y) + o);
      if (vec) {
        st16_nt(reinterpret_cast<int*>(d.Y) + o, v.x, v.y, v.z, v.w);
      } else {
        for (int e = 0; e < 4; ++e)
          if (n + e < N) y[e] = a[e];
      }
    } else {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (float)a[e] * (sa[p] * sw[e]);
      if (y_dtype == QIFT_BF16) {
        auto yo = as_global_out(reinterpret_cast<uint16_t*>(d.Y) + o);
        if (vec) {
          st8_nt(reinterpret_cast<uint16_t*>(d.Y) + o, pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yo[e] = float_to_bf16_bits(y[e]);
        }
      } else {
        auto yo = as_global_out(reinterpret_cast<float*>(d.Y) + o);
        if (vec) {
          st16_nt(reinterpret_cast<float*>(d.Y) + o, __float_as_uint(y[0]), __float_as_uint(y[1]),
               __float_as_uint(y[2]), __float_as_uint(y[3]));
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
    case QIFT_LEVELS_LUT:
    case QIFT_LEVELS_ASYM: decode_wave<QIFT_LEVELS_LUT>(d, n0, scale_f16, y_dtype, lane, epi); break;
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

// A linear call on its own (not grouped) has N / 256 workgroups of 64-channel
// waves, 16 for N = 4096: 16 of 256 CUs would carry its whole weight stream.
// Here a workgroup owns G consecutive 16-channel tiles and its S waves take
// every S-th K chunk (wave w: chunks w, w + S, ...), each with two chunks in
// flight; the S partial int32 blocks of each tile are summed through LDS
// (integer sums, so the result is the same as one wave walking all of K).
// G > 1 keeps a large call within one round of resident workgroups (a
// workgroup that ends after two chunks per wave would otherwise be followed
// by 2-3 more rounds, each paying the memory latency again). The epilogue's
// scales are fetched right after the first weight loads are issued, so their
// latency overlaps the stream instead of following the reduction.
// The activation row of a call with the rotation folded in (M = 1): each
// workgroup rotates and quantizes it into LDS itself (the same arithmetic as
// the rotation kernels), so the call needs no separate rotation launch and
// the row's latency overlaps the weight stream.
struct FusedRow {
  const void* X;   // [1, K] float32 or bfloat16
  int log2b;       // log2 of the Hadamard block
  float norm;      // 1 / sqrt(block)
  uint8_t* xq;     // LDS: [K / 2] int4 codes of the row
  float* s;        // LDS: its scale
  float* row;      // LDS: the padded row of the rotation (blocks above 256)
  float* red;      // LDS: one float per wave
};

// XT: void when the activations come quantized in d.xq / d.s_a; the dtype of
// X (uint16_t for bfloat16, float) when the workgroup rotates them itself.
template <int LV, int S, int G, typename XT>
__device__ __forceinline__ void decode_splitk_tiles(const qift_linear_desc& d, int scale_f16,
                                                    int y_dtype, int* red, const FusedRow& fr) {
  using F = Fmt<LV>;
  constexpr bool kFused = !std::is_same<XT, void>::value;
  constexpr int NT = 64 * S;
  // red: partial block of wave w for tile i: rows m, columns c at
  // 256 (w G + i) + 16 m + c
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int64_t M = d.M, K = d.K, N = d.N;
  const int64_t cw = F::code_words(K);
  const int64_t tiles = (N + 15) >> 4;
  const int64_t tn0 = (int64_t)blockIdx.x * G;  // first 16-channel tile of the workgroup
  const int64_t nchunks = (K + F::kChunkK - 1) / F::kChunkK;
  const bool act_row = r16 < M;
  const OpConsts km = op_consts(d.reserved, lane);
  uint32_t lut[G];
  tile_tables<LV>(d, km, scale_f16, [&](int i) { return (tn0 + i) * 16 + r16; }, lut);
  const int64_t t0 = wave;  // the wave's chunks are t0, t0 + S, ...

  // chunk t of the workgroup's tiles: the lane's 16-byte code unit of each
  // (chunk-major tiled layout: chunk t of tile tn at t * 256 * tiles +
  // tn * 16 * ut words) and the matching 32 (or 16) bytes of its activation
  // row. As in decode_wave, every load of a chunk is issued for every lane
  // from a clamped valid address (a chunk past the last reads the wave's
  // first chunk again, a tile past N the last tile); what such a slot reads
  // is never used, and a segment past K is zeroed through am. With the
  // rotation folded in, the activations are read from LDS when computed.
  struct Chunk {
    uint4 c[G];
    uint4 a0, a1;
    uint32_t ak;  // fused: byte offset of the segment in the LDS row
    uint32_t am;
  };
  auto load = [&](Chunk& ch, int64_t t) {
    const int64_t kseg = t * F::kChunkK + (int64_t)g * F::kLaneK;
    const bool kval = t < nchunks && kseg < K;
    const int64_t tl = t < nchunks ? t : (t0 < nchunks ? t0 : 0);
    const int64_t ut = cw - 16 * tl < 16 ? cw - 16 * tl : 16;
    const uint32_t* cb = d.codes + tl * 256 * tiles + 4 * lane;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t tn = tn0 + i < tiles ? tn0 + i : tiles - 1;
      ch.c[i] = ld16_stream(cb + tn * 16 * ut);
    }
    if constexpr (kFused) {
      ch.ak = kval ? (uint32_t)(kseg / 2) : 0u;
    } else {
      const uint8_t* ap = d.xq + (act_row ? (int64_t)r16 * (K / 2) : 0) + (kval ? kseg / 2 : 0);
      ch.a0 = ld16(ap);
      ch.a1 = F::kInt4 ? ch.a0 : ld16(ap + 16);
    }
    ch.am = kval ? 0xF0F0F0F0u : 0u;
  };
  v4i acc[G];
#pragma unroll
  for (int i = 0; i < G; ++i) acc[i] = v4i{0, 0, 0, 0};
  auto compute = [&](const Chunk& ch) {
    uint4 a0 = ch.a0, a1 = ch.a1;
    if constexpr (kFused) {
      a0 = *reinterpret_cast<const uint4*>(fr.xq + ch.ak);
      a1 = F::kInt4 ? a0 : *reinterpret_cast<const uint4*>(fr.xq + ch.ak + 16);
    }
#pragma unroll
    for (int s = 0; s < F::kSteps; ++s) {
      const v4i A = act_operand(a0, a1, s, ch.am);
#pragma unroll
      for (int i = 0; i < G; ++i) acc[i] = mfma16(A, weight_operand<LV>(ch.c[i], s, km, lut[i]), acc[i]);
    }
  };

  // the activation row's loads first (fused): the rotation can start on
  // them while the weight stream is still arriving (the scheduling barriers
  // keep the issue order: row, weights, scales)
  // (one group of 16 elements per thread covers the row: 8 waves take rows of
  // at most 16 chunks, K <= 4096, and 16 waves any K up to 16384)
  static_assert(!kFused || 16 * NT >= (S == 16 ? QIFT_MAX_ROW : 16 * F::kChunkK),
                "one group per thread");
  uint32_t xraw[1][16];
  if constexpr (kFused) {
    rotate_row_load<XT, NT, 1>(reinterpret_cast<const XT*>(fr.X), (int)K, xraw);
    __builtin_amdgcn_sched_barrier(0);
  }

  // NC chunks at a time (4 / G, so 4 tile units are held per wave), all
  // loads issued before any is used: a call with at most NC chunks per wave
  // requests its whole weight stream at the start; longer K repeats this in
  // groups. The first group is loaded without branches (clamped), so
  // nothing makes the compiler wait for it before the rotation.
  // (16 waves: 4 / G units, which keeps them within their registers; 8
  // waves: at least two chunks in flight however many tiles)
  constexpr int NC = S == 16 ? 4 / G : (4 / G > 2 ? 4 / G : 2);
  static_assert(NC >= 1, "at least one chunk per wave in flight");
  Chunk buf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) load(buf[c], t0 + c * S);
  if constexpr (kFused) __builtin_amdgcn_sched_barrier(0);

  // epilogue operands of wave w < G (tile tn0 + w): lane -> row m = lane / 4,
  // columns 4 (lane % 4) .. + 3. Every wave issues these loads (clamped
  // indices): under a branch the compiler would wait for them, and for the
  // chunk loads issued before them, at the branch's end.
  const int em = lane >> 2;
  const int64_t en = (tn0 + wave) * 16 + 4 * (lane & 3);
  const bool storer = wave < G && tn0 + wave < tiles && em < M;
  const float kappa = level_kappa(LV);
  float sa = 0.f;
  if constexpr (!kFused) sa = *as_global(d.s_a + (em < M ? em : M - 1));
  float sw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    sw[e] = load_scale_nb(d.scales, en + e < N ? en + e : N - 1, scale_f16) * kappa;

  if constexpr (kFused) {
    __builtin_amdgcn_sched_barrier(0);
    rotate_row_finish<XT, NT, 1>(xraw, (int)K, fr.log2b, fr.norm, fr.xq, fr.s, nullptr, fr.row,
                              fr.red);
    lds_barrier();  // the row's codes and scale, for every wave; the weights stay in flight
    sa = *fr.s;
    // workgroup 0 also writes the row's codes and scale, as the rotation
    // call would
    if (blockIdx.x == 0) {
      for (int64_t i = threadIdx.x; i < K / 32; i += NT) {
        const uint4 w = *reinterpret_cast<const uint4*>(fr.xq + 16 * i);
        st16(const_cast<uint8_t*>(d.xq) + 16 * i, w.x, w.y, w.z, w.w);
      }
      if (threadIdx.x == 0) *as_global_out(const_cast<float*>(d.s_a)) = sa;
    }
  }

  for (int64_t base = t0; base < nchunks; base += NC * S) {
    if (base != t0) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (base + c * S < nchunks) load(buf[c], base + c * S);  // wave-uniform
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (base + c * S < nchunks) compute(buf[c]);
  }

  // partial sums: the lane holds rows 4g + r of column r16 of each tile
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[256 * (wave * G + i) + 16 * (4 * g + r) + r16] = acc[i][r];
  lds_barrier();
  if (!storer) return;
  int a[4] = {0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < S; ++w) {
    const int4 v4 = *reinterpret_cast<const int4*>(&red[256 * (w * G + wave) + 16 * em + 4 * (lane & 3)]);
    a[0] += v4.x;
    a[1] += v4.y;
    a[2] += v4.z;
    a[3] += v4.w;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] >>= F::kShift;
  const int64_t n = en;
  const int64_t o = (int64_t)em * N + n;
  const bool vec = (N & 3) == 0 && n + 4 <= N && (reinterpret_cast<uintptr_t>(d.Y) & 15) == 0;
  if (y_dtype == QIFT_I32) {
    auto yo = as_global_out(reinterpret_cast<int*>(d.Y) + o);
    if (vec) {
      st16(reinterpret_cast<int*>(d.Y) + o, a[0], a[1], a[2], a[3]);
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) yo[e] = a[e];
    }
    return;
  }
  float yv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) yv[e] = (float)a[e] * (sa * sw[e]);
  if (y_dtype == QIFT_BF16) {
    auto yo = as_global_out(reinterpret_cast<uint16_t*>(d.Y) + o);
    if (vec) {
      st8(reinterpret_cast<uint16_t*>(d.Y) + o, pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]));
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) yo[e] = float_to_bf16_bits(yv[e]);
    }
  } else {
    auto yo = as_global_out(reinterpret_cast<float*>(d.Y) + o);
    if (vec) {
      st16(reinterpret_cast<float*>(d.Y) + o, __float_as_uint(yv[0]), __float_as_uint(yv[1]),
           __float_as_uint(yv[2]), __float_as_uint(yv[3]));
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < N) yo[e] = yv[e];
    }
  }
}

template <int LV, int S, int G>
__global__ __launch_bounds__(64 * S) void linear_decode_splitk_kernel(qift_linear_desc d,
                                                                      int scale_f16,
                                                                      int y_dtype) {
  __shared__ __attribute__((aligned(16))) int red[S * G * 256];
  decode_splitk_tiles<LV, S, G, void>(d, scale_f16, y_dtype, red, FusedRow{});
}

// one token row (M = 1) rotated, quantized and applied in one launch; the
// dynamic LDS is the rotation's padded row (K + K / 16 floats) when the
// block exceeds 256
template <int LV, int S, int G, typename XT>
__global__ __launch_bounds__(64 * S) void rotate_linear_decode_kernel(qift_linear_desc d,
                                                                      const XT* __restrict__ X,
                                                                      int log2b, float norm,
                                                                      int scale_f16,
                                                                      int y_dtype) {
  extern __shared__ float rot_row[];
  __shared__ __attribute__((aligned(16))) int red[S * G * 256];
  __shared__ __attribute__((aligned(16))) uint8_t xq_row[QIFT_MAX_ROW / 2];
  __shared__ float s_row;
  __shared__ float rot_red[S];
  const FusedRow fr{X, log2b, norm, xq_row, &s_row, rot_row, rot_red};
  decode_splitk_tiles<LV, S, G, XT>(d, scale_f16, y_dtype, red, fr);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// 64-channel waves when they alone give at least two workgroups per CU
// (N >= 131072); else G 16-channel tiles per workgroup with K split over
// S = 4, 8 or 16 waves by the number of K chunks, so that each wave has about
// two chunks: the whole weight stream of a LLaMA-sized call is in flight at
// once. G is the smallest of 1, 2, 4 that keeps the grid within the
// workgroups resident at once (1024, 512 or 256 for S = 4, 8, 16: 2048
// threads per CU).
constexpr int64_t kDecodeWideMinTiles = 512;

template <int LV, int S>
hipError_t launch_decode_splitk_s(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                  hipStream_t s) {
  const int64_t tiles = (d.N + 15) / 16;
  const int64_t resident = 256 * (2048 / (64 * S));
  int G = 1;
  while (G < 2 && (tiles + G - 1) / G > resident) G *= 2;
  const dim3 grid((unsigned)((tiles + G - 1) / G));
  if (G == 1)
    hipLaunchKernelGGL((linear_decode_splitk_kernel<LV, S, 1>), grid, dim3(64 * S), 0, s, d,
                       scale_f16, y_dtype);
  else if (G == 2)
    hipLaunchKernelGGL((linear_decode_splitk_kernel<LV, S, 2>), grid, dim3(64 * S), 0, s, d,
                       scale_f16, y_dtype);
  else
    hipLaunchKernelGGL((linear_decode_splitk_kernel<LV, S, 4>), grid, dim3(64 * S), 0, s, d,
                       scale_f16, y_dtype);
  return hipGetLastError();
}

// Waves per workgroup: 4 (each wave loads its up to 4 chunks at once) up to
// 16 chunks, 8 beyond (K = 11008: 5-6 chunks per wave). Measured per call on
// weights streamed from HBM (M = 1, one HIP graph of calls): 4096 x 4096
// 3.4 us (S = 4; 4.0 with S = 8), 4096 -> 12288 5.8 us, 4096 -> 22016 8.0 us
// (S = 4, G = 2), 11008 -> 4096 5.9 us (S = 8; 6.6 with S = 4 or 16).
template <int LV>
hipError_t launch_decode_splitk(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                hipStream_t s) {
  using F = Fmt<LV>;
  const int64_t nchunks = (d.K + F::kChunkK - 1) / F::kChunkK;
  if (nchunks <= 16) return launch_decode_splitk_s<LV, 4>(d, scale_f16, y_dtype, s);
  return launch_decode_splitk_s<LV, 8>(d, scale_f16, y_dtype, s);
}

template <int LV, int S, typename XT>
hipError_t launch_rotate_linear_s(const qift_linear_desc& d, const void* X, int log2b, float norm,
                                  int scale_f16, int y_dtype, hipStream_t s) {
  // every workgroup rotates the row again: about one workgroup per CU, so G
  // is the smallest tile count per workgroup that keeps the grid within 256
  // workgroups (8 waves: 1, 2, 3, 4 or 6 tiles; 16 waves: 1, 2 or 4)
  const int64_t tiles = (d.N + 15) / 16;
  static constexpr int kG8[] = {1, 2, 3, 4, 6};
  static constexpr int kG16[] = {1, 2, 4};
  const int* gs = S == 16 ? kG16 : kG8;
  const int ng = S == 16 ? 3 : 5;
  int G = gs[ng - 1];
  for (int i = 0; i < ng; ++i)
    if ((tiles + gs[i] - 1) / gs[i] <= 256) {
      G = gs[i];
      break;
    }
  const dim3 grid((unsigned)((tiles + G - 1) / G));
  const size_t lds = log2b > kRegLog2B ? (size_t)(d.K + d.K / 16) * sizeof(float) : 0;
  const XT* x = reinterpret_cast<const XT*>(X);
#define QIFT_ROT_LIN(GG)                                                                    \
  hipLaunchKernelGGL((rotate_linear_decode_kernel<LV, S, GG, XT>), grid, dim3(64 * S), lds, s, \
                     d, x, log2b, norm, scale_f16, y_dtype)
  if (G == 1) QIFT_ROT_LIN(1);
  else if (G == 2) QIFT_ROT_LIN(2);
  else if (G == 4) QIFT_ROT_LIN(4);
  else if constexpr (S == 8) {
    if (G == 3) QIFT_ROT_LIN(3);
    else QIFT_ROT_LIN(6);
  }
#undef QIFT_ROT_LIN
  return hipGetLastError();
}

template <int LV, typename XT>
hipError_t launch_rotate_linear_lv(const qift_linear_desc& d, const void* X, int log2b,
                                   float norm, int scale_f16, int y_dtype, hipStream_t s) {
  // 8 waves up to 16 chunks, 16 beyond. Measured per fused call (M = 1,
  // weights from HBM): 4096 x 4096 5.4 us, 4096 -> 12288 7.2 us (G = 4),
  // 4096 -> 22016 10.0 us (G = 4), 11008 -> 4096 7.4 us
  using F = Fmt<LV>;
  const int64_t nchunks = (d.K + F::kChunkK - 1) / F::kChunkK;
  // (8 waves hold one 16-element group of the row per thread up to 16 chunks)
  if (nchunks <= 16) return launch_rotate_linear_s<LV, 8, XT>(d, X, log2b, norm, scale_f16, y_dtype, s);
  return launch_rotate_linear_s<LV, 16, XT>(d, X, log2b, norm, scale_f16, y_dtype, s);
}

// the fused decode of one token row (M = 1, K % 16 == 0, block >= 16,
// 16-byte aligned X and xq): d.xq and d.s_a receive the row's codes and scale
hipError_t launch_rotate_linear_decode(const qift_linear_desc& d, const void* X, int x_bf16,
                                       int had_block, int scale_f16, int y_dtype, hipStream_t s) {
  int log2b = 0;
  while ((1 << log2b) < had_block) ++log2b;
  const float norm = (float)(1.0 / __builtin_sqrt((double)had_block));
  if (x_bf16) {
    switch (d.levels) {
      case QIFT_LEVELS_MNZ: return launch_rotate_linear_lv<QIFT_LEVELS_MNZ, uint16_t>(d, X, log2b, norm, scale_f16, y_dtype, s);
      case QIFT_LEVELS_POT: return launch_rotate_linear_lv<QIFT_LEVELS_POT, uint16_t>(d, X, log2b, norm, scale_f16, y_dtype, s);
      case QIFT_LEVELS_LUT:
      case QIFT_LEVELS_ASYM: return launch_rotate_linear_lv<QIFT_LEVELS_LUT, uint16_t>(d, X, log2b, norm, scale_f16, y_dtype, s);
      default: return launch_rotate_linear_lv<QIFT_LEVELS_INT4, uint16_t>(d, X, log2b, norm, scale_f16, y_dtype, s);
    }
  }
  switch (d.levels) {
    case QIFT_LEVELS_MNZ: return launch_rotate_linear_lv<QIFT_LEVELS_MNZ, float>(d, X, log2b, norm, scale_f16, y_dtype, s);
    case QIFT_LEVELS_POT: return launch_rotate_linear_lv<QIFT_LEVELS_POT, float>(d, X, log2b, norm, scale_f16, y_dtype, s);
    case QIFT_LEVELS_LUT:
    case QIFT_LEVELS_ASYM: return launch_rotate_linear_lv<QIFT_LEVELS_LUT, float>(d, X, log2b, norm, scale_f16, y_dtype, s);
    default: return launch_rotate_linear_lv<QIFT_LEVELS_INT4, float>(d, X, log2b, norm, scale_f16, y_dtype, s);
  }
}

hipError_t launch_linear_decode(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                hipStream_t s) {
  const int64_t tiles = (d.N + kDecodeRowsPerTile - 1) / kDecodeRowsPerTile;
  if (tiles < kDecodeWideMinTiles) {
    switch (d.levels) {
      case QIFT_LEVELS_MNZ: return launch_decode_splitk<QIFT_LEVELS_MNZ>(d, scale_f16, y_dtype, s);
      case QIFT_LEVELS_POT: return launch_decode_splitk<QIFT_LEVELS_POT>(d, scale_f16, y_dtype, s);
      case QIFT_LEVELS_LUT:
      case QIFT_LEVELS_ASYM: return launch_decode_splitk<QIFT_LEVELS_LUT>(d, scale_f16, y_dtype, s);
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
