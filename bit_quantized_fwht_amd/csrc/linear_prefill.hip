// The rotated W2A4 linear, prefill side (M > 16): Y = (q . level^T) * s_a *
// s_w * kappa with an exact int32 accumulator (Qift abstract: decoded weight
// application of the no-zero two-bit level sets, per-channel scale, 4-bit
// activations).
//
// 128x128 output tiles on v_mfma_i32_16x16x64_i8; packed operands are staged
// through LDS and unpacked into matrix-core operands in registers.
#include <type_traits>

#include "linear_common.h"

namespace qift {

#ifndef QIFT_PREFILL_MINBLOCKS
#define QIFT_PREFILL_MINBLOCKS 2
#endif

// ---------------------------------------------------------------------------
// prefill: M > 16
// ---------------------------------------------------------------------------

// General path (K a multiple of 64, tokens staged through registers):
// workgroup = 2 x 2 waves; a wave computes kWaveTM x kWaveTN fragments of
// 16 x 16, so the workgroup tile is (32 kWaveTM) tokens x (32 kWaveTN)
// channels. Larger wave tiles amortize the operand unpacking (about 6 VALU
// instructions per activation fragment and 7 per weight fragment per MFMA
// step) over more MFMAs.
constexpr int kWaveTM = 4, kWaveTN = 4;
constexpr int kBM = 32 * kWaveTM, kBN = 32 * kWaveTN;

template <int LV>
struct PrefillCfg {
  using F = Fmt<LV>;
  static constexpr int kBK = F::kChunkK;                  // features per LDS stage
  static constexpr int kARowBytes = kBK / 2;              // int4 activations
  // padded by 8 bytes: the 8-byte reads of 16 consecutive rows cover all 32
  // banks once
  static constexpr int kAStride = kARowBytes + 8;
  static constexpr int kAUnits = kARowBytes / 16;         // 16-byte units per row
  static constexpr int kALoads = kBM * kAUnits / 256;     // 16-byte loads per thread
  // weights: one 1 KB tiled chunk per 16-channel tile, copied verbatim
  static constexpr int kBLoads = (kBN / 16) * 64 / 256;
  // one stage = A tile then B tile
  static constexpr int kBOffset = (kBM * kAStride + 15) / 16 * 16;
  static constexpr int kStage = kBOffset + (kBN / 16) * 1024;
  static constexpr int kLds = kStage;
  static_assert(kALoads * 256 == kBM * kAUnits, "A tile load split");
  static_assert(kBLoads * 256 == (kBN / 16) * 64, "B tile load split");
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
  const int wm = (wave >> 1) * (16 * kWaveTM);  // wave offset inside the tile, M side
  const int wn = (wave & 1) * (16 * kWaveTN);   // N side
  const int64_t M = d.M, K = d.K, N = d.N;
  const int64_t cw = F::code_words(K);
  const int64_t tiles = (N + 15) >> 4;          // 16-channel weight tiles
  const int64_t arow = K / 2;                   // bytes per activation row
  const OpConsts km = op_consts(d.reserved, lane);
  uint32_t lut[kWaveTN];
  tile_tables<LV>(d, km, scale_f16, [&](int j) { return nt0 + wn + 16 * j + r16; }, lut);
  uint8_t* As = lds;                // stage buffer b: A at b * kStage, B after it
  uint8_t* Bs = lds + C::kBOffset;

  v4i acc[kWaveTM][kWaveTN];
#pragma unroll
  for (int i = 0; i < kWaveTM; ++i)
#pragma unroll
    for (int j = 0; j < kWaveTN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // global -> registers for one stage. Out-of-range units load from the
  // tile origin (always valid) and are zeroed afterwards, so the loads need
  // no branches.
  uint4 ra[C::kALoads], rb[C::kBLoads];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i) {
      const int u = tid + 256 * i;
      const int row = u / C::kAUnits, ch = u % C::kAUnits;
      const int64_t m = m0 + row;
      const int64_t kb = k0 / 2 + 16 * ch;  // byte offset in the row
      const bool ok = m < M && 2 * kb < K;
      const uint4 v = ld16(d.xq + (ok ? m * arow + kb : 0));
      ra[i] = ok ? v : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i) {
      const int u = tid + 256 * i;       // 16-byte unit: tile u / 64, lane u % 64
      const int64_t tn = nt0 + 16 * (u >> 6);
      const int ul = u & 63;
      const bool ok = tn < N && k0 + (int64_t)(ul >> 4) * F::kLaneK < K;
      const int64_t c = k0 / C::kBK;       // chunk (16 words per channel unless last)
      const int64_t uc = cw - 16 * c < 16 ? cw - 16 * c : 16;
      const uint4 v = ld16(d.codes + (ok ? c * 256 * tiles + (tn >> 4) * 16 * uc + 4 * ul : 0));
      rb[i] = ok ? v : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* as = As + buf * C::kStage;
    uint8_t* bs = Bs + buf * C::kStage;
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i) {
      const int u = tid + 256 * i;
      const int row = u / C::kAUnits, ch = u % C::kAUnits;
      uint2* dst = reinterpret_cast<uint2*>(as + row * C::kAStride + 16 * ch);
      dst[0] = uint2{ra[i].x, ra[i].y};
      dst[1] = uint2{ra[i].z, ra[i].w};
    }
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i)
      *reinterpret_cast<uint4*>(bs + 16 * (tid + 256 * i)) = rb[i];
  };
  auto compute = [&](int buf) {
    const uint8_t* as = As + buf * C::kStage;
    const uint8_t* bs = Bs + buf * C::kStage;
    // this lane's weight units for the stage (16 bytes per fragment)
    uint4 fb[kWaveTN];
#pragma unroll
    for (int j = 0; j < kWaveTN; ++j)
      fb[j] = *reinterpret_cast<const uint4*>(bs + ((wn >> 4) + j) * 1024 + 16 * lane);
#pragma unroll
    for (int s = 0; s < F::kSteps; ++s) {
      // activation fragments of this step: 8 bytes = 16 features per lane
      v4i A[kWaveTM];
#pragma unroll
      for (int i = 0; i < kWaveTM; ++i) {
        const uint2 a = *reinterpret_cast<const uint2*>(
            as + (wm + 16 * i + r16) * C::kAStride + g * (F::kLaneK / 2) + 8 * s);
        A[i] = int4_operand(a.x, a.y);
      }
#pragma unroll
      for (int j = 0; j < kWaveTN; ++j) {
        const v4i B = weight_operand<LV>(fb[j], s, km, lut[j]);
#pragma unroll
        for (int i = 0; i < kWaveTM; ++i) acc[i][j] = mfma16(A[i], B, acc[i][j]);
      }
    }
  };

  const int64_t nstages = (K + C::kBK - 1) / C::kBK;
  // one LDS stage; the next stage's global loads are in flight in registers
  // while the current stage computes
  gload(0);
  for (int64_t st = 0; st < nstages; ++st) {
    __syncthreads();  // previous stage's LDS reads are done
    lstore(0);
    __syncthreads();
    if (st + 1 < nstages) gload((st + 1) * C::kBK);
    compute(0);
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

// ---------------------------------------------------------------------------
// prefill, direct-to-LDS path (K a multiple of 256)
//
// Workgroup tile 128 tokens x 128 channels. Stages of 256 features are
// double-buffered in LDS and filled with gfx950's global_load_lds_dwordx4
// (each lane's 16 bytes land at base + 16 * lane), so the next stage streams
// in while the current one computes, with one barrier per stage and no
// staging registers. Activation rows (128 bytes per stage) are stored
// unpadded with an XOR swizzle (slot of 16-byte unit c in row r is
// c ^ ((r / 2) % 8)); weight tiles are copied verbatim, their tiled layout
// already being lane order.
//
// Split K inside the workgroup: each wave sums a 128 x 64 block over half of
// every stage's features (waves 0, 1: one half; waves 2, 3: the other). A
// weight operand is then unpacked once per workgroup and reused by 8 MFMAs,
// an activation operand twice and reused by 4: about 2.5 VALU instructions per
// MFMA for the 2-bit formats against 3.3 for 2 x 2 waves of 64 x 64 blocks.
// The two waves of a column block finally swap halves of their partial sums
// through LDS, so that each wave adds up and stores one 64 x 64 block.
// ---------------------------------------------------------------------------

constexpr int kDlBN = 128;  // workgroup tile: 16 RB tokens x 128 channels

// Epilogue staging (defined with the epilogue below): 32 rows of 68 words per
// wave.
constexpr int kEpiStride = 68;                        // words per staged row
constexpr int kEpiWaveBytes = 32 * kEpiStride * 4;    // 8704 B per wave

// RB: 16-row blocks per wave and workgroup tile (8: 128 x 128 tiles; 4: 64 x
// 128 tiles for launches whose 128 x 128 tiles would not fill the GPU).
template <int LV, int RB>
struct DlCfg {
  static_assert(RB == 8 || RB == 4, "128- or 64-row tiles");
  static constexpr bool kInt4 = LV == QIFT_LEVELS_INT4;
  static constexpr int kBM = 16 * RB;
  static constexpr int kStageK = 256;
  static constexpr int kABytes = kBM * 128;                         // 16 or 8 KB
  static constexpr int kBChunks = kInt4 ? 2 : 1;                     // 1 KB chunks per tile
  static constexpr int kBBytes = (kDlBN / 16) * kBChunks * 1024;    // 8 or 16 KB
  static constexpr int kStage = kABytes + kBBytes;
  static constexpr int kLds = 2 * kStage > 4 * kEpiWaveBytes ? 2 * kStage : 4 * kEpiWaveBytes;
  static constexpr int kAInstr = kABytes / 1024 / 4;                // per wave per stage
  static constexpr int kBInstr = kBBytes / 1024 / 4;
};

// 16 bytes per lane from global memory straight into LDS at
// lds_wave_base + 16 * lane (lds_wave_base must be the same for the whole wave)
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void gl_lds16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}

// Epilogue of a wave's 64 x 64 block. The accumulators sit in MFMA output
// order (a lane holds 4 rows of one column per 16 x 16 tile), which would make
// every global store a 4-row scatter of 4-byte pieces. The block is instead
// staged through a wave-private LDS region, 32 rows at a time, as int32 rows
// padded to 68 words, and read back row-major so that each lane owns 4 (float32,
// int32) or 8 (bfloat16) consecutive columns of one row and stores them as one
// 16-byte piece; the scales are applied after the transpose, from LDS tables
// of the tile's activation scales (sa_t, by row) and channel scales times
// kappa (sw_t, by column) that were fetched when the tile started. The output
// is written once and not read back by this kernel: non-temporal stores
// (2-5% faster on the largest outputs).
// The output type and the accumulator rows (I0 .. I0 + 3 of an accumulator
// array of NI rows) are fixed at compile time, so that the row loop unrolls
// and no register is selected at run time.
template <int LV, int YD, int NI, int I0, int NP>
__device__ __forceinline__ void epilogue_blk(const qift_linear_desc& d, const v4i (&acc)[NI][4],
                                             int64_t mb, int64_t nb, const float* sa_t,
                                             const float* sw_t, uint8_t* lds_w, int lane) {
  using F = Fmt<LV>;
  constexpr bool kBf = YD == QIFT_BF16;
  constexpr int kCpl = kBf ? 8 : 4;     // columns per lane
  constexpr int kLpr = 64 / kCpl;       // lanes per staged row
  constexpr int kRstep = 64 / kLpr;     // rows covered by one read of the wave
  int* st = reinterpret_cast<int*>(lds_w);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t M = d.M, N = d.N;
  const int c0 = (lane % kLpr) * kCpl;
  const int rsub = lane / kLpr;
  const int64_t n = nb + c0;
  float sw[kCpl];
  if constexpr (YD != QIFT_I32) {
#pragma unroll
    for (int e = 0; e < kCpl; ++e) sw[e] = sw_t[c0 + e];
  }
  const bool vec = (N % kCpl) == 0 && n + kCpl <= N &&
                   (reinterpret_cast<uintptr_t>(d.Y) & 15) == 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st[(16 * ii + 4 * g + r) * kEpiStride + 16 * j + r16] =
              acc[I0 + 2 * p + ii][j][r] >> F::kShift;
    // one wave writes and reads its own region: its LDS operations complete in order
#pragma unroll
    for (int tr = 0; tr < 32 / kRstep; ++tr) {
      const int row = rsub + kRstep * tr;
      const int64_t m = mb + 32 * p + row;
      int v[kCpl];
#pragma unroll
      for (int q = 0; q < kCpl; q += 4)
        *reinterpret_cast<int4*>(&v[q]) =
            *reinterpret_cast<const int4*>(&st[row * kEpiStride + c0 + q]);
      if (m >= M) continue;
      const int64_t o = m * N + n;
      if constexpr (YD == QIFT_I32) {
        int* y = reinterpret_cast<int*>(d.Y) + o;
        if (vec) {
          __builtin_nontemporal_store(v4u{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]},
                                      reinterpret_cast<v4u*>(y));
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < N) y[e] = v[e];
        }
      } else {
        const float sa = sa_t[32 * p + row];
        float y[kCpl];
#pragma unroll
        for (int e = 0; e < kCpl; ++e) y[e] = (float)v[e] * (sa * sw[e]);
        if constexpr (kBf) {
          uint16_t* yo = reinterpret_cast<uint16_t*>(d.Y) + o;
          if (vec) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
            __builtin_nontemporal_store(v4u{w[0], w[1], w[2], w[3]}, reinterpret_cast<v4u*>(yo));
          } else {
            for (int e = 0; e < 8; ++e)
              if (n + e < N) yo[e] = float_to_bf16_bits(y[e]);
          }
        } else {
          float* yo = reinterpret_cast<float*>(d.Y) + o;
          if (vec) {
            __builtin_nontemporal_store(v4u{__float_as_uint(y[0]), __float_as_uint(y[1]),
                                            __float_as_uint(y[2]), __float_as_uint(y[3])},
                                        reinterpret_cast<v4u*>(yo));
          } else {
            for (int e = 0; e < 4; ++e)
              if (n + e < N) yo[e] = y[e];
          }
        }
      }
    }
  }
}

template <int LV, int NI, int I0, int NP>
__device__ __forceinline__ void epilogue_any(const qift_linear_desc& d, const v4i (&acc)[NI][4],
                                             int64_t mb, int64_t nb, const float* sa_t,
                                             const float* sw_t, int y_dtype, uint8_t* lds_w,
                                             int lane) {
  if (y_dtype == QIFT_BF16)
    epilogue_blk<LV, QIFT_BF16, NI, I0, NP>(d, acc, mb, nb, sa_t, sw_t, lds_w, lane);
  else if (y_dtype == QIFT_I32)
    epilogue_blk<LV, QIFT_I32, NI, I0, NP>(d, acc, mb, nb, sa_t, sw_t, lds_w, lane);
  else
    epilogue_blk<LV, QIFT_F32, NI, I0, NP>(d, acc, mb, nb, sa_t, sw_t, lds_w, lane);
}

// A-tile slot of 16-byte unit c in row r: rows r and r + 1 share a swizzle
// so that the 16 rows read by one 16-lane phase of a 16-byte LDS read land in
// 16 different 16-byte bank groups (the row pitch is 128 B, two rows per
// 256-byte bank line).
__device__ __forceinline__ int sk_slot(int c, int row) { return c ^ ((row >> 1) & 7); }

template <int LV, int RB>
__device__ __forceinline__ void prefill_tile_sk(const qift_linear_desc& d, int64_t m0,
                                                int64_t nt0, int scale_f16, int y_dtype,
                                                uint8_t* lds, float* scl) {
  using C = DlCfg<LV, RB>;
  constexpr int kHalf = RB / 2;          // row blocks each wave keeps after the swap
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int kh = wave >> 1;              // which half of each stage's features
  const int wn = (wave & 1) * 64;        // the wave's 64 channels in the tile
  const int64_t M = d.M, K = d.K, N = d.N;
  const int64_t arow = K / 2;
  const int64_t np16 = (N + 15) >> 4;
  const OpConsts km = op_consts(d.reserved, lane);
  uint32_t lut[4];
  tile_tables<LV>(d, km, scale_f16, [&](int j) { return nt0 + wn + 16 * j + r16; }, lut);

  int64_t a_off[C::kAInstr];
#pragma unroll
  for (int p = 0; p < C::kAInstr; ++p) {
    const int row = 8 * (wave * C::kAInstr + p) + (lane >> 3);
    int64_t m = m0 + row;
    m = m < M ? m : M - 1;                // rows past M only feed discarded outputs
    const int c = sk_slot(lane & 7, row);
    a_off[p] = m * arow + 16 * c;
  }
  int64_t b_off[C::kBInstr];
#pragma unroll
  for (int p = 0; p < C::kBInstr; ++p) {
    const int unit_blk = wave * C::kBInstr + p;
    const int tile = unit_blk / C::kBChunks, chunk = unit_blk % C::kBChunks;
    int64_t t = (nt0 >> 4) + tile;
    t = t < np16 ? t : np16 - 1;          // tiles past N only feed discarded outputs
    b_off[p] = chunk * 256 * np16 + t * 256 + 4 * lane;  // full chunks: K % 256 == 0
  }
  auto issue = [&](int64_t st, int buf) {
    uint8_t* as = lds + buf * C::kStage;
    uint8_t* bs = as + C::kABytes;
#pragma unroll
    for (int p = 0; p < C::kAInstr; ++p)
      gl_lds16(d.xq + a_off[p] + st * 128, as + (wave * C::kAInstr + p) * 1024);
#pragma unroll
    for (int p = 0; p < C::kBInstr; ++p)
      gl_lds16(d.codes + b_off[p] + st * C::kBChunks * 256 * np16,
               bs + (wave * C::kBInstr + p) * 1024);
  };

  // written first by the first stage's MFMAs, whose accumulator input is
  // the constant 0 (no separate zeroing of the accumulators per tile)
  v4i acc[RB][4];

  // int4 weights: the lane's 16-byte unit of chunk kh (32 features, two
  // steps); 2-bit weights: words 2 kh, 2 kh + 1 of the lane's 16-byte unit.
  using BFrag = typename std::conditional<C::kInt4, uint4, uint2>::type;
  struct Frag {
    uint4 a[RB];
    BFrag b[4];
  };
  // reads all of a stage's fragments before the next stage's loads are
  // issued (the compiler would otherwise wait for those loads first)
  auto fetch = [&](int buf, Frag& f) {
    __builtin_amdgcn_s_setprio(1);
    const uint8_t* as = lds + buf * C::kStage;
    const uint8_t* bs = as + C::kABytes;
    const int c = C::kInt4 ? 4 * kh + g : 2 * g + kh;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      // accumulator i <- row block i + RB/2 kh
      const int row = 16 * ((i + kHalf * kh) & (RB - 1)) + r16;
      f.a[i] = *reinterpret_cast<const uint4*>(as + row * 128 + 16 * sk_slot(c, row));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tile = (wn >> 4) + j;
      if constexpr (C::kInt4)
        f.b[j] = *reinterpret_cast<const uint4*>(bs + (tile * 2 + kh) * 1024 + 16 * lane);
      else
        f.b[j] = *reinterpret_cast<const uint2*>(bs + tile * 1024 + 16 * lane + 8 * kh);
    }
  };
  // Wave priorities (s_setprio; the two workgroups of a CU put two waves on
  // every SIMD): the matrix-core phase of a stage runs at 2, the fragment
  // reads that feed it at 1, everything else (stage waits and barriers, the
  // partial-sum swap, the epilogue) at 0. When both waves of a SIMD can
  // issue, the one in its MFMA phase goes first and keeps the matrix core
  // fed while the other's LDS reads, waits and stores fill its gaps: down_proj
  // 0.48 -> 0.51 and the PoT gate 0.45 -> 0.50 of the int8 peak (one level
  // for both phases was no faster than none).
  auto mma = [&](const Frag& f, bool first) {
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      v4i B[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (C::kInt4)
          B[j] = s2 == 0 ? int4_operand(f.b[j].x, f.b[j].y) : int4_operand(f.b[j].z, f.b[j].w);
        else if constexpr (LV == QIFT_LEVELS_MNZ)
          B[j] = mnz_operand(s2 == 0 ? f.b[j].x : f.b[j].y, km);
        else if constexpr (LV == QIFT_LEVELS_LUT)
          B[j] = lut_operand(s2 == 0 ? f.b[j].x : f.b[j].y, lut[j]);
        else
          B[j] = pot_operand(s2 == 0 ? f.b[j].x : f.b[j].y);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const v4i A = s2 == 0 ? int4_operand(f.a[i].x, f.a[i].y) : int4_operand(f.a[i].z, f.a[i].w);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma16(A, B[j], (first && s2 == 0) ? v4i{0, 0, 0, 0} : acc[i][j]);
      }
      // Issue order: each MFMA followed by two VALU instructions (the unpack
      // of later operands). Issue is in order within a wave, so a burst of
      // back-to-back MFMAs would hold the following unpack work until the
      // last of them has issued; interleaved, the unpack runs while the
      // matrix core is busy. 4-5% faster than the compiler's own order.
#pragma unroll
      for (int k = 0; k < 4 * RB; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // the epilogue's scales, fetched now so that their latency is hidden by the
  // main loop: thread t < kBM holds the activation scale of row t of the
  // tile, thread kBM + c the channel scale (times kappa) of column c
  float pre_scale = 0.f;
  {
    const int64_t m = m0 + tid, n = nt0 + (tid - C::kBM);
    if (tid < C::kBM)
      pre_scale = m < M ? d.s_a[m] : 0.f;
    else if (tid < C::kBM + kDlBN)
      pre_scale = n < N ? load_scale(d.scales, n, scale_f16) * level_kappa(LV) : 0.f;
  }

  const int64_t nstages = K / C::kStageK;
  issue(0, 0);
  {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Frag f;
    fetch(0, f);
    if (nstages > 1) issue(1, 1);
    mma(f, true);
  }
  for (int64_t st = 1; st < nstages; ++st) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of stage st have landed
    __syncthreads();                 // ... everyone's; and stage st-1 is consumed
    Frag f;
    fetch((int)(st & 1), f);
    if (st + 1 < nstages) issue(st + 1, (int)((st + 1) & 1));
    mma(f, false);
  }
  if (tid < C::kBM + kDlBN) scl[tid] = pre_scale;  // read after the exchange's barriers

  // Swap halves with the partner wave (same channels, other feature half).
  // Accumulator i of wave kh holds row block (i + RB/2 kh) mod RB, so every
  // wave keeps accumulators 0 .. RB/2 - 1 (its RB/2 row blocks) and sends the
  // others, which are exactly the partner's kept rows; RB/4 rounds of 32 rows
  // (8 KB per wave).
  static_assert(4 * 8 * 64 * 16 <= C::kLds, "partial-sum exchange fits in the stage buffers");
  static_assert(4 * kEpiWaveBytes <= C::kLds, "epilogue staging fits in the stage buffers");
  int4* ex = reinterpret_cast<int4*>(lds);
  const int partner = wave ^ 2;
  __syncthreads();  // every wave is done reading the stage buffers
#pragma unroll
  for (int sp = 0; sp < RB / 4; ++sp) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i v = acc[kHalf + 2 * sp + ii][j];
        ex[(wave * 8 + ii * 4 + j) * 64 + lane] = int4{v[0], v[1], v[2], v[3]};
      }
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int4 r = ex[(partner * 8 + ii * 4 + j) * 64 + lane];
        v4i& a = acc[2 * sp + ii][j];
        a = v4i{a[0] + r.x, a[1] + r.y, a[2] + r.z, a[3] + r.w};
      }
    __syncthreads();
  }
  epilogue_any<LV, RB, 0, RB / 4>(d, acc, m0 + 16 * kHalf * kh, nt0 + wn,
                                  scl + 16 * kHalf * kh, scl + C::kBM + wn, y_dtype,
                                  lds + wave * kEpiWaveBytes, lane);
}

// Tile order: with T tiles and T % 8 == 0, consecutive workgroups (which the
// dispatcher spreads round-robin over the 8 XCDs) are mapped so that each XCD
// works through a contiguous block of tiles, N-tile major, so the weight
// panel of an N-tile and the activation panels stay in that XCD's L2.
__device__ __forceinline__ void dl_tile_of(int64_t b, int64_t nM, int64_t nN, int64_t* tm,
                                           int64_t* tn) {
  const int64_t T = nM * nN;
  int64_t t = b;
  if ((T & 7) == 0) t = (b & 7) * (T >> 3) + (b >> 3);
  *tn = t / nM;
  *tm = t % nM;
}

// 128-row tiles: two workgroups per CU (<= 256 registers per lane) so that
// each SIMD has a second wave to switch to while one waits on LDS or a
// barrier; 64-row tiles: three.
template <int LV, int RB>
__global__ __launch_bounds__(256, RB == 8 ? QIFT_PREFILL_MINBLOCKS : 3) void linear_prefill_sk_kernel(
    qift_linear_desc d, int scale_f16, int y_dtype) {
  using C = DlCfg<LV, RB>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];
  __shared__ float scl[C::kBM + kDlBN];
  const int64_t nM = (d.M + C::kBM - 1) / C::kBM, nN = (d.N + kDlBN - 1) / kDlBN;
  int64_t tm, tn;
  dl_tile_of(blockIdx.x, nM, nN, &tm, &tn);
  prefill_tile_sk<LV, RB>(d, tm * C::kBM, tn * kDlBN, scale_f16, y_dtype, lds, scl);
}

template <int LV>
__global__ __launch_bounds__(256) void linear_prefill_kernel(qift_linear_desc d, int scale_f16,
                                                             int y_dtype) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[PrefillCfg<LV>::kLds];
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  prefill_tile<LV>(d, m0, n0, scale_f16, y_dtype, lds);
}

// workgroup slots of one round of 128-row tiles: two per CU on 256 CUs
constexpr int64_t kPrefillSlots = 512;

hipError_t launch_linear_prefill(const qift_linear_desc& d, int scale_f16, int y_dtype,
                                 hipStream_t s) {
  if (d.K % 256 == 0) {
    // 64-row tiles when 128-row tiles would leave workgroup slots (two per
    // CU) empty
    const int64_t nN = (d.N + kDlBN - 1) / kDlBN;
    const bool small = ((d.M + 127) / 128) * nN < kPrefillSlots;
    const int64_t bm = small ? 64 : 128;
    const dim3 g1((unsigned)(nN * ((d.M + bm - 1) / bm)));
#define QIFT_SK_LAUNCH(LVV)                                                                  \
  if (small)                                                                                 \
    hipLaunchKernelGGL((linear_prefill_sk_kernel<LVV, 4>), g1, dim3(256), 0, s, d, scale_f16, \
                       y_dtype);                                                             \
  else                                                                                       \
    hipLaunchKernelGGL((linear_prefill_sk_kernel<LVV, 8>), g1, dim3(256), 0, s, d, scale_f16, \
                       y_dtype);
    switch (d.levels) {
      case QIFT_LEVELS_MNZ: QIFT_SK_LAUNCH(QIFT_LEVELS_MNZ) break;
      case QIFT_LEVELS_POT: QIFT_SK_LAUNCH(QIFT_LEVELS_POT) break;
      case QIFT_LEVELS_LUT:
      case QIFT_LEVELS_ASYM: QIFT_SK_LAUNCH(QIFT_LEVELS_LUT) break;
      default: QIFT_SK_LAUNCH(QIFT_LEVELS_INT4) break;
    }
#undef QIFT_SK_LAUNCH
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((d.N + kBN - 1) / kBN), (unsigned)((d.M + kBM - 1) / kBM));
  switch (d.levels) {
    case QIFT_LEVELS_MNZ:
      hipLaunchKernelGGL(linear_prefill_kernel<QIFT_LEVELS_MNZ>, grid, dim3(256), 0, s, d,
                         scale_f16, y_dtype);
      break;
    case QIFT_LEVELS_LUT:
    case QIFT_LEVELS_ASYM:
      hipLaunchKernelGGL(linear_prefill_kernel<QIFT_LEVELS_LUT>, grid, dim3(256), 0, s, d,
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

}  // namespace qift
