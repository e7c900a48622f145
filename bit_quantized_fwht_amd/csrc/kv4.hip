// KV4 quantizer: every head vector of a [T, H, D] key or value tensor is
// rotated by a block Hadamard transform along D and quantized to int4 with
// its own absmax scale (the "KV4" of rotated W2A4/KV4 inference, Qift
// abstract).
//
// Two kernels: bfloat16 vectors of 64, 128 or 256 elements with a block of
// at least 32 run the transform on the matrix cores (kv4_mfma_kernel, below:
// about 11 vector instructions per element against 16.5); every other case
// runs kv4_kernel, all butterflies.
//
// kv4_kernel's layout on the GPU: a head vector of D elements is held by L = D/E lanes of
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
  // stored * sigma * (norm / s) is within three roundings of x' / s with
  // x' = fl(v * norm) the rotated value (int4x8_rint_fma's margin covers it)
  const float rl = sigma * (norm * rs);
  uint32_t words[E / 8];
  float dmax = 0.f;
#pragma unroll
  for (int w = 0; w < E / 8; ++w) words[w] = int4x8_rint_fma(v + 8 * w, rl, dmax);
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

// ---------------------------------------------------------------------------
// bfloat16 head vectors of D = 32 NCH elements with a block of 2^LB >= 32
// elements: the transform on the matrix cores.
//
// Index bits split the block transform: for e = 32 c + k (chunk c, k < 32)
// and i = 32 c' + i', (-1)^popcount(i & e) = (-1)^popcount(c' & c) *
// (-1)^popcount(i' & k), so H_(2^LB) = H_(2^LB / 32) (x) H_32 over (chunk,
// position in chunk). One v_mfma_f32_16x16x32_bf16 applies H_32 to one
// chunk of 16 head vectors at once (the bfloat16 inputs times +-1 are exact
// products, summed in float32), and LB - 5 butterfly stages across the
// chunks, in each lane's registers, finish the block.
//
// A wave owns a tile of 16 head vectors. Operand B of chunk c is
// X[t][32 c + k], which the MFMA layout gives lane (t = lane % 16, g = lane
// / 16) as k = 8 g .. 8 g + 7: one 16-byte piece of the row. The tile is
// first copied to LDS in contiguous kilobytes (global_load_lds, the pieces
// XOR-swizzled so that the operand reads are conflict-free): 4-6% faster for
// 128- and 256-element vectors than loading the operand pieces straight into
// registers, whose load instructions each cover 64 bytes of 16 vectors. Operand A holds
// 16 rows of H_32 for each half h of the outputs; its row slots are permuted
// (slot p <- output 8 (p / 4) + 4 h + p % 4) so that the four results of
// slot rows 4 g .. 4 g + 3 that the MFMA leaves in lane (t, g) are, over
// both halves, the eight consecutive outputs 8 g .. 8 g + 7 of the chunk:
// one 32-bit word of codes per chunk and lane. The words of a vector are
// regrouped through a wave-private LDS row so that each lane stores NCH
// consecutive words (16 bytes of codes for D = 128, the 16 vectors' codes
// one contiguous kilobyte). Absmax, scale and codes are the same arithmetic
// as in kv4_kernel (sigma = 1).
// ---------------------------------------------------------------------------

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (gfx950 row-pair swaps)
__device__ __forceinline__ float max_lanes_16_32(float m) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr int kKvMfmaWaves = 4;

// One tile of 16 head vectors whose NCH 16-byte operand loads (xb) have been
// issued: transform, quantize and store it.
template <int NCH, int LB>
__device__ __forceinline__ void kv4_mfma_tile(const v4u (&xb)[NCH], const v4u (&ha)[2], int64_t r0,
                                              int64_t rows, float norm, uint8_t* __restrict__ kvq,
                                              float* __restrict__ scales, uint32_t* stage, int t,
                                              int g) {
  constexpr int D = 32 * NCH;
  constexpr int kPitch = 4 * NCH + 4;
  // v[c][j]: output 32 c + 8 g + j of vector t (unnormalized)
  float v[NCH][8];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xb[c]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4f y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, ha[h]), b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[c][4 * h + i] = y[i];
    }
  }
  // butterflies across the chunks of a block (chunk strides 1 .. 2^(LB-6))
#pragma unroll
  for (int st = 0; st < LB - 5; ++st) {
    const int hs = 1 << st;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (!(c & hs)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float a = v[c][j], b = v[c + hs][j];
          v[c][j] = a + b;
          v[c + hs][j] = a - b;
        }
      }
    }
  }

  float m = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[c][j]));
  m = max_lanes_16_32(m);
  m *= norm;  // rounding is monotonic: max(|v|) * norm == max(|v * norm|)
  const float s = __fdiv_rn(m, 7.0f);
  const float rs = s != 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  const float rl = norm * rs;
  uint32_t words[NCH];
  float dmax = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) words[c] = int4x8_rint_fma(v[c], rl, dmax);
  if (!(dmax <= 0.49999f) || !rint_path_ok(rs)) {
    // a value within 1e-5 of a rounding tie (rare): exact division
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = v[c][j] * norm;
      words[c] = int4x8_exact(x, s);
    }
  }

  // word c of lane (t, g) is word 4 c + g of vector t's code row; lane (t, g)
  // stores words NCH g .. NCH g + NCH - 1 (the stage rows are the wave's
  // own: its LDS accesses complete in order)
  uint32_t* st = stage + t * kPitch;
#pragma unroll
  for (int c = 0; c < NCH; ++c) st[4 * c + g] = words[c];
  __builtin_amdgcn_wave_barrier();
  const int64_t r = r0 + t;
  if (r < rows) {
    uint8_t* dst = kvq + r * (D / 2) + 4 * NCH * g;
    if constexpr (NCH == 2) {
      const uint2 o = *reinterpret_cast<const uint2*>(st + 2 * g);
      *reinterpret_cast<uint2*>(dst) = o;
    } else {
#pragma unroll
      for (int q = 0; q < NCH / 4; ++q) {
        const uint4 o = *reinterpret_cast<const uint4*>(st + NCH * g + 4 * q);
        __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w}, reinterpret_cast<v4u*>(dst) + q);
      }
    }
    if (g == 0) scales[r] = s;
  }
}

// The tensors of one launch of the matrix-core kernel: one, or the K and V
// caches of a layer (same shape), each with its codes and scales.
struct KvSet {
  const uint16_t* kv[2];
  uint8_t* q[2];
  float* s[2];
};

// One tile of 16 head vectors per wave. (Waves that walk several tiles with
// the next tile's loads in flight measured 5-10% slower on the LLaMA-shaped
// K and V: the loads of all tiles are in flight at once either way, and a
// streaming probe of the same bytes in the same pattern is only ~20% faster
// than this kernel.)
typedef __attribute__((address_space(3))) void kv_lds_void;

template <int NCH, int LB>
__global__ __launch_bounds__(64 * kKvMfmaWaves) void kv4_mfma_kernel(KvSet set, int64_t rows,
                                                                     int64_t blocks, float norm) {
  static_assert(NCH == 2 || NCH == 4 || NCH == 8, "D = 64, 128 or 256");
  static_assert(LB >= 5 && (1 << LB) <= 32 * NCH, "block between 32 and D");
  constexpr int kPieces = 4 * NCH;     // 16-byte pieces per head vector
  __shared__ __attribute__((aligned(1024))) uint8_t tile_lds[kKvMfmaWaves][1024 * NCH];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = lane & 15, g = lane >> 4;
  // workgroups 0 .. blocks - 1 take tensor 0, the next blocks tensor 1
  const int which = blockIdx.x >= blocks;
  const uint16_t* __restrict__ KV = which ? set.kv[1] : set.kv[0];
  uint8_t* __restrict__ kvq = which ? set.q[1] : set.q[0];
  float* __restrict__ scales = which ? set.s[1] : set.s[0];
  const int64_t r0 = (((int64_t)blockIdx.x - which * blocks) * kKvMfmaWaves + wave) * 16;
  if (r0 >= rows) return;  // uniform over the wave; no workgroup barrier below
  uint8_t* wl = tile_lds[wave];
  // the tile's 16 vectors, one contiguous kilobyte per instruction, straight
  // to LDS: lane l of instruction q fills slot s = 64 q + l (vector s /
  // kPieces, position j = s % kPieces) with piece j ^ (vector % kPieces), so
  // that the operand reads below are conflict-free
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int slot = 64 * q + lane;
    const int tv = slot / kPieces, j = slot % kPieces;
    const int p = j ^ (tv & (kPieces - 1));
    int64_t r = r0 + tv;
    r = r < rows ? r : rows - 1;  // a row past the end reads the last row
    __builtin_amdgcn_global_load_lds(KV + r * (32 * NCH) + 8 * p, (kv_lds_void*)(wl + 1024 * q), 16,
                                     0, 0);
  }
  // operand A of half h: lane (slot p = lane % 16, k group lane / 16) holds
  // the eight bfloat16 entries H_32[i][8 (lane / 16) + j], i = 8 (p / 4) +
  // 4 h + p % 4: the sign (-1)^popcount(i & k) is H_8[4 h + p % 4][j] times
  // (-1)^popcount((p / 4) & (lane / 16)) (bits 0-2 and 3-4 of i and k)
  v4u ha[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) ha[h] = h32_operand_bf16(4 * h + (t & 3), (t >> 2) & g);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // operand B of chunk c: piece 4 c + g of vector t
  v4u xb[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    xb[c] = *reinterpret_cast<const v4u*>(wl + 16 * (t * kPieces + ((4 * c + g) ^ (t & (kPieces - 1)))));
  // (the code staging below reuses the wave's tile area: its LDS accesses
  // complete in order)
  kv4_mfma_tile<NCH, LB>(xb, ha, r0, rows, norm, kvq, scales, reinterpret_cast<uint32_t*>(wl), t, g);
}

template <int NCH, int LB>
static void launch_kv4_mfma_lb(const KvSet& set, int count, int64_t rows, int log2b, float norm,
                               hipStream_t s) {
  if constexpr ((1 << LB) <= 32 * NCH) {
    if (log2b == LB) {
      const int64_t tiles = (rows + 15) / 16;
      const int64_t blocks = (tiles + kKvMfmaWaves - 1) / kKvMfmaWaves;
      hipLaunchKernelGGL((kv4_mfma_kernel<NCH, LB>), dim3((unsigned)(count * blocks)),
                         dim3(64 * kKvMfmaWaves), 0, s, set, rows, blocks, norm);
      return;
    }
    launch_kv4_mfma_lb<NCH, LB + 1>(set, count, rows, log2b, norm, s);
  }
}

// bfloat16 vectors of 64, 128 or 256 elements with a block of at least 32 run
// on the matrix cores
static bool kv4_mfma_ok(int bf16, int D, int had_block) {
  return bf16 && had_block >= 32 && (D == 64 || D == 128 || D == 256);
}

// count tensors (1 or 2) of rows vectors each in one launch; log2b in [5, log2 D]
static void launch_kv4_mfma(const KvSet& set, int count, int64_t rows, int D, int log2b,
                            float norm, hipStream_t s) {
  if (D == 64) launch_kv4_mfma_lb<2, 5>(set, count, rows, log2b, norm, s);
  else if (D == 128) launch_kv4_mfma_lb<4, 5>(set, count, rows, log2b, norm, s);
  else launch_kv4_mfma_lb<8, 5>(set, count, rows, log2b, norm, s);
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

static int kv4_log2(int had_block) {
  int log2b = 0;
  while ((1 << log2b) < had_block) ++log2b;
  return log2b;
}

hipError_t launch_kv4(const void* KV, int bf16, int64_t rows, int D, int had_block, uint8_t* kvq,
                      float* scales, hipStream_t s) {
  const int log2b = kv4_log2(had_block);
  const float norm = (float)(1.0 / __builtin_sqrt((double)had_block));
  if (kv4_mfma_ok(bf16, D, had_block)) {
    const KvSet set{{reinterpret_cast<const uint16_t*>(KV), nullptr}, {kvq, nullptr},
                    {scales, nullptr}};
    launch_kv4_mfma(set, 1, rows, D, log2b, norm, s);
    return hipGetLastError();
  }
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

// K and V of one layer: one launch on the matrix-core path (each launch has a
// ramp at its start and a tail at its end that one launch of twice the rows
// pays once), else one launch each
hipError_t launch_kv4_pair(const void* K, const void* V, int bf16, int64_t rows, int D,
                           int had_block, uint8_t* kq, float* ks, uint8_t* vq, float* vs,
                           hipStream_t s) {
  if (kv4_mfma_ok(bf16, D, had_block)) {
    const KvSet set{{reinterpret_cast<const uint16_t*>(K), reinterpret_cast<const uint16_t*>(V)},
                    {kq, vq}, {ks, vs}};
    launch_kv4_mfma(set, 2, rows, D, kv4_log2(had_block),
                    (float)(1.0 / __builtin_sqrt((double)had_block)), s);
    return hipGetLastError();
  }
  hipError_t e = launch_kv4(K, bf16, rows, D, had_block, kq, ks, s);
  if (e != hipSuccess) return e;
  return launch_kv4(V, bf16, rows, D, had_block, vq, vs, s);
}

}  // namespace qift
