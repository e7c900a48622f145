// Decode attention over a KV4 cache: the consumer of the 4-bit KV cache of
// rotated W2A4/KV4 inference (Qift abstract). The cache holds every head
// vector rotated by H_B / sqrt(B) along D and quantized to int4 with one scale
// per (token, head) (qift_kv4_quant). The query is rotated by the same
// orthogonal map, so q' . k' = q . k: scores are taken in the rotated domain
// against the dequantized codes, the softmax-weighted sum of the dequantized
// values is formed there, and the result is rotated back (H_B / sqrt(B) is its
// own inverse).
//
// Split-T ("flash decoding"): kernel 1 gives each workgroup a run of tokens of
// one sequence for a pair of heads, whose codes are one 128-byte line per
// token (64 bytes of K or V per head at D = 128). A thread owns one (head,
// quarter of D) pair and one of 32 token slots: it holds 32 rotated query
// values, reads 16 bytes of K and 16 bytes of V codes per token, sums its
// quarter of the dot product (the four quarters meet by DPP quad moves) and
// keeps an online softmax (running max m, sum l, 32 accumulators), four
// tokens' loads in flight. The token
// slots of a head are merged through LDS and the workgroup writes (m, l,
// o'[D]) per head. Runs are sized for about 512 workgroups in all, so a head
// has few runs (32 at one sequence of 4096 tokens and 32 heads) and the
// partial results stay small (1/32 of the cache bytes there). Kernel 2 merges
// the runs of each (sequence, head) with independent loads, divides by l and
// rotates back.
#include <mutex>

#include "lane_butterfly.h"

namespace qift {

constexpr int kAttnThreads = 256;
constexpr int kAttnD = 128;             // head dimension
constexpr int kAttnQ = kAttnD / 4;      // dims per thread (a quarter of D)
constexpr int kAttnPart = 2 + kAttnD;   // floats per (run, head): m, l, o'[D]
constexpr int kAttnG = 2;               // heads per workgroup
constexpr int kAttnP = kAttnThreads / (4 * kAttnG);  // token slots (32)

template <typename T>
__device__ __forceinline__ float attn_ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float attn_ld<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float attn_ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}

// Unnormalized block Walsh-Hadamard transform, blocks of 2^log2b along the
// n floats of an LDS array (n a multiple of the block), by the whole
// workgroup of nthr threads.
__device__ __forceinline__ void lds_fwht(float* x, int n, int log2b, int tid, int nthr) {
  for (int st = 0; st < log2b; ++st) {
    const int h = 1 << st;
    for (int p = tid; p < n / 2; p += nthr) {
      const int i = (p >> st) * 2 * h + (p & (h - 1));
      const float a = x[i], b = x[i + h];
      x[i] = a + b;
      x[i + h] = a - b;
    }
    __syncthreads();
  }
}

// code e of the 32 int4 codes in 16 bytes (element 2j in the low nibble of
// byte j, so element i of a word at bits 4i..4i+3), sign-extended: the nibble
// is shifted to the top of the word and shifted back arithmetically
__device__ __forceinline__ float int4_at(const uint4& u, int e) {
  const uint32_t w = e < 8 ? u.x : e < 16 ? u.y : e < 24 ? u.z : u.w;
  return (float)((int32_t)(w << (28 - 4 * (e & 7))) >> 28);
}

// Merge of two online-softmax states (m, l, acc): weights exp(m - M), a state
// without tokens (l = 0) weighs nothing.
__device__ __forceinline__ void attn_merge(float& m, float& l, float* acc, float m2, float l2,
                                           const float* acc2) {
  const float M = fmaxf(m, m2);
  const float w1 = l > 0.f ? __expf(m - M) : 0.f;
  const float w2 = l2 > 0.f ? __expf(m2 - M) : 0.f;
  l = l * w1 + l2 * w2;
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) acc[j] = acc[j] * w1 + acc2[j] * w2;
  m = M;
}

// Kernel 1: grid (runs, ceil(H / 2), S). Run r of sequence s covers tokens
// [r * tpr, min(T, (r + 1) * tpr)).
// tokens per load group, two groups in flight (groups of 4 time the same and
// need 226 registers instead of 162; a once-per-group softmax rescale with
// 4-token groups needs 256 and runs 35% slower)
constexpr int kAttnU = 2;
template <typename TQ>
__global__ __launch_bounds__(kAttnThreads) void kv4_attn_partial_kernel(
    const TQ* __restrict__ q, int64_t T, int H, int log2b, float norm, float softmax_scale,
    const uint8_t* __restrict__ kq, const float* __restrict__ ks,
    const uint8_t* __restrict__ vq, const float* __restrict__ vs, int64_t tpr,
    float* __restrict__ part) {
  constexpr int kRec = 2 + kAttnQ;
  constexpr int kPairs = 4 * kAttnG;
  __shared__ float qr[kAttnG * kAttnD];
  __shared__ float mrg[(kAttnThreads / 64) * kPairs * kRec];  // [wave][head, quarter][m, l, acc]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t run = blockIdx.x, runs = gridDim.x;
  const int h0 = blockIdx.y * kAttnG;
  const int64_t sq = blockIdx.z;
  const int nh = H - h0 < kAttnG ? H - h0 : kAttnG;  // heads of this workgroup

  // rotated queries of the workgroup's heads: element i = tid (two heads of
  // 128); stages on index bits 0-5 by lane shuffles, bit 6 through LDS
  float x = tid < nh * kAttnD ? attn_ld<TQ>(q, (sq * H + h0) * kAttnD + tid) : 0.f;
  for (int st = 0; st < log2b && st < 6; ++st) {
    const float y = __shfl_xor(x, 1 << st, 64);
    x = (tid >> st) & 1 ? y - x : x + y;
  }
  qr[tid] = x;
  __syncthreads();
  if (log2b > 6) {
    const float y = qr[tid ^ 64];
    __syncthreads();
    qr[tid] = (tid & 64) ? y - x : x + y;
    __syncthreads();
  }

  const int slot = tid / kPairs;
  const int hq = tid - slot * kPairs;
  const int hl = hq >> 2, quarter = hq & 3;
  const int head = h0 + (hl < nh ? hl : 0);  // a missing head reads head h0 and is discarded
  float qv[kAttnQ];
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) qv[j] = qr[hl * kAttnD + quarter * kAttnQ + j] * norm;

  const int64_t t0 = run * tpr;
  const int64_t t1 = t0 + tpr < T ? t0 + tpr : T;
  float m = -__builtin_huge_valf(), l = 0.f;
  float acc[kAttnQ];
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) acc[j] = 0.f;

  const int64_t row_bytes = (int64_t)H * (kAttnD / 2);
  const uint8_t* kbase = kq + head * (kAttnD / 2) + quarter * 16;
  const uint8_t* vbase = vq + head * (kAttnD / 2) + quarter * 16;
  // the slot's tokens t0 + slot + 32 i; group g holds i = 4g .. 4g + 3; a
  // token past t1 is not loaded (zero codes and scales) and not counted
  const int64_t n_iter = (t1 - t0 + kAttnP - 1) / kAttnP;
  const int64_t n_grp = (n_iter + kAttnU - 1) / kAttnU;
  struct Grp {
    uint4 k[kAttnU], v[kAttnU];
    float ks[kAttnU], vs[kAttnU];
  };
  auto load = [&](Grp& G, int64_t g) {
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      const int64_t t = t0 + slot + kAttnP * (kAttnU * g + u);
      const bool ok = t < t1;
      const int64_t row = sq * T + t;
      G.k[u] = ok ? *reinterpret_cast<const uint4*>(kbase + row * row_bytes) : uint4{0u, 0u, 0u, 0u};
      G.v[u] = ok ? *reinterpret_cast<const uint4*>(vbase + row * row_bytes) : uint4{0u, 0u, 0u, 0u};
      G.ks[u] = ok ? ks[row * H + head] : 0.f;
      G.vs[u] = ok ? vs[row * H + head] : 0.f;
    }
  };
  // per token: the dot product of the thread's quarter, the quad sum (DPP),
  // then one online-softmax update of (m, l, acc)
  auto compute = [&](const Grp& G, int64_t g) {
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < kAttnQ; ++j) dot = fmaf(qv[j], int4_at(G.k[u], j), dot);
      dot += quad_xor<1>(dot);
      dot += quad_xor<2>(dot);
      if (t0 + slot + kAttnP * (kAttnU * g + u) >= t1) continue;
      const float sc = dot * G.ks[u] * softmax_scale;
      if (sc > m) {
        // a new running maximum (every token early on, rarely later): the
        // state is rescaled only then (0 on the first token, m = -inf)
        const float alpha = __expf(m - sc);
        l *= alpha;
#pragma unroll
        for (int j = 0; j < kAttnQ; ++j) acc[j] *= alpha;
        m = sc;
      }
      const float p = __expf(sc - m);
      l += p;
      const float pv = p * G.vs[u];
#pragma unroll
      for (int j = 0; j < kAttnQ; ++j) acc[j] = fmaf(pv, int4_at(G.v[u], j), acc[j]);
    }
  };
  Grp ga, gb;
  load(ga, 0);
  for (int64_t g = 0; g < n_grp; g += 2) {
    load(gb, g + 1);
    compute(ga, g);
    load(ga, g + 2);
    if (g + 1 < n_grp) compute(gb, g + 1);
  }

  // merge the token slots of each (head, quarter): the 8 slots of a wave
  // (lanes 8 apart) by shuffles, then the 4 waves through LDS
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float l2 = __shfl_xor(l, off, 64);
    float a2[kAttnQ];
#pragma unroll
    for (int j = 0; j < kAttnQ; ++j) a2[j] = __shfl_xor(acc[j], off, 64);
    attn_merge(m, l, acc, m2, l2, a2);
  }
  if (lane < kPairs) {
    float* r = mrg + (wave * kPairs + lane) * kRec;
    r[0] = m;
    r[1] = l;
#pragma unroll
    for (int j = 0; j < kAttnQ; ++j) r[2 + j] = acc[j];
  }
  __syncthreads();
  // thread -> (pair, element j of its quarter): 8 pairs x 32 = 256
  {
    const int pr = tid >> 5, j = tid & 31;
    const int phl = pr >> 2, pq = pr & 3;
    if (phl >= nh) return;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) M = fmaxf(M, mrg[(w * kPairs + pr) * kRec]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnThreads / 64; ++w) {
      const float* r = mrg + (w * kPairs + pr) * kRec;
      const float wt = r[1] > 0.f ? __expf(r[0] - M) : 0.f;
      L = fmaf(r[1], wt, L);
      o = fmaf(r[2 + j], wt, o);
    }
    float* dst = part + ((sq * runs + run) * H + h0 + phl) * kAttnPart;
    if (pq == 0 && j == 0) {
      dst[0] = M;
      dst[1] = L;
    }
    dst[2 + pq * kAttnQ + j] = o;
  }
}

// Kernel 2: grid (H, S), 256 threads. Merge the runs of one (sequence, head),
// divide by the softmax sum and rotate back. Runs are taken 64 at a time:
// thread (run, quarter) loads its 32 partial outputs at once, scales them by
// the run's weight and parks them in LDS; 128 threads then sum over the runs.
constexpr int kAttnMaxRuns = 1024;
constexpr int kAttnCombineThreads = 256;
__global__ __launch_bounds__(kAttnCombineThreads) void kv4_attn_combine_kernel(
    const float* __restrict__ part, int64_t runs, int H, int log2b, float norm,
    void* __restrict__ out, int out_bf16) {
  __shared__ float o[kAttnD];
  __shared__ float wr[kAttnMaxRuns];  // run weights exp(m_r - M), 0 for an empty run
  __shared__ float red[kAttnCombineThreads / 64];
  __shared__ float cell[64 * (kAttnD + 1)];  // [run][d], padded rows
  const int tid = threadIdx.x;
  const int64_t head = blockIdx.x, sq = blockIdx.y;
  const float* p0 = part + (sq * runs * H + head) * kAttnPart;
  const int64_t stride = (int64_t)H * kAttnPart;
  // the maximum of the runs' m
  float mx = -__builtin_huge_valf();
  for (int64_t r = tid; r < runs; r += kAttnCombineThreads) mx = fmaxf(mx, p0[r * stride]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kAttnCombineThreads / 64; ++w) M = fmaxf(M, red[w]);
  // run weights and the total sum
  float lsum = 0.f;
  for (int64_t r = tid; r < runs; r += kAttnCombineThreads) {
    const float lr = p0[r * stride + 1];
    const float w = lr > 0.f ? __expf(p0[r * stride] - M) : 0.f;
    wr[r] = w;
    lsum = fmaf(lr, w, lsum);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
  __syncthreads();  // every thread has read M from red; the weights are in wr
  if ((tid & 63) == 0) red[tid >> 6] = lsum;
  __syncthreads();
  float L = red[0];
#pragma unroll
  for (int w = 1; w < kAttnCombineThreads / 64; ++w) L += red[w];
  // weighted sum of the partial outputs, 64 runs at a time
  const int rl = tid >> 2, qd = (tid & 3) * kAttnQ;
  float acc = 0.f;  // thread d < 128: dimension d
  for (int64_t r0 = 0; r0 < runs; r0 += 64) {
    const int64_t r = r0 + rl;
    if (r < runs) {
      const float2* src = reinterpret_cast<const float2*>(p0 + r * stride + 2 + qd);
      float2 v[kAttnQ / 2];
#pragma unroll
      for (int i = 0; i < kAttnQ / 2; ++i) v[i] = src[i];
      const float w = wr[r];
#pragma unroll
      for (int i = 0; i < kAttnQ / 2; ++i) {
        cell[rl * (kAttnD + 1) + qd + 2 * i] = v[i].x * w;
        cell[rl * (kAttnD + 1) + qd + 2 * i + 1] = v[i].y * w;
      }
    }
    __syncthreads();
    if (tid < kAttnD) {
      const int64_t nr = runs - r0 < 64 ? runs - r0 : 64;
      for (int64_t i = 0; i < nr; ++i) acc += cell[i * (kAttnD + 1) + tid];
    }
    __syncthreads();
  }
  if (tid < kAttnD) o[tid] = acc / L;
  __syncthreads();
  lds_fwht(o, kAttnD, log2b, tid, kAttnCombineThreads);
  if (tid >= kAttnD) return;
  const float y = o[tid] * norm;
  const int64_t idx = (sq * H + head) * kAttnD + tid;
  if (out_bf16)
    reinterpret_cast<uint16_t*>(out)[idx] = float_to_bf16_bits(y);
  else
    reinterpret_cast<float*>(out)[idx] = y;
}

// tokens per run: about 512 workgroups over all sequences and head pairs
// (a run is at least one token per slot: 32 tokens; a multiple of 32)
int64_t kv4_attn_tokens_per_run(int64_t S, int64_t T, int H) {
  const int64_t groups = S * ((H + kAttnG - 1) / kAttnG);
  const int64_t runs = (512 + groups - 1) / groups;
  int64_t tpr = (T + runs - 1) / runs;
  tpr = (tpr + kAttnP - 1) / kAttnP * kAttnP;
  return tpr;
}

size_t kv4_attn_workspace_bytes(int64_t S, int64_t T, int H) {
  const int64_t tpr = kv4_attn_tokens_per_run(S, T, H);
  const int64_t runs = (T + tpr - 1) / tpr;
  return (size_t)(S * runs * H * kAttnPart) * sizeof(float);
}

static int ilog2_attn(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

// ---------------------------------------------------------------------------
// partial results of the allocation-free entry point
// ---------------------------------------------------------------------------

// One fixed array per GPU, held from the first use of this code object on
// that GPU until the process ends. Every entry the combine kernel reads is
// written by the partial kernel of the same call, so nothing needs clearing
// between calls. In host code `scratch` names a host-side stand-in, not the
// device array: kernels receive the address kv4_attn_scratch returns.
static __device__ __align__(256) float scratch[QIFT_ATTENTION_SCRATCH_BYTES / sizeof(float)];

constexpr int kScratchMaxDevices = 64;

// The address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
hipError_t kv4_attn_scratch(float** ptr) {
  static std::mutex mu;
  static float* addr[kScratchMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_kv4_attention(const void* q, int q_bf16, int64_t S, int64_t T, int H,
                                int had_block, const uint8_t* kq, const float* ks,
                                const uint8_t* vq, const float* vs, float softmax_scale,
                                void* out, int out_bf16, float* part, hipStream_t s) {
  const int64_t tpr = kv4_attn_tokens_per_run(S, T, H);
  const int64_t runs = (T + tpr - 1) / tpr;
  const int lb = ilog2_attn(had_block);
  const float nrm = (float)(1.0 / __builtin_sqrt((double)had_block));
  const dim3 g1((unsigned)runs, (unsigned)((H + kAttnG - 1) / kAttnG), (unsigned)S);
  if (q_bf16)
    hipLaunchKernelGGL(kv4_attn_partial_kernel<uint16_t>, g1, dim3(kAttnThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(q), T, H, lb, nrm, softmax_scale, kq,
                       ks, vq, vs, tpr, part);
  else
    hipLaunchKernelGGL(kv4_attn_partial_kernel<float>, g1, dim3(kAttnThreads), 0, s,
                       reinterpret_cast<const float*>(q), T, H, lb, nrm, softmax_scale, kq, ks,
                       vq, vs, tpr, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv4_attn_combine_kernel, dim3((unsigned)H, (unsigned)S),
                     dim3(kAttnCombineThreads), 0, s, part, runs, H, lb, nrm, out, out_bf16);
  return hipGetLastError();
}

}  // namespace qift
