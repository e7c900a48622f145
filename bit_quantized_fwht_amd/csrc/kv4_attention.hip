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
// keeps an online softmax (reference point m, kept within a fixed slack of
// the running maximum, sum l, 32 accumulators), four
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

__device__ __forceinline__ float attn_f32(float v) { return v; }
__device__ __forceinline__ float attn_f32(uint16_t v) { return bf16_bits_to_float(v); }

// 16 times the 32 int4 codes in 16 bytes (element 2j in the low nibble of
// byte j, so element i of a word at bits 4i..4i+3). Each nibble is put in
// the high half of a byte whose low half is 0, whose value as a signed byte
// is then 16 times the code: odd elements are there already (a mask of the
// word), even ones move up by one shift and the same mask, and the conversion
// reads its byte straight from the masked word, sign-extended (one
// v_cvt_f32_i32 with a byte-select source per element, against a bit-field
// extract and a conversion). The empty asm statements hide the masked words
// from the optimizer, which would otherwise rewrite some of the byte reads
// into separate shifts and masks. The factor 16 is a power of two: it is
// taken out of the other operand or of the sum, exactly.
__device__ __forceinline__ void int4x32_x16(const uint4& u, float (&c)[32]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t odd = w[i] & 0xF0F0F0F0u, even = (w[i] << 4) & 0xF0F0F0F0u;
    asm("" : "+v"(odd));
    asm("" : "+v"(even));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[8 * i + 2 * b] = (float)(int8_t)(even >> (8 * b));
      c[8 * i + 2 * b + 1] = (float)(int8_t)(odd >> (8 * b));
    }
  }
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
// how far a score may exceed the state's reference point before the state is
// rescaled: p = exp(score - m) <= e^8, so l and acc stay far inside the
// float32 range (at most T e^8 times the values of a state kept at the
// running maximum)
constexpr float kAttnSlack = 8.0f;
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

  const int slot = tid / kPairs;
  const int hq = tid - slot * kPairs;
  const int hl = hq >> 2, quarter = hq & 3;
  const int head = h0 + (hl < nh ? hl : 0);  // a missing head reads head h0 and is discarded
  const int64_t t0 = run * tpr;
  const int64_t t1 = t0 + tpr < T ? t0 + tpr : T;
  const int64_t row_bytes = (int64_t)H * (kAttnD / 2);
  const uint8_t* kbase = kq + head * (kAttnD / 2) + quarter * 16;
  const uint8_t* vbase = vq + head * (kAttnD / 2) + quarter * 16;
  // the slot's tokens t0 + slot + 32 i; group g holds i = kAttnU g ..
  // kAttnU (g + 1) - 1; a token past t1 is not counted
  const int64_t n_iter = (t1 - t0 + kAttnP - 1) / kAttnP;
  const int64_t n_grp = (n_iter + kAttnU - 1) / kAttnU;
  struct Grp {
    uint4 k[kAttnU], v[kAttnU];
    float ks[kAttnU], vs[kAttnU];
  };
  // every lane loads from a valid row: a token past the run reads the run's
  // last row, and compute() skips it after its dot product (whose quad sum
  // every lane takes part in), so the loads need no per-lane branch and no
  // zeroing. Groups past the last are not loaded, except group 1 of a run
  // of one group (its last row again), so that the query's wait below counts
  // exactly the sixteen loads issued after it
  auto load = [&](Grp& G, int64_t g) {
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      const int64_t t = t0 + slot + kAttnP * (kAttnU * g + u);
      const int64_t row = sq * T + (t < t1 ? t : t1 - 1);
      G.k[u] = *reinterpret_cast<const uint4*>(kbase + row * row_bytes);
      G.v[u] = *reinterpret_cast<const uint4*>(vbase + row * row_bytes);
      G.ks[u] = ks[row * H + head];
      G.vs[u] = vs[row * H + head];
    }
  };
  // the query is requested first and the first two groups right after it,
  // so that the query's latency and theirs overlap (the query is waited for
  // alone: loads complete in order)
  const TQ xq = q[(sq * H + h0) * kAttnD + (tid < nh * kAttnD ? tid : 0)];
  __builtin_amdgcn_sched_barrier(0);  // the query's load first
  Grp ga, gb;
  load(ga, 0);
  load(gb, 1);
  __builtin_amdgcn_sched_barrier(0);  // all seventeen loads issued before the query is used

  // rotated queries of the workgroup's heads: element i = tid (two heads of
  // 128); stages on index bits 0-5 by lane shuffles, bit 6 through LDS
  float x = tid < nh * kAttnD ? attn_f32(xq) : 0.f;
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
  // the thread's 32 query values, divided by 16 against the codes' factor
  // of 16 (int4x32_x16): the products, and so the dot products, are unchanged
  const float qn = norm * 0.0625f;
  float qv[kAttnQ];
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) qv[j] = qr[hl * kAttnD + quarter * kAttnQ + j] * qn;

  // online softmax; acc holds 16 times the weighted sum of the values (codes
  // times 16), taken out when the run's state is written
  float m = -__builtin_huge_valf(), l = 0.f;
  float acc[kAttnQ];
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) acc[j] = 0.f;

  // per token: the dot product of the thread's quarter, the quad sum (DPP),
  // then one online-softmax update of (m, l, acc)
  auto compute = [&](const Grp& G, int64_t g) {
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      float c[kAttnQ];
      int4x32_x16(G.k[u], c);
      float dot = 0.f;
#pragma unroll
      for (int j = 0; j < kAttnQ; ++j) dot = fmaf(qv[j], c[j], dot);
      dot += quad_xor<1>(dot);
      dot += quad_xor<2>(dot);
      // a token past the run takes the score -inf and the weight 0 (no
      // branch: a branch around the update made the compiler wait for more
      // of the other group's loads)
      const bool valid = t0 + slot + kAttnP * (kAttnU * g + u) < t1;
      const float sc = valid ? dot * G.ks[u] * softmax_scale : -__builtin_huge_valf();
      if (sc > m + kAttnSlack) {
        // the reference point m of the state moves only when a score exceeds
        // it by more than the slack (the first token, with m = -inf; rarely
        // later): a wave takes this branch whenever one of its lanes does, so
        // moving m on every new maximum rescaled the state on most tokens.
        // Every term of l and acc carries the same factor exp(-m), which
        // cancels in acc / l and in the merges; p stays below exp(slack).
        const float alpha = __expf(m - sc);
        l *= alpha;
#pragma unroll
        for (int j = 0; j < kAttnQ; ++j) acc[j] *= alpha;
        m = sc;
      }
      const float p = valid ? __expf(sc - m) : 0.f;
      l += p;
      const float pv = p * G.vs[u];
      int4x32_x16(G.v[u], c);
#pragma unroll
      for (int j = 0; j < kAttnQ; ++j) acc[j] = fmaf(pv, c[j], acc[j]);
    }
  };
  // steady state: every load of the loop body is unconditional, so the wait
  // for a group counts exactly the other group's loads issued after it (a
  // load under a branch made the compiler wait for all loads where the
  // branches met, emptying the second buffer); the last two or three groups
  // follow the loop
  int64_t g = 0;
  for (; g + 3 < n_grp; g += 2) {
    compute(ga, g);
    load(ga, g + 2);
    __builtin_amdgcn_sched_barrier(0);  // issued before the other group is used
    compute(gb, g + 1);
    load(gb, g + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  compute(ga, g);
  if (g + 2 < n_grp) load(ga, g + 2);
  if (g + 1 < n_grp) compute(gb, g + 1);
  if (g + 2 < n_grp) compute(ga, g + 2);

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
    dst[2 + pq * kAttnQ + j] = o * 0.0625f;  // the codes' factor of 16
  }
}

// Kernel 2: grid (H, S), 256 threads. Merge the runs of one (sequence, head),
// divide by the softmax sum and rotate back. Runs are taken 64 at a time
// (one pass for up to 64 runs): thread (run, quarter) loads the run's m and l
// and its 32 partial outputs together, the chunk's maximum comes from
// shuffles and one LDS exchange, the outputs weighted by exp(m_r - M) are
// parked in LDS and 128 threads sum over the runs; chunks after the first
// are merged into the running state as two online-softmax states are. The
// back rotation runs on the 128 sums in registers: index bits 0-5 by lane
// shuffles, bit 6 through LDS.
constexpr int kAttnCombineThreads = 256;
__global__ __launch_bounds__(kAttnCombineThreads) void kv4_attn_combine_kernel(
    const float* __restrict__ part, int64_t runs, int H, int log2b, float norm,
    void* __restrict__ out, int out_bf16) {
  constexpr int kWaves = kAttnCombineThreads / 64;
  __shared__ float cell[64 * (kAttnD + 1)];  // [run][d], padded rows
  __shared__ float red[2][kWaves];           // per wave: chunk maximum, chunk sum of l
  __shared__ float xo[kAttnD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t head = blockIdx.x, sq = blockIdx.y;
  const float* p0 = part + (sq * runs * H + head) * kAttnPart;
  const int64_t stride = (int64_t)H * kAttnPart;
  const int rl = tid >> 2, qd = (tid & 3) * kAttnQ;
  // running state over the chunks so far; thread d < 128 holds dimension d
  float M = -__builtin_huge_valf(), L = 0.f, acc = 0.f;
  for (int64_t r0 = 0; r0 < runs; r0 += 64) {
    const int64_t r = r0 + rl;
    const bool ok = r < runs;
    const float* src = p0 + (ok ? r : r0) * stride;  // a missing run reads run r0, weighs 0
    const float mr0 = src[0], lr0 = src[1];
    float2 v[kAttnQ / 2];
#pragma unroll
    for (int i = 0; i < kAttnQ / 2; ++i) v[i] = reinterpret_cast<const float2*>(src + 2 + qd)[i];
    const float mr = ok ? mr0 : -__builtin_huge_valf();
    const float lr = ok ? lr0 : 0.f;
    // the chunk's maximum (the four threads of a run hold the same m)
    float mc = mr;
#pragma unroll
    for (int off = 32; off >= 4; off >>= 1) mc = fmaxf(mc, __shfl_xor(mc, off, 64));
    if (lane == 0) red[0][wave] = mc;
    __syncthreads();
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) mc = fmaxf(mc, red[0][wv]);
    const float Mn = fmaxf(M, mc);
    const float w = lr > 0.f ? __expf(mr - Mn) : 0.f;
#pragma unroll
    for (int i = 0; i < kAttnQ / 2; ++i) {
      cell[rl * (kAttnD + 1) + qd + 2 * i] = v[i].x * w;
      cell[rl * (kAttnD + 1) + qd + 2 * i + 1] = v[i].y * w;
    }
    float ls = (tid & 3) == 0 ? lr * w : 0.f;
#pragma unroll
    for (int off = 32; off >= 4; off >>= 1) ls += __shfl_xor(ls, off, 64);
    if (lane == 0) red[1][wave] = ls;
    __syncthreads();
    // the state so far, rescaled to the new maximum (weight 0 before the first chunk)
    const float a = L > 0.f ? __expf(M - Mn) : 0.f;
    float lc = 0.f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) lc += red[1][wv];
    L = fmaf(L, a, lc);
    if (tid < kAttnD) {
      const int64_t nr = runs - r0 < 64 ? runs - r0 : 64;
      float sum = 0.f;
      for (int64_t i = 0; i < nr; ++i) sum += cell[i * (kAttnD + 1) + tid];
      acc = fmaf(acc, a, sum);
    }
    M = Mn;
    __syncthreads();  // cell and red are written again by the next chunk
  }
  float y = tid < kAttnD ? acc / L : 0.f;
  for (int st = 0; st < log2b && st < 6; ++st) {
    const float z = __shfl_xor(y, 1 << st, 64);
    y = (tid >> st) & 1 ? z - y : y + z;
  }
  if (log2b > 6) {
    if (tid < kAttnD) xo[tid] = y;
    __syncthreads();
    if (tid < kAttnD) {
      const float z = xo[tid ^ 64];
      y = (tid & 64) ? z - y : y + z;
    }
  }
  if (tid >= kAttnD) return;
  y *= norm;
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
