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
// one sequence for all heads, so every token row of the cache ([H, D/2] codes,
// 2 KB for H = 32, D = 128) is read with whole-row coalesced loads. A thread
// owns one (head, quarter of D) pair and one token slot: it holds 32 rotated
// query values, reads 16 bytes of K and 16 bytes of V codes per token, sums
// its quarter of the dot product (the four quarters meet by quad shuffles)
// and keeps an online softmax (running max m, sum l, 32 accumulators). The
// token slots of a head are merged through LDS and the workgroup writes
// (m, l, o'[D]) per head. Kernel 2 merges the runs of each (sequence, head),
// divides by l and rotates back.
#include "qift_internal.h"

namespace qift {

constexpr int kAttnThreads = 256;
constexpr int kAttnD = 128;             // head dimension
constexpr int kAttnQ = kAttnD / 4;      // dims per thread (a quarter of D)
constexpr int kAttnPart = 2 + kAttnD;   // floats per (run, head): m, l, o'[D]

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

// Kernel 1: grid (runs, S). Run r of sequence s covers tokens
// [r * tpr, min(T, (r + 1) * tpr)).
template <typename TQ>
__global__ __launch_bounds__(kAttnThreads) void kv4_attn_partial_kernel(
    const TQ* __restrict__ q, int64_t T, int H, int log2b, float norm, float softmax_scale,
    const uint8_t* __restrict__ kq, const float* __restrict__ ks,
    const uint8_t* __restrict__ vq, const float* __restrict__ vs, int64_t tpr,
    float* __restrict__ part) {
  extern __shared__ float lds[];  // q' [H * D], then the slot merge
  const int tid = threadIdx.x;
  const int64_t sq = blockIdx.y;
  const int64_t run = blockIdx.x;
  const int64_t runs = gridDim.x;
  const int HD = H * kAttnD;

  // rotated queries of all heads
  for (int i = tid; i < HD; i += kAttnThreads) lds[i] = attn_ld<TQ>(q, sq * HD + i);
  __syncthreads();
  lds_fwht(lds, HD, log2b, tid, kAttnThreads);

  const int pairs = 4 * H;                 // (head, quarter) pairs
  const int P = kAttnThreads / pairs;      // token slots
  const int slot = tid / pairs;
  const int hq = tid - slot * pairs;
  const int head = hq >> 2, quarter = hq & 3;
  const bool active = slot < P;
  float qv[kAttnQ];
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j)
    qv[j] = active ? lds[head * kAttnD + quarter * kAttnQ + j] * norm : 0.f;

  const int64_t t0 = run * tpr;
  const int64_t t1 = t0 + tpr < T ? t0 + tpr : T;
  float m = -__builtin_huge_valf(), l = 0.f;
  float acc[kAttnQ];
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) acc[j] = 0.f;

  // byte offset of (token t, this head, this quarter) in a code array
  const int64_t row_bytes = (int64_t)H * (kAttnD / 2);
  auto code_off = [&](int64_t t) {
    return ((sq * T + t) * row_bytes) + head * (kAttnD / 2) + quarter * 16;
  };
  // every lane of a wave runs the same number of iterations: the loop bound
  // is uniform, and lanes of inactive slots or past t1 load a valid token
  // (t0) and discard it
  const int64_t n_iter = (t1 - t0 + P - 1) / P;
  uint4 kc = uint4{0u, 0u, 0u, 0u}, vc = kc;
  float ksc = 0.f, vsc = 0.f;
  auto load = [&](int64_t i) {
    int64_t t = t0 + slot + P * i;
    t = (active && t < t1) ? t : t0;
    kc = *reinterpret_cast<const uint4*>(kq + code_off(t));
    vc = *reinterpret_cast<const uint4*>(vq + code_off(t));
    ksc = ks[(sq * T + t) * H + head];
    vsc = vs[(sq * T + t) * H + head];
  };
  if (n_iter > 0) load(0);
  for (int64_t i = 0; i < n_iter; ++i) {
    const uint4 k = kc, v = vc;
    const float kscale = ksc, vscale = vsc;
    if (i + 1 < n_iter) load(i + 1);
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < kAttnQ; ++j) dot = fmaf(qv[j], int4_at(k, j), dot);
    dot += __shfl_xor(dot, 1, 64);
    dot += __shfl_xor(dot, 2, 64);
    const int64_t t = t0 + slot + P * i;
    if (!(active && t < t1)) continue;
    const float sc = dot * kscale * softmax_scale;
    const float m_new = fmaxf(m, sc);
    const float alpha = __expf(m - m_new);  // 0 on the first token (m = -inf)
    const float p = __expf(sc - m_new);
    l = l * alpha + p;
    const float pv = p * vscale;
#pragma unroll
    for (int j = 0; j < kAttnQ; ++j) acc[j] = fmaf(acc[j], alpha, pv * int4_at(v, j));
    m = m_new;
  }

  // merge the token slots of each (head, quarter): slot 0 combines
  __syncthreads();  // done with q'
  float* mrg = lds;  // [P][pairs][2 + kAttnQ]
  constexpr int kRec = 2 + kAttnQ;
  if (active) {
    float* r = mrg + (slot * pairs + hq) * kRec;
    r[0] = m;
    r[1] = l;
#pragma unroll
    for (int j = 0; j < kAttnQ; ++j) r[2 + j] = acc[j];
  }
  __syncthreads();
  if (slot != 0) return;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < P; ++s) M = fmaxf(M, mrg[(s * pairs + hq) * kRec]);
  float L = 0.f;
  float o[kAttnQ];
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) o[j] = 0.f;
  for (int s = 0; s < P; ++s) {
    const float* r = mrg + (s * pairs + hq) * kRec;
    const float w = r[1] > 0.f ? __expf(r[0] - M) : 0.f;  // a slot without tokens adds nothing
    L = fmaf(r[1], w, L);
#pragma unroll
    for (int j = 0; j < kAttnQ; ++j) o[j] = fmaf(r[2 + j], w, o[j]);
  }
  float* dst = part + ((sq * runs + run) * H + head) * kAttnPart;
  if (quarter == 0) {
    dst[0] = M;
    dst[1] = L;
  }
#pragma unroll
  for (int j = 0; j < kAttnQ; ++j) dst[2 + quarter * kAttnQ + j] = o[j];
}

// Kernel 2: grid (H, S), kAttnD threads. Merge the runs of one (sequence,
// head), divide by the softmax sum and rotate back.
__global__ __launch_bounds__(kAttnD) void kv4_attn_combine_kernel(
    const float* __restrict__ part, int64_t runs, int H, int log2b, float norm,
    void* __restrict__ out, int out_bf16) {
  __shared__ float o[kAttnD];
  const int d = threadIdx.x;
  const int64_t head = blockIdx.x, sq = blockIdx.y;
  const float* p0 = part + (sq * runs * H + head) * kAttnPart;
  const int64_t stride = (int64_t)H * kAttnPart;
  float M = -__builtin_huge_valf();
  for (int64_t r = 0; r < runs; ++r) M = fmaxf(M, p0[r * stride]);
  float L = 0.f, acc = 0.f;
  for (int64_t r = 0; r < runs; ++r) {
    const float* pr = p0 + r * stride;
    const float w = pr[1] > 0.f ? __expf(pr[0] - M) : 0.f;
    L = fmaf(pr[1], w, L);
    acc = fmaf(pr[2 + d], w, acc);
  }
  o[d] = acc / L;
  __syncthreads();
  lds_fwht(o, kAttnD, log2b, d, kAttnD);
  const float y = o[d] * norm;
  const int64_t idx = (sq * H + head) * kAttnD + d;
  if (out_bf16)
    reinterpret_cast<uint16_t*>(out)[idx] = float_to_bf16_bits(y);
  else
    reinterpret_cast<float*>(out)[idx] = y;
}

// tokens per run: about 512 workgroups over all sequences, at least 16
// tokens per run (each run writes H * (2 + D) floats of partial results: at
// 16 tokens that is 1/8 of the cache bytes it reads), a multiple of the token
// slots
int64_t kv4_attn_tokens_per_run(int64_t S, int64_t T, int H) {
  const int64_t P = kAttnThreads / (4 * H);
  int64_t tpr = (S * T + 511) / 512;
  if (tpr < 16) tpr = 16;
  tpr = (tpr + P - 1) / P * P;
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

hipError_t launch_kv4_attention(const void* q, int q_bf16, int64_t S, int64_t T, int H,
                                int had_block, const uint8_t* kq, const float* ks,
                                const uint8_t* vq, const float* vs, float softmax_scale,
                                void* out, int out_bf16, float* part, hipStream_t s) {
  const int64_t tpr = kv4_attn_tokens_per_run(S, T, H);
  const int64_t runs = (T + tpr - 1) / tpr;
  const int lb = ilog2_attn(had_block);
  const float nrm = (float)(1.0 / __builtin_sqrt((double)had_block));
  const int pairs = 4 * H;
  const size_t merge = (size_t)(kAttnThreads / pairs) * pairs * (2 + kAttnQ);
  const size_t lds = (size_t)H * kAttnD > merge ? (size_t)H * kAttnD : merge;
  const dim3 g1((unsigned)runs, (unsigned)S);
  if (q_bf16)
    hipLaunchKernelGGL(kv4_attn_partial_kernel<uint16_t>, g1, dim3(kAttnThreads),
                       lds * sizeof(float), s, reinterpret_cast<const uint16_t*>(q), T, H, lb,
                       nrm, softmax_scale, kq, ks, vq, vs, tpr, part);
  else
    hipLaunchKernelGGL(kv4_attn_partial_kernel<float>, g1, dim3(kAttnThreads),
                       lds * sizeof(float), s, reinterpret_cast<const float*>(q), T, H, lb, nrm,
                       softmax_scale, kq, ks, vq, vs, tpr, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv4_attn_combine_kernel, dim3((unsigned)H, (unsigned)S), dim3(kAttnD), 0, s,
                     part, runs, H, lb, nrm, out, out_bf16);
  return hipGetLastError();
}

}  // namespace qift
