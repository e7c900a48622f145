// Error-compensated weight quantization with the fixed no-zero levels: GPTQ's
// column-by-column quantization (quantizing one column updates the ones after
// it; QTEA abstract), applied with the Qift level sets and their per-channel
// scale (Qift abstract, which reports the "GPTQ residual behavior" of its
// level sets). Everything after the code decisions is float64.
//
// Steps on the device:
//  1. the calibration activations and the weights are rotated like the
//     linear's inputs (block Walsh-Hadamard along K, float64); the weights are
//     then rounded to float32, the values the plain quantizer decides on;
//  2. H = X'^T X' on the float64 matrix cores (v_mfma_f64_16x16x4f64);
//  3. per-channel scales by the plain quantizer's rule, from the rotated
//     weights before any update;
//  4. dead features (H[k][k] = 0) get H[k][k] = 1 and weight 0; the damping
//     damp * mean(diag H) is added to the diagonal;
//  5. U with U^T U = H^-1, upper triangular: if J reverses the order of the
//     features and J H J = L L^T (Cholesky), then U = J L^-1 J. So: a blocked
//     right-looking Cholesky of the reversed H and a blocked right-looking
//     inverse of the lower factor, both made of small in-LDS kernels for the
//     64-row diagonal steps and float64 matrix-core products of rank 64 for
//     everything below them;
//  6. the features in blocks of 64: one thread per channel row runs the 64
//     decisions of the block with the row's 64 weights in registers, each
//     decision's error divided by U[k][k] is removed from the later weights of
//     the block along row k of U, and the errors of the block are removed from
//     all later features by one matrix-core product E * U[block, later];
//  7. the codes are packed into the chunk-major tiled layout of the linear.
#include "weight_codes.h"

namespace qift {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kGptqThreads = 256;
constexpr int kTri = 64;       // diagonal block of the factorizations
constexpr int kColBlock = 64;  // features per column block of the quantization loop
constexpr int64_t kCalibChunk = 4096;  // calibration rows rotated per product

// --- 1. rotation into float64 -------------------------------------------------

__device__ __forceinline__ double load_f64(const float* p, int64_t i) { return (double)p[i]; }
__device__ __forceinline__ double load_f64(const uint16_t* p, int64_t i) {
  return (double)bf16_bits_to_float(p[i]);
}

// One workgroup per segment of L consecutive features of one row (L a power
// of two, a multiple of the block, L | K): log2(block) butterfly stages in LDS,
// then the 1/sqrt(block) normalization; round_f32 rounds every result to
// float32 (kept in float64).
template <typename T>
__global__ __launch_bounds__(kGptqThreads) void rotate_rows_f64_kernel(
    const T* __restrict__ src, int64_t K, int L, int log2b, double norm, int round_f32,
    double* __restrict__ dst) {
  __shared__ double seg[4096];
  const int tid = threadIdx.x;
  const int64_t per_row = K / L;
  const int64_t row = blockIdx.x / per_row;
  const int64_t base = row * K + (int64_t)(blockIdx.x % per_row) * L;
  for (int i = tid; i < L; i += kGptqThreads) seg[i] = load_f64(src, base + i);
  __syncthreads();
  for (int st = 0; st < log2b; ++st) {
    const int h = 1 << st;
    for (int p = tid; p < L / 2; p += kGptqThreads) {
      const int i = ((p >> st) << (st + 1)) | (p & (h - 1));
      const double a = seg[i], b = seg[i + h];
      seg[i] = a + b;
      seg[i + h] = a - b;
    }
    __syncthreads();
  }
  for (int i = tid; i < L; i += kGptqThreads) {
    double v = seg[i] * norm;
    if (round_f32) v = (double)(float)v;
    dst[base + i] = v;
  }
}

// --- 2. float64 products on the matrix cores --------------------------------------
//
// C(m, n) = alpha * sum_k opA(m, k) opB(k, n) + beta * C(m, n) (C is not read
// when beta == 0), opA(m, k) = A[m lda + k] or, transposed, A[k lda + m];
// opB(k, n) = B[k ldb + n] or B[n ldb + k]. lower: only n <= m is computed
// and written. 64 x 64 tiles, 16 features per LDS stage, four waves of 32 x
// 32, each as 2 x 2 blocks of v_mfma_f64_16x16x4f64 (operand lane l: row or
// column l % 16, feature l / 16; result register r of lane l: row l / 16 +
// 4 r, column l % 16 -- the rows interleave, unlike the 32-bit results).

struct GemmArgs {
  const double* A;
  int64_t lda;
  int ta;
  const double* B;
  int64_t ldb;
  int tb;
  double* C;
  int64_t ldc;
  int64_t M, N, K;
  double alpha, beta;
  int lower;
};

constexpr int kGT = 64, kGK = 16;

__global__ __launch_bounds__(kGptqThreads) void gemm_f64_kernel(GemmArgs g) {
  __shared__ double As[kGK][kGT + 1];
  __shared__ double Bs[kGK][kGT + 1];
  const int64_t m0 = (int64_t)blockIdx.y * kGT, n0 = (int64_t)blockIdx.x * kGT;
  if (g.lower && n0 > m0 + kGT - 1) return;  // tile entirely above the diagonal
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int r16 = lane & 15, kq = lane >> 4;
  v4d acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};

  // the stage's tiles go global -> registers -> LDS; the next stage's global
  // loads are issued before the current stage's products, so their latency
  // is hidden (the contiguous dimension across neighbouring threads)
  double ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int mm, kk;
      if (g.ta) {
        mm = tid & 63;
        kk = (tid >> 6) + 4 * i;
      } else {
        kk = tid & 15;
        mm = (tid >> 4) + 16 * i;
      }
      const int64_t m = m0 + mm, k = k0 + kk;
      ra[i] = (m < g.M && k < g.K) ? (g.ta ? g.A[k * g.lda + m] : g.A[m * g.lda + k]) : 0.0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int nn, kk;
      if (g.tb) {
        kk = tid & 15;
        nn = (tid >> 4) + 16 * i;
      } else {
        nn = tid & 63;
        kk = (tid >> 6) + 4 * i;
      }
      const int64_t n = n0 + nn, k = k0 + kk;
      rb[i] = (n < g.N && k < g.K) ? (g.tb ? g.B[n * g.ldb + k] : g.B[k * g.ldb + n]) : 0.0;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (g.ta) As[(tid >> 6) + 4 * i][tid & 63] = ra[i];
      else As[tid & 15][(tid >> 4) + 16 * i] = ra[i];
      if (g.tb) Bs[tid & 15][(tid >> 4) + 16 * i] = rb[i];
      else Bs[(tid >> 6) + 4 * i][tid & 63] = rb[i];
    }
  };
  if (g.K > 0) gload(0);
  for (int64_t k0 = 0; k0 < g.K; k0 += kGK) {
    lstore();
    __syncthreads();
    if (k0 + kGK < g.K) gload(k0 + kGK);
#pragma unroll
    for (int ks = 0; ks < kGK; ks += 4) {
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[ks + kq][wm + 16 * i + r16];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[ks + kq][wn + 16 * j + r16];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm + 16 * i + kq + 4 * r;
        const int64_t n = n0 + wn + 16 * j + r16;
        if (m >= g.M || n >= g.N || (g.lower && n > m)) continue;
        double* c = g.C + m * g.ldc + n;
        const double v = g.alpha * acc[i][j][r];
        *c = g.beta != 0.0 ? v + g.beta * *c : v;
      }
}

static hipError_t gemm_f64(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((g.N + kGT - 1) / kGT), (unsigned)((g.M + kGT - 1) / kGT));
  hipLaunchKernelGGL(gemm_f64_kernel, grid, dim3(kGptqThreads), 0, s, g);
  return hipGetLastError();
}

// --- small kernels ------------------------------------------------------------------

__global__ void fill_f64_kernel(double* __restrict__ p, int64_t n, double v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// H[j][i] = H[i][j] for i > j (the products fill the lower triangle)
__global__ void mirror_kernel(double* __restrict__ H, int64_t K) {
  const int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  if (i < K && j < K && i > j) H[j * K + i] = H[i * K + j];
}

// 4. dead features and the damping: lam = damp * mean(diag H) after the dead
// diagonal entries became 1 (fixed summation order: one workgroup).
__global__ __launch_bounds__(kGptqThreads) void gptq_diag_kernel(const double* __restrict__ H,
                                                                 int64_t K, double damp,
                                                                 double* __restrict__ lam,
                                                                 uint8_t* __restrict__ dead) {
  __shared__ double red[kGptqThreads / 64];
  const int tid = threadIdx.x;
  double sum = 0.0;
  for (int64_t k = tid; k < K; k += kGptqThreads) {
    const double d = H[k * K + k];
    dead[k] = d == 0.0 ? 1 : 0;
    sum += d == 0.0 ? 1.0 : d;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kGptqThreads / 64; ++w) t += red[w];
    lam[0] = damp * (t / (double)K);
  }
}

// A = J H J + lam I with the dead diagonal entries set to 1 (the whole matrix;
// H symmetric)
__global__ void gptq_reverse_kernel(const double* __restrict__ H, int64_t K,
                                    const double* __restrict__ lam,
                                    const uint8_t* __restrict__ dead, double* __restrict__ A) {
  const int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  if (i >= K || j >= K) return;
  const int64_t si = K - 1 - i, sj = K - 1 - j;
  double v = H[si * K + sj];
  if (i == j) v = (dead[si] ? 1.0 : v) + lam[0];
  A[i * K + j] = v;
}

// U[i][j] = Li[K-1-i][K-1-j] (Li = L^-1, lower; U upper, its lower part 0)
__global__ void gptq_unreverse_kernel(const double* __restrict__ Li, int64_t K,
                                      double* __restrict__ U) {
  const int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  if (i >= K || j >= K) return;
  U[i * K + j] = j >= i ? Li[(K - 1 - i) * K + (K - 1 - j)] : 0.0;
}

// --- 5. Cholesky and the inverse of the lower factor ---------------------------------

// The 64 x 64 diagonal-step kernels below give each of 256 threads a 4 x 4
// piece of the block in registers (rows 4 (t / 16) .., columns 4 (t % 16) ..);
// the column (or row) that a step divides is passed through LDS, double
// buffered by the step's parity so that one barrier per step orders both its
// write and the previous step's reads. Outside the first jb (kb) rows and
// columns the block is the identity.

// Cholesky of the jb x jb diagonal block at (j0, j0) in place (lower part).
__global__ __launch_bounds__(kGptqThreads) void potrf_diag_kernel(double* __restrict__ A,
                                                                  int64_t K, int64_t j0, int jb) {
  __shared__ double col[2][kTri];
  __shared__ double dg[2];
  const int tid = threadIdx.x;
  const int rb = 4 * (tid >> 4), cb = 4 * (tid & 15);
  double a[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb + i, c = cb + j;
      a[i][j] = (r < jb && c <= r) ? A[(j0 + r) * K + j0 + c] : (r == c ? 1.0 : 0.0);
    }
  for (int blk = 0; blk < kTri / 4; ++blk) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int c = 4 * blk + cc, par = c & 1;
      if (rb == 4 * blk && cb == 4 * blk) {  // owner of the diagonal entry
        a[cc][cc] = sqrt(a[cc][cc]);
        dg[par] = a[cc][cc];
      }
      __syncthreads();
      if (cb == 4 * blk) {  // owners of column c
        const double d = dg[par];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (rb + i > c) a[i][cc] /= d;
          col[par][rb + i] = rb + i > c ? a[i][cc] : 0.0;
        }
      }
      __syncthreads();
      // branch-free: every entry reads the column and selects 0 where the
      // update does not apply (per-entry branches cost more than the FMAs)
      double cq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) cq[j] = col[par][cb + j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double lr = col[par][rb + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = cb + j;
          const double f = (q > c && rb + i >= q) ? cq[j] : 0.0;
          a[i][j] = __builtin_fma(-lr, f, a[i][j]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb + i, c = cb + j;
      if (r < jb && c <= r) A[(j0 + r) * K + j0 + c] = a[i][j];
    }
}

// Panel below the factored diagonal block: rows r >= j0 + jb get
// A[r, j0 : j0+jb] <- A[r, j0 : j0+jb] L_jj^-T. A workgroup solves 64 rows,
// one feature (column) per step, right-looking: once column c is final it is
// removed from the later columns.
__global__ __launch_bounds__(kGptqThreads) void trsm_panel_kernel(double* __restrict__ A,
                                                                  int64_t K, int64_t j0, int jb) {
  __shared__ double L[kTri][kTri + 1];
  __shared__ double col[2][kTri];
  const int tid = threadIdx.x;
  const int rb = 4 * (tid >> 4), cb = 4 * (tid & 15);
  const int64_t r0 = j0 + jb + (int64_t)blockIdx.x * kTri;
  const int rows = (int)(K - r0 < kTri ? K - r0 : kTri);
  for (int idx = tid; idx < kTri * kTri; idx += kGptqThreads) {
    const int r = idx / kTri, c = idx % kTri;
    L[r][c] = (r < jb && c <= r) ? A[(j0 + r) * K + j0 + c] : (r == c ? 1.0 : 0.0);
  }
  double x[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb + i, c = cb + j;
      x[i][j] = (r < rows && c < jb) ? A[(r0 + r) * K + j0 + c] : 0.0;
    }
  __syncthreads();
  for (int blk = 0; blk < kTri / 4; ++blk) {
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int c = 4 * blk + cc, par = c & 1;
      if (cb == 4 * blk) {
        const double d = L[c][c];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i][cc] /= d;
          col[par][rb + i] = x[i][cc];
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = cb + j;
        const double l = q > c ? L[q][c] : 0.0;  // branch-free
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i][j] = __builtin_fma(-col[par][rb + i], l, x[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb + i, c = cb + j;
      if (r < rows && c < jb) A[(r0 + r) * K + j0 + c] = x[i][j];
    }
}

// Block row k0 .. k0 + kb - 1 of the inverse, in place: the rows hold the
// right-hand side B (the identity minus the contributions of the earlier block
// rows) and become Y with L_kk Y = B. One workgroup per 64 columns (columns
// >= k0 + kb are zero and stay so), one row of Y per step (right-looking).
__global__ __launch_bounds__(kGptqThreads) void trsm_rows_kernel(const double* __restrict__ A,
                                                                 double* __restrict__ Li,
                                                                 int64_t K, int64_t k0, int kb) {
  __shared__ double L[kTri][kTri + 1];
  __shared__ double row[2][kTri];
  const int tid = threadIdx.x;
  const int rb = 4 * (tid >> 4), cb = 4 * (tid & 15);
  const int64_t c0 = (int64_t)blockIdx.x * kTri;
  const int cols = (int)(K - c0 < kTri ? K - c0 : kTri);
  for (int idx = tid; idx < kTri * kTri; idx += kGptqThreads) {
    const int r = idx / kTri, c = idx % kTri;
    L[r][c] = (r < kb && c <= r) ? A[(k0 + r) * K + k0 + c] : (r == c ? 1.0 : 0.0);
  }
  double y[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb + i, c = cb + j;
      y[i][j] = (r < kb && c < cols) ? Li[(k0 + r) * K + c0 + c] : 0.0;
    }
  __syncthreads();
  for (int blk = 0; blk < kTri / 4; ++blk) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int q = 4 * blk + qq, par = q & 1;
      if (rb == 4 * blk) {
        const double d = L[q][q];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[qq][j] /= d;
          row[par][cb + j] = y[qq][j];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb + i;
        const double l = r > q ? L[r][q] : 0.0;  // branch-free
#pragma unroll
        for (int j = 0; j < 4; ++j) y[i][j] = __builtin_fma(-l, row[par][cb + j], y[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rb + i, c = cb + j;
      if (r < kb && c < cols) Li[(k0 + r) * K + c0 + c] = y[i][j];
    }
}

// Li = I
__global__ void identity_kernel(double* __restrict__ Li, int64_t K) {
  const int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4);
  const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
  if (i < K && j < K) Li[i * K + j] = i == j ? 1.0 : 0.0;
}

// --- 3. scales ------------------------------------------------------------------------

__global__ __launch_bounds__(kRowThreads) void gptq_scales_kernel(
    const double* __restrict__ Wr, int K, int levels, uint32_t table, uint32_t pref,
    float outer, int mse_rule, void* __restrict__ scales, int scale_f16) {
  extern __shared__ float row[];
  __shared__ float red[kRowThreads / 64];
  __shared__ double red64[kRowThreads / 64];
  const int tid = threadIdx.x;
  const int64_t n = blockIdx.x;
  for (int i = tid; i < K; i += kRowThreads) row[i] = (float)Wr[n * K + i];  // exact
  __syncthreads();
  const float s32 =
      choose_scale(row, K, 1.0f, levels, table, pref, outer, mse_rule, scale_f16, red, red64);
  if (tid == 0) {
    if (scale_f16)
      reinterpret_cast<__half*>(scales)[n] = __float2half_rn(s32);
    else
      reinterpret_cast<float*>(scales)[n] = s32;
  }
}

// --- 6. one block of features ------------------------------------------------------------
//
// Features b0 .. b0 + bb - 1 of channel row n (one thread per row): feature j
// takes the code of its current weight rounded to float32 against the stored
// scale; err = (w - level * s) / U[j][j] is kept in E and removed from the
// later weights of the block along row j of U.
constexpr int kBlockThreads = 256;  // (one-wave workgroups, spread over more CUs, ran 20% slower)

__global__ __launch_bounds__(kBlockThreads) void gptq_block_kernel(
    double* __restrict__ Wr, int64_t N, int64_t K, int64_t b0, int bb,
    const double* __restrict__ U, const void* __restrict__ scales, int scale_f16, int levels,
    uint32_t table, uint32_t pref, const uint8_t* __restrict__ dead,
    uint8_t* __restrict__ codes8, double* __restrict__ E) {
  __shared__ double Ub[kColBlock][kColBlock + 1];
  __shared__ uint8_t dd[kColBlock];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kColBlock * kColBlock; idx += kBlockThreads) {
    const int j = idx / kColBlock, l = idx % kColBlock;
    Ub[j][l] = (j < bb && l < bb && l >= j) ? U[(b0 + j) * K + b0 + l] : (j == l ? 1.0 : 0.0);
  }
  if (tid < kColBlock) dd[tid] = tid < bb ? dead[b0 + tid] : 1;
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * kBlockThreads + tid;
  if (n >= N) return;
  const float sf = scale_f16 ? __half2float(reinterpret_cast<const __half*>(scales)[n])
                             : reinterpret_cast<const float*>(scales)[n];
  const double sd = (double)sf;
  const bool int4 = levels == QIFT_LEVELS_INT4;
  double* wrow = Wr + n * K + b0;
  double w[kColBlock];
#pragma unroll
  for (int j = 0; j < kColBlock; ++j) w[j] = (j < bb && !dd[j]) ? wrow[j] : 0.0;
#pragma unroll
  for (int j = 0; j < kColBlock; ++j) {
    if (j < bb) {
      const float w32 = (float)w[j];
      double deq;
      uint8_t c;
      if (int4) {
        const int q = quant_int4(w32, sf);
        c = (uint8_t)(q & 0xFF);
        deq = (double)q * sd;
      } else {
        const uint32_t cc = code2(levels, w32, sf, table, pref);
        c = (uint8_t)cc;
        deq = real_level(levels, cc, table) * sd;
      }
      codes8[n * K + b0 + j] = c;
      const double e = (w[j] - deq) / Ub[j][j];
      E[n * kColBlock + j] = e;
#pragma unroll
      for (int l = j + 1; l < kColBlock; ++l) w[l] -= e * Ub[j][l];
    }
  }
}

// --- 7. packing -------------------------------------------------------------------------

__global__ void gptq_pack_kernel(const uint8_t* __restrict__ codes8, int64_t N, int64_t K,
                                 int int4, uint32_t* __restrict__ codes) {
  const int64_t words = int4 ? K / 8 : K / 16;
  const int64_t tiles = (N + 15) >> 4;
  const int64_t total = tiles * 16 * words;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t n = idx / words, w = idx % words;
  uint32_t word = 0;
  if (n < N) {
    if (int4) {
      const uint8_t* c = codes8 + n * K + 8 * w;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= ((uint32_t)c[i] & 0xFu) << (4 * i);
    } else {
      const uint8_t* c = codes8 + n * K + 16 * w;
#pragma unroll
      for (int i = 0; i < 16; ++i) word |= ((uint32_t)c[i] & 3u) << code_bit_offset(i);
    }
  }
  codes[tiled_word(n, w, words, tiles)] = word;
}

// --- launchers ----------------------------------------------------------------------------

static int ilog2_i(int64_t v) {
  int r = 0;
  while (((int64_t)1 << r) < v) ++r;
  return r;
}

// segment of the rotation kernel: the largest power of two <= 4096 dividing K
// (at least the block)
static int rotate_segment(int64_t K, int had_block) {
  int L = 4096;
  while (L > had_block && K % L != 0) L >>= 1;
  return L;
}

static hipError_t rotate_rows_f64(const void* src, int bf16, int64_t rows, int64_t K,
                                  int had_block, int round_f32, double* dst, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int L = rotate_segment(K, had_block);
  const int lb = ilog2_i(had_block);
  const double norm = 1.0 / __builtin_sqrt((double)had_block);
  const unsigned grid = (unsigned)(rows * (K / L));
  if (bf16)
    hipLaunchKernelGGL(rotate_rows_f64_kernel<uint16_t>, dim3(grid), dim3(kGptqThreads), 0, s,
                       reinterpret_cast<const uint16_t*>(src), K, L, lb, norm, round_f32, dst);
  else
    hipLaunchKernelGGL(rotate_rows_f64_kernel<float>, dim3(grid), dim3(kGptqThreads), 0, s,
                       reinterpret_cast<const float*>(src), K, L, lb, norm, round_f32, dst);
  return hipGetLastError();
}

static dim3 grid16(int64_t K) {
  return dim3((unsigned)((K + 15) / 16), (unsigned)((K + 15) / 16));
}

size_t gptq_hessian_workspace_bytes(int64_t S, int64_t K) {
  const int64_t rows = S < kCalibChunk ? S : kCalibChunk;
  return (size_t)(rows > 0 ? rows : 1) * (size_t)K * sizeof(double);
}

hipError_t launch_gptq_hessian(const void* X, int x_bf16, int64_t S, int64_t K, int had_block,
                               int accumulate, double* H, void* workspace, hipStream_t s) {
  double* xr = reinterpret_cast<double*>(workspace);
  hipError_t e = hipSuccess;
  if (S == 0 && !accumulate) {
    hipLaunchKernelGGL(fill_f64_kernel, dim3(1024), dim3(256), 0, s, H, K * K, 0.0);
    return hipGetLastError();
  }
  const size_t esz = x_bf16 ? 2 : 4;
  for (int64_t c0 = 0; c0 < S; c0 += kCalibChunk) {
    const int64_t rows = S - c0 < kCalibChunk ? S - c0 : kCalibChunk;
    const void* src = reinterpret_cast<const char*>(X) + (size_t)c0 * (size_t)K * esz;
    if ((e = rotate_rows_f64(src, x_bf16, rows, K, had_block, 0, xr, s)) != hipSuccess) return e;
    GemmArgs g{xr, K, 1, xr, K, 0, H, K, K, K, rows, 1.0,
               (accumulate || c0 > 0) ? 1.0 : 0.0, 1};
    if ((e = gemm_f64(g, s)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mirror_kernel, grid16(K), dim3(256), 0, s, H, K);
  return hipGetLastError();
}

namespace {
struct GptqWork {
  double *Wr, *A, *Li, *E, *lam;
  uint8_t *codes8, *dead;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t carve(void* base, int64_t N, int64_t K, GptqWork* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = reinterpret_cast<char*>(base) + off;
    off = align256(off + bytes);
    return p;
  };
  const size_t d = sizeof(double);
  w->Wr = reinterpret_cast<double*>(take((size_t)N * K * d));
  w->A = reinterpret_cast<double*>(take((size_t)K * K * d));
  w->Li = reinterpret_cast<double*>(take((size_t)K * K * d));
  w->E = reinterpret_cast<double*>(take((size_t)N * kColBlock * d));
  w->lam = reinterpret_cast<double*>(take(d));
  w->codes8 = reinterpret_cast<uint8_t*>(take((size_t)N * K));
  w->dead = reinterpret_cast<uint8_t*>(take((size_t)K));
  return off;
}
}  // namespace

size_t gptq_workspace_bytes(int64_t N, int64_t K) {
  GptqWork w;
  return carve(nullptr, N, K, &w);
}

hipError_t launch_gptq_quantize(const void* W, int w_bf16, int64_t N, int64_t K,
                                const double* H, int had_block, int levels, uint32_t table,
                                int mse_rule, double damp, uint32_t* codes, void* scales,
                                int scale_f16, void* workspace, hipStream_t s) {
  GptqWork w;
  carve(workspace, N, K, &w);
  hipError_t e;
  // 1. rotated weights, rounded to float32
  if ((e = rotate_rows_f64(W, w_bf16, N, K, had_block, 1, w.Wr, s)) != hipSuccess) return e;
  // 3. scales
  uint32_t pref = 0;
  const float outer = level_outer_and_pref(levels, table, &pref);
  hipLaunchKernelGGL(gptq_scales_kernel, dim3((unsigned)N), dim3(kRowThreads),
                     (size_t)K * sizeof(float), s, w.Wr, (int)K, levels, table, pref, outer,
                     mse_rule, scales, scale_f16);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 4. damping, reversed order
  hipLaunchKernelGGL(gptq_diag_kernel, dim3(1), dim3(kGptqThreads), 0, s, H, K, damp, w.lam,
                     w.dead);
  hipLaunchKernelGGL(gptq_reverse_kernel, grid16(K), dim3(256), 0, s, H, K, w.lam, w.dead, w.A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 5a. Cholesky of the reversed matrix (lower factor in place)
  for (int64_t j0 = 0; j0 < K; j0 += kTri) {
    const int jb = (int)(K - j0 < kTri ? K - j0 : kTri);
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(kGptqThreads), 0, s, w.A, K, j0, jb);
    const int64_t rest = K - j0 - jb;
    if (rest > 0) {
      hipLaunchKernelGGL(trsm_panel_kernel, dim3((unsigned)((rest + kTri - 1) / kTri)),
                         dim3(kGptqThreads), 0, s, w.A, K, j0, jb);
      const double* P = w.A + (j0 + jb) * K + j0;
      GemmArgs g{P, K, 0, P, K, 1, w.A + (j0 + jb) * K + (j0 + jb), K, rest, rest, jb,
                 -1.0, 1.0, 1};
      if ((e = gemm_f64(g, s)) != hipSuccess) return e;
    }
  }
  // 5b. Li = L^-1, right-looking: block row k solved against L_kk, then
  // removed from every later block row (Li[k0+kb:, :k0+kb] -= L[k0+kb:, k] Y_k)
  hipLaunchKernelGGL(identity_kernel, grid16(K), dim3(256), 0, s, w.Li, K);
  for (int64_t k0 = 0; k0 < K; k0 += kTri) {
    const int kb = (int)(K - k0 < kTri ? K - k0 : kTri);
    const int64_t ncols = k0 + kb;
    hipLaunchKernelGGL(trsm_rows_kernel, dim3((unsigned)((ncols + kTri - 1) / kTri)),
                       dim3(kGptqThreads), 0, s, w.A, w.Li, K, k0, kb);
    const int64_t rest = K - k0 - kb;
    if (rest > 0) {
      GemmArgs g{w.A + (k0 + kb) * K + k0, K, 0, w.Li + k0 * K, K, 0, w.Li + (k0 + kb) * K, K,
                 rest, ncols, kb, -1.0, 1.0, 0};
      if ((e = gemm_f64(g, s)) != hipSuccess) return e;
    }
  }
  // U = J Li J, into A
  hipLaunchKernelGGL(gptq_unreverse_kernel, grid16(K), dim3(256), 0, s, w.Li, K, w.A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 6. the column blocks
  const unsigned rows_grid = (unsigned)((N + kBlockThreads - 1) / kBlockThreads);
  for (int64_t b0 = 0; b0 < K; b0 += kColBlock) {
    const int bb = (int)(K - b0 < kColBlock ? K - b0 : kColBlock);
    hipLaunchKernelGGL(gptq_block_kernel, dim3(rows_grid), dim3(kBlockThreads), 0, s, w.Wr, N, K,
                       b0, bb, w.A, scales, scale_f16, levels, table, pref, w.dead, w.codes8,
                       w.E);
    const int64_t rest = K - b0 - bb;
    if (rest > 0) {
      GemmArgs g{w.E, kColBlock, 0, w.A + b0 * K + b0 + bb, K, 0, w.Wr + b0 + bb, K, N, rest,
                 bb, -1.0, 1.0, 0};
      if ((e = gemm_f64(g, s)) != hipSuccess) return e;
    }
  }
  // 7. pack
  const int int4 = levels == QIFT_LEVELS_INT4;
  const int64_t total = (N + 15) / 16 * 16 * (int4 ? K / 8 : K / 16);
  hipLaunchKernelGGL(gptq_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     w.codes8, N, K, int4, codes);
  return hipGetLastError();
}

}  // namespace qift
