// C ABI of libqift: argument validation, dispatch to the HIP kernels, and the
// host side of the grouped-linear plan. Every check runs before anything is
// enqueued, so an invalid call touches neither the device nor the outputs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "qift.h"
#include "qift_measure.h"
#include "qift_internal.h"

namespace {

thread_local std::string g_last_error;

qift_status fail(qift_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

qift_status ok() {
  g_last_error.clear();
  return QIFT_OK;
}

qift_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QIFT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_levels(int lv) {
  return lv == QIFT_LEVELS_MNZ || lv == QIFT_LEVELS_POT || lv == QIFT_LEVELS_INT4 ||
         lv == QIFT_LEVELS_LUT || lv == QIFT_LEVELS_ASYM;
}

// The table word of a call: a level table (four signed bytes, |L| <= 15, not
// all zero) for QIFT_LEVELS_LUT, 0 for every other level kind.
qift_status check_table(int levels, uint32_t table) {
  if (levels != QIFT_LEVELS_LUT) {
    if (table != 0) return fail(QIFT_ERR_INVALID_ARG, "level table given for levels %d", levels);
    return QIFT_OK;
  }
  bool any = false;
  for (int c = 0; c < 4; ++c) {
    const int L = (int)(int8_t)((table >> (8 * c)) & 0xFFu);
    if (L < -15 || L > 15)
      return fail(QIFT_ERR_INVALID_ARG, "level table entry %d is %d, outside [-15, 15]", c, L);
    any = any || L != 0;
  }
  if (!any) return fail(QIFT_ERR_INVALID_ARG, "level table is all zero");
  return QIFT_OK;
}

constexpr int64_t kMaxLinearK = 65536;
constexpr int64_t kMaxGrid = 0x7fffffffLL;

qift_status check_had_block(int64_t B, int64_t K, int64_t max_b) {
  if (!is_pow2(B)) return fail(QIFT_ERR_INVALID_ARG, "had_block=%lld is not a power of two", (long long)B);
  if (B > max_b) return fail(QIFT_ERR_UNSUPPORTED, "had_block=%lld exceeds %lld", (long long)B, (long long)max_b);
  if (K % B != 0) return fail(QIFT_ERR_INVALID_ARG, "had_block=%lld does not divide K=%lld", (long long)B, (long long)K);
  return QIFT_OK;
}

// Shared rules of qift_w2a4_linear and of each grouped descriptor. With
// dtypes_known = false (sizing a grouped plan, before its dtypes are given)
// the dtype-dependent checks of scales and Y are left to the later call.
qift_status check_linear(const qift_linear_desc& d, qift_dtype scale_dtype, qift_dtype y_dtype,
                         bool dtypes_known = true) {
  if (d.M < 0 || d.N < 0) return fail(QIFT_ERR_INVALID_ARG, "negative M or N");
  if (d.K <= 0 || d.K % 64 != 0)
    return fail(QIFT_ERR_INVALID_ARG, "K=%lld must be a positive multiple of 64", (long long)d.K);
  if (d.K > kMaxLinearK)
    return fail(QIFT_ERR_UNSUPPORTED, "K=%lld exceeds %lld", (long long)d.K, (long long)kMaxLinearK);
  if (!valid_levels(d.levels)) return fail(QIFT_ERR_INVALID_ARG, "invalid levels %d", d.levels);
  qift_status tst = check_table(d.levels, (uint32_t)d.reserved);
  if (tst != QIFT_OK) return tst;
  if (dtypes_known && scale_dtype != QIFT_F32 && scale_dtype != QIFT_F16)
    return fail(QIFT_ERR_INVALID_ARG, "scale_dtype must be F32 or F16");
  if (dtypes_known && y_dtype != QIFT_F32 && y_dtype != QIFT_BF16 && y_dtype != QIFT_I32)
    return fail(QIFT_ERR_INVALID_ARG, "y_dtype must be F32, BF16 or I32");
  if (d.M == 0 || d.N == 0) return QIFT_OK;
  if (!d.xq || !d.s_a || !d.codes || !d.scales || !d.Y)
    return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(d.xq, 16) || !aligned(d.codes, 16))
    return fail(QIFT_ERR_ALIGNMENT, "xq and codes must be 16-byte aligned");
  if (!aligned(d.s_a, 4)) return fail(QIFT_ERR_ALIGNMENT, "s_a must be 4-byte aligned");
  if (dtypes_known && (!aligned(d.scales, scale_dtype == QIFT_F16 ? 2 : 4) ||
                       !aligned(d.Y, y_dtype == QIFT_BF16 ? 2 : 4)))
    return fail(QIFT_ERR_ALIGNMENT, "scales or Y misaligned for its dtype");
  if ((d.N + qift::kDecodeRowsPerTile - 1) / qift::kDecodeRowsPerTile > kMaxGrid)
    return fail(QIFT_ERR_UNSUPPORTED, "N too large");
  return QIFT_OK;
}

}  // namespace

extern "C" {

int32_t qift_abi_version(void) { return QIFT_ABI_VERSION; }

const char* qift_last_error(void) { return g_last_error.c_str(); }

const char* qift_status_string(qift_status s) {
  switch (s) {
    case QIFT_OK: return "QIFT_OK";
    case QIFT_ERR_INVALID_ARG: return "QIFT_ERR_INVALID_ARG";
    case QIFT_ERR_ALIGNMENT: return "QIFT_ERR_ALIGNMENT";
    case QIFT_ERR_UNSUPPORTED: return "QIFT_ERR_UNSUPPORTED";
    case QIFT_ERR_HIP: return "QIFT_ERR_HIP";
  }
  return "QIFT_ERR_UNKNOWN";
}

qift_status qift_quantize_weights(const void* W, qift_dtype w_dtype, int64_t N, int64_t K,
                                  int32_t had_block, qift_levels levels, uint32_t* codes,
                                  void* scales, qift_dtype scale_dtype, qift_stream stream) {
  return qift_quantize_weights_ex(W, w_dtype, N, K, had_block, levels, 0u, QIFT_SCALE_ABSMAX,
                                  codes, scales, scale_dtype, stream);
}

qift_status qift_quantize_weights_ex(const void* W, qift_dtype w_dtype, int64_t N, int64_t K,
                                     int32_t had_block, qift_levels levels, uint32_t level_table,
                                     qift_scale_rule scale_rule, uint32_t* codes, void* scales,
                                     qift_dtype scale_dtype, qift_stream stream) {
  if (w_dtype != QIFT_F32 && w_dtype != QIFT_BF16)
    return fail(QIFT_ERR_INVALID_ARG, "w_dtype must be F32 or BF16");
  if (scale_dtype != QIFT_F32 && scale_dtype != QIFT_F16)
    return fail(QIFT_ERR_INVALID_ARG, "scale_dtype must be F32 or F16");
  if (!valid_levels(levels)) return fail(QIFT_ERR_INVALID_ARG, "invalid levels %d", (int)levels);
  qift_status tst = check_table((int)levels, level_table);
  if (tst != QIFT_OK) return tst;
  if (scale_rule != QIFT_SCALE_ABSMAX && scale_rule != QIFT_SCALE_MSE)
    return fail(QIFT_ERR_INVALID_ARG, "invalid scale_rule %d", (int)scale_rule);
  if (levels == QIFT_LEVELS_ASYM && scale_rule != QIFT_SCALE_ABSMAX)
    return fail(QIFT_ERR_INVALID_ARG, "the asymmetric grid takes its step from the range (ABSMAX)");
  if (N < 0) return fail(QIFT_ERR_INVALID_ARG, "negative N");
  if (K <= 0 || K % 64 != 0)
    return fail(QIFT_ERR_INVALID_ARG, "K=%lld must be a positive multiple of 64", (long long)K);
  if (K > QIFT_MAX_ROW)
    return fail(QIFT_ERR_UNSUPPORTED, "K=%lld exceeds %d", (long long)K, QIFT_MAX_ROW);
  qift_status st = check_had_block(had_block, K, QIFT_MAX_HAD_BLOCK);
  if (st != QIFT_OK) return st;
  if (N == 0) return ok();
  if (N > kMaxGrid) return fail(QIFT_ERR_UNSUPPORTED, "N too large");
  if (!W || !codes || !scales) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(codes, 16)) return fail(QIFT_ERR_ALIGNMENT, "codes must be 16-byte aligned");
  if (!aligned(W, w_dtype == QIFT_F32 ? 4 : 2) || !aligned(scales, scale_dtype == QIFT_F16 ? 2 : 4))
    return fail(QIFT_ERR_ALIGNMENT, "W or scales misaligned for its dtype");
  return hip_result(qift::launch_quantize_weights(W, w_dtype == QIFT_BF16, N, K, had_block,
                                                  (int)levels, level_table,
                                                  scale_rule == QIFT_SCALE_MSE, codes, scales,
                                                  scale_dtype == QIFT_F16,
                                                  reinterpret_cast<hipStream_t>(stream)),
                    "qift_quantize_weights launch");
}

static qift_status check_rotate(const void* X, qift_dtype x_dtype, int64_t M, int64_t K,
                                int32_t had_block, const uint8_t* xq, const float* s_a,
                                const float* x_rot) {
  if (x_dtype != QIFT_F32 && x_dtype != QIFT_BF16)
    return fail(QIFT_ERR_INVALID_ARG, "x_dtype must be F32 or BF16");
  if (M < 0) return fail(QIFT_ERR_INVALID_ARG, "negative M");
  if (K <= 0 || K % 2 != 0)
    return fail(QIFT_ERR_INVALID_ARG, "K=%lld must be positive and even", (long long)K);
  if (K > QIFT_MAX_ROW)
    return fail(QIFT_ERR_UNSUPPORTED, "K=%lld exceeds %d", (long long)K, QIFT_MAX_ROW);
  qift_status st = check_had_block(had_block, K, QIFT_MAX_HAD_BLOCK);
  if (st != QIFT_OK) return st;
  if (M == 0) return QIFT_OK;
  if (M > kMaxGrid) return fail(QIFT_ERR_UNSUPPORTED, "M too large");
  if (!X || !xq || !s_a) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(xq, 16)) return fail(QIFT_ERR_ALIGNMENT, "xq must be 16-byte aligned");
  if (!aligned(X, x_dtype == QIFT_F32 ? 4 : 2) || !aligned(s_a, 4) || (x_rot && !aligned(x_rot, 4)))
    return fail(QIFT_ERR_ALIGNMENT, "X, s_a or x_rot misaligned for its dtype");
  return QIFT_OK;
}

qift_status qift_rotate_quant_act_batched(const qift_rotate_desc* descs, int32_t count,
                                          qift_stream stream) {
  if (count < 0 || count > QIFT_MAX_ROTATE_BATCH)
    return fail(QIFT_ERR_INVALID_ARG, "count=%d outside 0..%d", (int)count,
                QIFT_MAX_ROTATE_BATCH);
  if (count == 0) return ok();
  if (!descs) return fail(QIFT_ERR_INVALID_ARG, "null descs");
  int64_t total = 0;
  for (int j = 0; j < count; ++j) {
    const qift_rotate_desc& r = descs[j];
    qift_status st = check_rotate(r.X, r.x_dtype, r.M, r.K, r.had_block, r.xq, r.s_a, r.x_rot);
    if (st != QIFT_OK) return st;
    total += r.M;
  }
  if (total > kMaxGrid) return fail(QIFT_ERR_UNSUPPORTED, "too many rows in total");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  qift::RotJob jobs[QIFT_MAX_ROTATE_BATCH];
  int64_t rows[QIFT_MAX_ROTATE_BATCH];
  int nj = 0;
  for (int j = 0; j < count; ++j) {
    const qift_rotate_desc& r = descs[j];
    if (r.M == 0) continue;
    if (qift::rotate_fast_ok(r.X, r.K, r.had_block, r.xq, r.x_rot)) {
      jobs[nj] = qift::RotJob{r.X, r.xq, r.s_a, r.x_rot, (int)r.K, (int)r.had_block, 0, 0.f,
                              r.x_dtype == QIFT_BF16};
      rows[nj] = r.M;
      ++nj;
    } else {
      hipError_t e = qift::launch_rotate_quant_act(r.X, r.x_dtype == QIFT_BF16, r.M, r.K,
                                                   r.had_block, r.xq, r.s_a, r.x_rot, s);
      if (e != hipSuccess) return hip_result(e, "qift_rotate_quant_act_batched launch");
    }
  }
  return hip_result(qift::launch_rotate_quant_act_batched(jobs, rows, nj, s),
                    "qift_rotate_quant_act_batched launch");
}

qift_status qift_rotate_quant_act(const void* X, qift_dtype x_dtype, int64_t M, int64_t K,
                                  int32_t had_block, uint8_t* xq, float* s_a, float* x_rot,
                                  qift_stream stream) {
  qift_status st = check_rotate(X, x_dtype, M, K, had_block, xq, s_a, x_rot);
  if (st != QIFT_OK) return st;
  if (M == 0) return ok();
  return hip_result(qift::launch_rotate_quant_act(X, x_dtype == QIFT_BF16, M, K, had_block, xq,
                                                  s_a, x_rot,
                                                  reinterpret_cast<hipStream_t>(stream)),
                    "qift_rotate_quant_act launch");
}

qift_status qift_w2a4_linear(const uint8_t* xq, const float* s_a, int64_t M, int64_t K,
                             const uint32_t* codes, const void* scales, qift_dtype scale_dtype,
                             qift_levels levels, int64_t N, void* Y, qift_dtype y_dtype,
                             qift_stream stream) {
  return qift_w2a4_linear_ex(xq, s_a, M, K, codes, scales, scale_dtype, levels, 0u, N, Y, y_dtype,
                             stream);
}

qift_status qift_w2a4_linear_ex(const uint8_t* xq, const float* s_a, int64_t M, int64_t K,
                                const uint32_t* codes, const void* scales, qift_dtype scale_dtype,
                                qift_levels levels, uint32_t level_table, int64_t N, void* Y,
                                qift_dtype y_dtype, qift_stream stream) {
  qift_linear_desc d{};
  d.reserved = (int32_t)level_table;
  d.xq = xq;
  d.s_a = s_a;
  d.codes = codes;
  d.scales = scales;
  d.Y = Y;
  d.M = M;
  d.K = K;
  d.N = N;
  d.levels = (int32_t)levels;
  qift_status st = check_linear(d, scale_dtype, y_dtype);
  if (st != QIFT_OK) return st;
  if (M == 0 || N == 0) return ok();
  if ((M + 127) / 128 > 65535) return fail(QIFT_ERR_UNSUPPORTED, "M too large");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int sf16 = scale_dtype == QIFT_F16;
  if (M <= 16) return hip_result(qift::launch_linear_decode(d, sf16, y_dtype, s), "qift_w2a4_linear decode launch");
  return hip_result(qift::launch_linear_prefill(d, sf16, y_dtype, s), "qift_w2a4_linear prefill launch");
}

qift_status qift_rotate_w2a4_linear(const void* X, qift_dtype x_dtype, int64_t M, int64_t K,
                                    int32_t had_block, uint8_t* xq, float* s_a,
                                    const uint32_t* codes, const void* scales,
                                    qift_dtype scale_dtype, qift_levels levels,
                                    uint32_t level_table, int64_t N, void* Y, qift_dtype y_dtype,
                                    qift_stream stream) {
  qift_status st = check_rotate(X, x_dtype, M, K, had_block, xq, s_a, nullptr);
  if (st != QIFT_OK) return st;
  qift_linear_desc d{};
  d.reserved = (int32_t)level_table;
  d.xq = xq;
  d.s_a = s_a;
  d.codes = codes;
  d.scales = scales;
  d.Y = Y;
  d.M = M;
  d.K = K;
  d.N = N;
  d.levels = (int32_t)levels;
  st = check_linear(d, scale_dtype, y_dtype);
  if (st != QIFT_OK) return st;
  if (M == 0) return ok();
  if ((M + 127) / 128 > 65535) return fail(QIFT_ERR_UNSUPPORTED, "M too large");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int sf16 = scale_dtype == QIFT_F16;
  // one token row on the fast rotation path: one fused launch
  if (M == 1 && N > 0 && qift::rotate_fast_ok(X, K, had_block, xq, nullptr))
    return hip_result(qift::launch_rotate_linear_decode(d, X, x_dtype == QIFT_BF16, had_block, sf16,
                                                        y_dtype, s),
                      "qift_rotate_w2a4_linear fused launch");
  hipError_t e = qift::launch_rotate_quant_act(X, x_dtype == QIFT_BF16, M, K, had_block, xq, s_a,
                                               nullptr, s);
  if (e != hipSuccess) return hip_result(e, "qift_rotate_w2a4_linear rotation launch");
  if (N == 0) return ok();
  if (M <= 16)
    return hip_result(qift::launch_linear_decode(d, sf16, y_dtype, s), "qift_rotate_w2a4_linear decode launch");
  return hip_result(qift::launch_linear_prefill(d, sf16, y_dtype, s), "qift_rotate_w2a4_linear prefill launch");
}

static qift_status check_kv4(const void* KV, qift_dtype dtype, int64_t T, int64_t H, int64_t D,
                             int32_t had_block, const uint8_t* kvq, const float* scales) {
  if (dtype != QIFT_F32 && dtype != QIFT_BF16)
    return fail(QIFT_ERR_INVALID_ARG, "dtype must be F32 or BF16");
  if (T < 0 || H < 0) return fail(QIFT_ERR_INVALID_ARG, "negative T or H");
  if (!(D == 16 || D == 32 || D == 64 || D == 128 || D == 256))
    return fail(QIFT_ERR_UNSUPPORTED, "D=%lld must be 16, 32, 64, 128 or 256", (long long)D);
  qift_status st = check_had_block(had_block, D, D);
  if (st != QIFT_OK) return st;
  const int64_t rows = T * H;
  if (rows == 0) return QIFT_OK;
  if (rows / 8 + 1 > kMaxGrid) return fail(QIFT_ERR_UNSUPPORTED, "T*H too large");
  if (!KV || !kvq || !scales) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(KV, 16) || !aligned(kvq, 16) || !aligned(scales, 4))
    return fail(QIFT_ERR_ALIGNMENT, "KV and kvq must be 16-byte aligned, scales 4-byte");
  return QIFT_OK;
}

qift_status qift_kv4_quant(const void* KV, qift_dtype dtype, int64_t T, int64_t H, int64_t D,
                           int32_t had_block, uint8_t* kvq, float* scales, qift_stream stream) {
  qift_status st = check_kv4(KV, dtype, T, H, D, had_block, kvq, scales);
  if (st != QIFT_OK) return st;
  if (T * H == 0) return ok();
  return hip_result(qift::launch_kv4(KV, dtype == QIFT_BF16, T * H, (int)D, had_block, kvq, scales,
                                     reinterpret_cast<hipStream_t>(stream)),
                    "qift_kv4_quant launch");
}

static bool ranges_overlap(const void* a, const void* b, size_t bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bytes && y < x + bytes;
}

qift_status qift_kv4_quant_kv(const void* K, const void* V, qift_dtype dtype, int64_t T,
                              int64_t H, int64_t D, int32_t had_block, uint8_t* kq, float* ks,
                              uint8_t* vq, float* vs, qift_stream stream) {
  qift_status st = check_kv4(K, dtype, T, H, D, had_block, kq, ks);
  if (st != QIFT_OK) return st;
  st = check_kv4(V, dtype, T, H, D, had_block, vq, vs);
  if (st != QIFT_OK) return st;
  const int64_t rows = T * H;
  if (rows == 0) return ok();
  if (ranges_overlap(kq, vq, (size_t)(rows * (D / 2))) ||
      ranges_overlap(ks, vs, (size_t)rows * sizeof(float)))
    return fail(QIFT_ERR_INVALID_ARG, "the outputs of K and V overlap");
  return hip_result(qift::launch_kv4_pair(K, V, dtype == QIFT_BF16, rows, (int)D, had_block, kq, ks,
                                          vq, vs, reinterpret_cast<hipStream_t>(stream)),
                    "qift_kv4_quant_kv launch");
}

// --- decode attention over the KV4 cache ------------------------------------------

static qift_status check_attention(int64_t S, int64_t T, int64_t H, int64_t D) {
  if (S < 0 || T < 0 || H < 0) return fail(QIFT_ERR_INVALID_ARG, "negative S, T or H");
  if (D != 128) return fail(QIFT_ERR_UNSUPPORTED, "D=%lld: attention takes D = 128", (long long)D);
  if (H > 64) return fail(QIFT_ERR_UNSUPPORTED, "H=%lld exceeds 64", (long long)H);
  if (S > 65535) return fail(QIFT_ERR_UNSUPPORTED, "S=%lld exceeds 65535", (long long)S);
  if (S > 0 && (T < 1 || H < 1)) return fail(QIFT_ERR_UNSUPPORTED, "T and H must be at least 1");
  return QIFT_OK;
}

qift_status qift_kv4_attention_workspace_bytes(int64_t S, int64_t T, int64_t H, int64_t D,
                                               size_t* bytes) {
  if (!bytes) return fail(QIFT_ERR_INVALID_ARG, "null bytes");
  qift_status st = check_attention(S, T, H, D);
  if (st != QIFT_OK) return st;
  *bytes = S == 0 ? 0 : qift::kv4_attn_workspace_bytes(S, T, (int)H);
  return ok();
}

// Rules shared by both decode-attention entry points (everything except the
// buffer of partial results).
static qift_status check_attention_call(const void* q, qift_dtype q_dtype, int64_t S, int64_t T,
                                        int64_t H, int64_t D, int32_t had_block,
                                        const uint8_t* kq, const float* ks, const uint8_t* vq,
                                        const float* vs, float softmax_scale, const void* out,
                                        qift_dtype out_dtype) {
  if (q_dtype != QIFT_F32 && q_dtype != QIFT_BF16)
    return fail(QIFT_ERR_INVALID_ARG, "q_dtype must be F32 or BF16");
  if (out_dtype != QIFT_F32 && out_dtype != QIFT_BF16)
    return fail(QIFT_ERR_INVALID_ARG, "out_dtype must be F32 or BF16");
  qift_status st = check_attention(S, T, H, D);
  if (st != QIFT_OK) return st;
  st = check_had_block(had_block, D, D);
  if (st != QIFT_OK) return st;
  if (!(softmax_scale == softmax_scale) || softmax_scale > 3.4e38f || softmax_scale < -3.4e38f)
    return fail(QIFT_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (S == 0) return QIFT_OK;
  if (!q || !kq || !ks || !vq || !vs || !out) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(kq, 16) || !aligned(vq, 16))
    return fail(QIFT_ERR_ALIGNMENT, "kq and vq must be 16-byte aligned");
  if (!aligned(q, q_dtype == QIFT_F32 ? 4 : 2) || !aligned(out, out_dtype == QIFT_F32 ? 4 : 2) ||
      !aligned(ks, 4) || !aligned(vs, 4))
    return fail(QIFT_ERR_ALIGNMENT, "q, out, ks or vs misaligned for its dtype");
  return QIFT_OK;
}

qift_status qift_kv4_attention_decode(const void* q, qift_dtype q_dtype, int64_t S, int64_t T,
                                      int64_t H, int64_t D, int32_t had_block,
                                      const uint8_t* kq, const float* ks, const uint8_t* vq,
                                      const float* vs, float softmax_scale, void* out,
                                      qift_dtype out_dtype, void* workspace,
                                      size_t workspace_bytes, qift_stream stream) {
  qift_status st = check_attention_call(q, q_dtype, S, T, H, D, had_block, kq, ks, vq, vs,
                                        softmax_scale, out, out_dtype);
  if (st != QIFT_OK) return st;
  if (S == 0) return ok();
  if (!workspace) return fail(QIFT_ERR_INVALID_ARG, "null workspace");
  if (!aligned(workspace, 256)) return fail(QIFT_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  const size_t need = qift::kv4_attn_workspace_bytes(S, T, (int)H);
  if (workspace_bytes < need)
    return fail(QIFT_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return hip_result(qift::launch_kv4_attention(q, q_dtype == QIFT_BF16, S, T, (int)H, had_block,
                                               kq, ks, vq, vs, softmax_scale, out,
                                               out_dtype == QIFT_BF16,
                                               reinterpret_cast<float*>(workspace),
                                               reinterpret_cast<hipStream_t>(stream)),
                    "qift_kv4_attention_decode launch");
}

qift_status qift_kv4_attention_decode_noalloc(const void* q, qift_dtype q_dtype, int64_t S,
                                              int64_t T, int64_t H, int64_t D, int32_t had_block,
                                              const uint8_t* kq, const float* ks,
                                              const uint8_t* vq, const float* vs,
                                              float softmax_scale, void* out,
                                              qift_dtype out_dtype, qift_stream stream) {
  qift_status st = check_attention_call(q, q_dtype, S, T, H, D, had_block, kq, ks, vq, vs,
                                        softmax_scale, out, out_dtype);
  if (st != QIFT_OK) return st;
  if (S == 0) return ok();
  const size_t need = qift::kv4_attn_workspace_bytes(S, T, (int)H);
  if (need > (size_t)QIFT_ATTENTION_SCRATCH_BYTES)
    return fail(QIFT_ERR_UNSUPPORTED,
                "partial results of %zu bytes exceed the fixed array of %zu bytes "
                "(use qift_kv4_attention_decode with a workspace)",
                need, (size_t)QIFT_ATTENTION_SCRATCH_BYTES);
  float* part = nullptr;
  hipError_t e = qift::kv4_attn_scratch(&part);
  if (e != hipSuccess) return hip_result(e, "qift_kv4_attention_decode_noalloc: scratch address");
  return hip_result(qift::launch_kv4_attention(q, q_dtype == QIFT_BF16, S, T, (int)H, had_block,
                                               kq, ks, vq, vs, softmax_scale, out,
                                               out_dtype == QIFT_BF16, part,
                                               reinterpret_cast<hipStream_t>(stream)),
                    "qift_kv4_attention_decode_noalloc launch");
}

// --- error-compensated weight quantization ----------------------------------------

static qift_status check_gptq_shape(int64_t K, int32_t had_block) {
  if (K <= 0 || K % 64 != 0)
    return fail(QIFT_ERR_INVALID_ARG, "K=%lld must be a positive multiple of 64", (long long)K);
  if (K > QIFT_MAX_ROW)
    return fail(QIFT_ERR_UNSUPPORTED, "K=%lld exceeds %d", (long long)K, QIFT_MAX_ROW);
  return check_had_block(had_block, K, QIFT_MAX_HAD_BLOCK);
}

qift_status qift_gptq_hessian_workspace_bytes(int64_t S, int64_t K, size_t* bytes) {
  if (!bytes) return fail(QIFT_ERR_INVALID_ARG, "null bytes");
  if (S < 0) return fail(QIFT_ERR_INVALID_ARG, "negative S");
  if (K <= 0 || K % 64 != 0)
    return fail(QIFT_ERR_INVALID_ARG, "K=%lld must be a positive multiple of 64", (long long)K);
  if (K > QIFT_MAX_ROW)
    return fail(QIFT_ERR_UNSUPPORTED, "K=%lld exceeds %d", (long long)K, QIFT_MAX_ROW);
  *bytes = qift::gptq_hessian_workspace_bytes(S, K);
  return ok();
}

qift_status qift_gptq_hessian(const void* X, qift_dtype x_dtype, int64_t S, int64_t K,
                              int32_t had_block, int32_t accumulate, double* H, void* workspace,
                              size_t workspace_bytes, qift_stream stream) {
  if (x_dtype != QIFT_F32 && x_dtype != QIFT_BF16)
    return fail(QIFT_ERR_INVALID_ARG, "x_dtype must be F32 or BF16");
  if (S < 0) return fail(QIFT_ERR_INVALID_ARG, "negative S");
  if (accumulate != 0 && accumulate != 1)
    return fail(QIFT_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  qift_status st = check_gptq_shape(K, had_block);
  if (st != QIFT_OK) return st;
  if (S == 0 && accumulate) return ok();
  if (!H || !workspace || (S > 0 && !X)) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(H, 8) || !aligned(workspace, 256) || (S > 0 && !aligned(X, x_dtype == QIFT_F32 ? 4 : 2)))
    return fail(QIFT_ERR_ALIGNMENT, "H 8-byte, workspace 256-byte, X dtype-aligned");
  const size_t need = qift::gptq_hessian_workspace_bytes(S, K);
  if (workspace_bytes < need)
    return fail(QIFT_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return hip_result(qift::launch_gptq_hessian(X, x_dtype == QIFT_BF16, S, K, had_block,
                                              accumulate, H, workspace,
                                              reinterpret_cast<hipStream_t>(stream)),
                    "qift_gptq_hessian launch");
}

qift_status qift_gptq_workspace_bytes(int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(QIFT_ERR_INVALID_ARG, "null bytes");
  if (N < 0) return fail(QIFT_ERR_INVALID_ARG, "negative N");
  if (K <= 0 || K % 64 != 0)
    return fail(QIFT_ERR_INVALID_ARG, "K=%lld must be a positive multiple of 64", (long long)K);
  if (K > QIFT_MAX_ROW)
    return fail(QIFT_ERR_UNSUPPORTED, "K=%lld exceeds %d", (long long)K, QIFT_MAX_ROW);
  *bytes = N == 0 ? 0 : qift::gptq_workspace_bytes(N, K);
  return ok();
}

qift_status qift_gptq_quantize_weights(const void* W, qift_dtype w_dtype, int64_t N, int64_t K,
                                       const double* H, int32_t had_block, qift_levels levels,
                                       uint32_t level_table, qift_scale_rule scale_rule,
                                       double damp, uint32_t* codes, void* scales,
                                       qift_dtype scale_dtype, void* workspace,
                                       size_t workspace_bytes, qift_stream stream) {
  if (w_dtype != QIFT_F32 && w_dtype != QIFT_BF16)
    return fail(QIFT_ERR_INVALID_ARG, "w_dtype must be F32 or BF16");
  if (scale_dtype != QIFT_F32 && scale_dtype != QIFT_F16)
    return fail(QIFT_ERR_INVALID_ARG, "scale_dtype must be F32 or F16");
  if (!valid_levels(levels)) return fail(QIFT_ERR_INVALID_ARG, "invalid levels %d", (int)levels);
  if (levels == QIFT_LEVELS_ASYM)
    return fail(QIFT_ERR_INVALID_ARG, "error-compensated quantization takes the fixed level sets");
  qift_status tst = check_table((int)levels, level_table);
  if (tst != QIFT_OK) return tst;
  if (scale_rule != QIFT_SCALE_ABSMAX && scale_rule != QIFT_SCALE_MSE)
    return fail(QIFT_ERR_INVALID_ARG, "invalid scale_rule %d", (int)scale_rule);
  if (!(damp > 0.0) || damp > 1e300) return fail(QIFT_ERR_INVALID_ARG, "damp must be > 0 and finite");
  if (N < 0) return fail(QIFT_ERR_INVALID_ARG, "negative N");
  qift_status st = check_gptq_shape(K, had_block);
  if (st != QIFT_OK) return st;
  if (N == 0) return ok();
  // the rotation launches one workgroup per segment of at least 64 features
  if (N > kMaxGrid / (K / 64)) return fail(QIFT_ERR_UNSUPPORTED, "N too large");
  if (!W || !H || !codes || !scales || !workspace) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(codes, 16) || !aligned(workspace, 256) || !aligned(H, 8))
    return fail(QIFT_ERR_ALIGNMENT, "codes 16-byte, workspace 256-byte, H 8-byte aligned");
  if (!aligned(W, w_dtype == QIFT_F32 ? 4 : 2) || !aligned(scales, scale_dtype == QIFT_F16 ? 2 : 4))
    return fail(QIFT_ERR_ALIGNMENT, "W or scales misaligned for its dtype");
  const size_t need = qift::gptq_workspace_bytes(N, K);
  if (workspace_bytes < need)
    return fail(QIFT_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return hip_result(qift::launch_gptq_quantize(W, w_dtype == QIFT_BF16, N, K, H, had_block,
                                               (int)levels, level_table,
                                               scale_rule == QIFT_SCALE_MSE, damp, codes, scales,
                                               scale_dtype == QIFT_F16, workspace,
                                               reinterpret_cast<hipStream_t>(stream)),
                    "qift_gptq_quantize_weights launch");
}

// --- grouped linear ------------------------------------------------------------

static qift_status check_group(const qift_linear_desc* descs, int32_t count, qift_dtype scale_dtype,
                               qift_dtype y_dtype, int64_t* total_tiles,
                               bool dtypes_known = true) {
  if (count < 0) return fail(QIFT_ERR_INVALID_ARG, "negative count");
  if (count > 0 && !descs) return fail(QIFT_ERR_INVALID_ARG, "null descriptor array");
  int64_t tiles = 0;
  for (int32_t i = 0; i < count; ++i) {
    const qift_linear_desc& d = descs[i];
    qift_status st = check_linear(d, scale_dtype, y_dtype, dtypes_known);
    if (st != QIFT_OK) {
      g_last_error = "descriptor " + std::to_string(i) + ": " + g_last_error;
      return st;
    }
    if (d.M > 16) return fail(QIFT_ERR_UNSUPPORTED, "descriptor %d: grouped linears take M <= 16", i);
    if (d.M > 0) tiles += (d.N + qift::kDecodeRowsPerTile - 1) / qift::kDecodeRowsPerTile;
  }
  if (tiles > kMaxGrid) return fail(QIFT_ERR_UNSUPPORTED, "too many tiles");
  *total_tiles = tiles;
  return QIFT_OK;
}

static size_t plan_bytes(int32_t count, int64_t tiles) {
  size_t b = sizeof(qift::PlanHeader) + (size_t)count * sizeof(qift::PlanEntry) + (size_t)tiles * 4;
  return (b + 255) & ~(size_t)255;
}

qift_status qift_linear_group_workspace_bytes(const qift_linear_desc* descs, int32_t count,
                                              size_t* bytes) {
  if (!bytes) return fail(QIFT_ERR_INVALID_ARG, "null bytes");
  int64_t tiles = 0;
  // the plan's size does not depend on the dtypes, which prepare checks
  qift_status st = check_group(descs, count, QIFT_F32, QIFT_F32, &tiles, false);
  if (st != QIFT_OK) return st;
  *bytes = plan_bytes(count, tiles);
  return ok();
}

qift_status qift_linear_group_prepare(const qift_linear_desc* descs, int32_t count,
                                      qift_dtype scale_dtype, qift_dtype y_dtype, void* workspace,
                                      size_t workspace_bytes, int64_t* launch_tiles,
                                      qift_stream stream) {
  if (!launch_tiles) return fail(QIFT_ERR_INVALID_ARG, "null launch_tiles");
  int64_t tiles = 0;
  qift_status st = check_group(descs, count, scale_dtype, y_dtype, &tiles);
  if (st != QIFT_OK) return st;
  const size_t need = plan_bytes(count, tiles);
  if (!workspace) return fail(QIFT_ERR_INVALID_ARG, "null workspace");
  if (!aligned(workspace, 256)) return fail(QIFT_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(QIFT_ERR_INVALID_ARG, "workspace has %zu bytes, plan needs %zu", workspace_bytes, need);

  std::vector<uint8_t> host(need, 0);
  auto* h = reinterpret_cast<qift::PlanHeader*>(host.data());
  h->magic = qift::kPlanMagic;
  h->count = count;
  h->scale_f16 = scale_dtype == QIFT_F16;
  h->y_dtype = (int32_t)y_dtype;
  h->total_tiles = tiles;
  h->entries_offset = sizeof(qift::PlanHeader);
  h->tile_map_offset = sizeof(qift::PlanHeader) + (int64_t)count * sizeof(qift::PlanEntry);
  auto* ent = reinterpret_cast<qift::PlanEntry*>(host.data() + h->entries_offset);
  auto* map = reinterpret_cast<int32_t*>(host.data() + h->tile_map_offset);

  // longest rows (largest K) first, so the longest tiles are dispatched first
  std::vector<int32_t> order(count);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return descs[a].K > descs[b].K; });
  int64_t t = 0;
  for (int32_t i = 0; i < count; ++i) {
    ent[i].d = descs[i];
    ent[i].tile_begin = 0;
    ent[i].n_tiles = 0;
  }
  for (int32_t oi = 0; oi < count; ++oi) {
    const int32_t i = order[oi];
    const qift_linear_desc& d = descs[i];
    const int64_t n = (d.M > 0) ? (d.N + qift::kDecodeRowsPerTile - 1) / qift::kDecodeRowsPerTile : 0;
    ent[i].tile_begin = t;
    ent[i].n_tiles = n;
    for (int64_t k = 0; k < n; ++k) map[t + k] = i;
    t += n;
  }
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(workspace, host.data(), need, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_result(e, "qift_linear_group_prepare copy");
  *launch_tiles = tiles;
  return ok();
}

qift_status qift_w2a4_linear_grouped(const void* workspace, int64_t launch_tiles,
                                     qift_stream stream) {
  if (!workspace) return fail(QIFT_ERR_INVALID_ARG, "null workspace");
  if (!aligned(workspace, 256)) return fail(QIFT_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (launch_tiles < 0 || launch_tiles > kMaxGrid)
    return fail(QIFT_ERR_INVALID_ARG, "launch_tiles out of range");
  if (launch_tiles == 0) return ok();
  return hip_result(qift::launch_linear_grouped(workspace, launch_tiles, 0, 0,
                                                reinterpret_cast<hipStream_t>(stream)),
                    "qift_w2a4_linear_grouped launch");
}

qift_status qift_measure_stream(const void* src, void* dst, int64_t bytes, int32_t mode,
                                uint32_t* sink, qift_stream stream) {
  if (mode != 0 && mode != 1) return fail(QIFT_ERR_INVALID_ARG, "mode must be 0 or 1");
  if (bytes <= 0 || bytes % 16 != 0 || bytes > (int64_t(1) << 40))
    return fail(QIFT_ERR_INVALID_ARG, "bytes=%lld must be a positive multiple of 16, at most 2^40",
                (long long)bytes);
  if (!src || !sink || (mode == 1 && !dst)) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(src, 16) || (mode == 1 && !aligned(dst, 16)) || !aligned(sink, 4))
    return fail(QIFT_ERR_ALIGNMENT, "src and dst must be 16-byte aligned, sink 4-byte");
  if (mode == 1) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes)
      return fail(QIFT_ERR_INVALID_ARG, "src and dst overlap");
  }
  return hip_result(qift::launch_measure_stream(src, mode == 1 ? dst : nullptr, bytes, mode, sink,
                                                reinterpret_cast<hipStream_t>(stream)),
                    "qift_measure_stream launch");
}

qift_status qift_measure_mfma_i8(int64_t iters, int64_t workgroups, uint32_t* sink,
                                 uint64_t* clk, qift_stream stream) {
  if (iters < 1 || iters > (int64_t(1) << 24))
    return fail(QIFT_ERR_INVALID_ARG, "iters=%lld outside [1, 2^24]", (long long)iters);
  if (workgroups < 1 || workgroups > (int64_t(1) << 20))
    return fail(QIFT_ERR_INVALID_ARG, "workgroups=%lld outside [1, 2^20]", (long long)workgroups);
  if (!sink || !clk) return fail(QIFT_ERR_INVALID_ARG, "null buffer");
  if (!aligned(sink, 4) || !aligned(clk, 16))
    return fail(QIFT_ERR_ALIGNMENT, "sink must be 4-byte aligned, clk 16-byte");
  return hip_result(qift::launch_measure_mfma_i8(iters, workgroups, sink, clk,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    "qift_measure_mfma_i8 launch");
}

}  // extern "C"
