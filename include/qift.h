/*
 * qift.h -- C ABI of libqift.so: the rotated W2A4 linear layer and the KV4
 * quantizer on AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "Qift: Shift-Friendly No-Zero W2 Post-Training
 * Quantization for Rotated W2A4/KV4 LLM Inference" (arXiv 2606.02823,
 * abstract): weights and activations are rotated by a Hadamard transform,
 * two-bit weights take a fixed no-zero level set ({+-0.5, +-1.5}, i.e.
 * {+-1, +-3} at half scale, or the power-of-two {+-1, +-4} applied by sign and
 * shift) with one scale per output channel and no zero point; activations and
 * the KV cache are 4-bit.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every buffer argument is a DEVICE pointer owned by the caller. The library
 *   allocates no device memory and keeps no state (the plan of a grouped
 *   launch lives in a caller-owned workspace), except the fixed per-GPU array
 *   of qift_kv4_attention_decode_noalloc; it is safe to call from several
 *   host threads.
 * - Calls are asynchronous: they validate, enqueue on `stream` and return.
 *   Outputs are valid in stream order. `stream` is a hipStream_t passed as
 *   void* (NULL = the null stream).
 * - Arguments are validated before anything is launched. On an error the
 *   call returns a non-zero status, launches nothing and writes nothing;
 *   qift_last_error() then returns a description (per host thread).
 * - Layouts are dense and row-major; no strides.
 * - NaN or Inf inputs give unspecified (but memory-safe) results.
 *
 * Packed layouts
 * --------------
 * int4 (activations xq, KV codes, 4-bit weights): element 2j of a row sits in
 *   the low nibble of byte j, element 2j+1 in the high nibble, two's
 *   complement. Read as little-endian 32-bit words, element i of a word is at
 *   bits 4i..4i+3. Values are in [-7, 7].
 * 2-bit weight codes, in-word layout: the K codes of a channel row form K/16
 *   32-bit words; word j holds features k = 16j..16j+15, feature 16j + i at
 *   bit offset 8*((i>>1)&3) + 4*(i>>3) + 2*(i&1), i.e. byte b holds features
 *   2b, 2b+1, 8+2b, 9+2b in bit pairs 0-1, 2-3, 4-5, 6-7. (This pairs each
 *   code with the nibble order of the int4 activations so that both unpack
 *   to matrix-core operands with shifts and masks only.)
 * 4-bit weight codes, in-word layout: K/8 words per channel row in the int4
 *   order above (feature 8j + i at bits 4i of word j).
 * Weight buffers, tiled layout (chunk-major): channels are grouped in tiles
 *   of 16 and padded with zero codes to Np = ceil(N/16)*16 (T = Np/16 tiles).
 *   With W the words per channel row (K/16 or K/8), the row is cut into
 *   chunks of 16 words (the last one may be shorter: u_c = min(16, W - 16c)
 *   words); word w of channel n, with c = w/16, is stored at index
 *       c * 256*T  +  (n/16) * 16*u_c  +  (16*((w%16)/4) + n%16) * 4  +  w%4
 *   so chunk c of every tile comes before chunk c+1 of any tile, and inside
 *   a chunk each tile holds the 16-byte units that one 64-lane wave loads for
 *   16 channels x 256 features (2-bit) or x 128 features (4-bit): unit
 *   16g + i (channel i, word group g) at byte 16*(16g + i). A weight buffer
 *   holds Np*W words. (A decoder streams chunk c of all tiles together, so
 *   the whole GPU reads one contiguous stretch of memory at a time.)
 * Code values:
 *   QIFT_LEVELS_MNZ : the code read as a 2-bit two's-complement integer t
 *                     gives the half-scale level 2t+1 in {-3,-1,+1,+3};
 *                     weight = (2t+1) * s / 2, i.e. {+-0.5, +-1.5} * s.
 *                     (00 -> +0.5s, 01 -> +1.5s, 10 -> -1.5s, 11 -> -0.5s)
 *   QIFT_LEVELS_POT : bit 1 is the sign, bit 0 the shift by two:
 *                     level = +-(1 << 2*bit0) in {+-1, +-4}; weight = level*s.
 *                     (00 -> +s, 01 -> +4s, 10 -> -s, 11 -> -4s)
 *   QIFT_LEVELS_INT4: 4-bit two's-complement weights in [-7, 7]
 *                     (the 4-bit layers of an L-layer mixed W2/W4 stack).
 *   QIFT_LEVELS_LUT : a level table (the level-set comparisons of the
 *                     abstract: the standard {-2,-1,0,+1} set, a Lloyd-like
 *                     {+-3, +-10}, ...): a uint32 whose byte c is the signed
 *                     integer level L[c] in [-15, 15] of code c (not all
 *                     zero); weight = L[c] * s. {1, 3, -3, -1} decodes MNZ
 *                     codes at step s/2, {1, 4, -1, -4} PoT codes.
 *   QIFT_LEVELS_ASYM: the conventional asymmetric two-bit grid with a zero
 *                     point, the baseline the abstract compares with: the
 *                     code read as an unsigned integer c in {0,1,2,3} and
 *                     the channel's integer zero point z_n in {0,1,2,3} give
 *                     weight = (c - z_n) * s_n. Its scales buffer holds 2N
 *                     values of the scale dtype: s_0 .. s_{N-1}, then
 *                     z_0 .. z_{N-1} (a zero point outside {0,1,2,3} is
 *                     clamped into it, a fractional one truncated).
 *
 * Hadamard rotation
 * -----------------
 * had_block = B, a power of two dividing K: every run of B consecutive
 * features is multiplied by H_B / sqrt(B), H_B the Sylvester Hadamard matrix
 * in natural order (H_1 = [1], H_2n = [[H, H], [H, -H]]). B = 1 is the
 * identity. The same B must be used for a linear's weights and its input.
 */
#ifndef QIFT_H
#define QIFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QIFT_ABI_VERSION 8

typedef enum {
  QIFT_OK = 0,
  QIFT_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad enum value          */
  QIFT_ERR_ALIGNMENT = 2,   /* a buffer is not aligned as documented           */
  QIFT_ERR_UNSUPPORTED = 3, /* valid request outside this library's limits     */
  QIFT_ERR_HIP = 4          /* the HIP runtime reported an error on launch     */
} qift_status;

typedef enum { QIFT_F32 = 0, QIFT_BF16 = 1, QIFT_F16 = 2, QIFT_I32 = 3 } qift_dtype;

typedef enum {
  QIFT_LEVELS_MNZ = 0,  /* {+-0.5, +-1.5} * s, 2-bit codes              */
  QIFT_LEVELS_POT = 1,  /* {+-1, +-4} * s, 2-bit codes, sign-and-shift  */
  QIFT_LEVELS_INT4 = 2, /* [-7, 7] * s, 4-bit codes                     */
  QIFT_LEVELS_LUT = 3,  /* table[code] * s, 2-bit codes (level table)   */
  QIFT_LEVELS_ASYM = 4  /* (c - z_n) * s, 2-bit codes, zero point z_n   */
} qift_levels;

/* Per-channel scale rule of the weight quantizer. */
typedef enum {
  QIFT_SCALE_ABSMAX = 0, /* s = absmax / outer level                        */
  QIFT_SCALE_MSE = 1     /* the best of 64 fractions of it (least squares)  */
} qift_scale_rule;

typedef void* qift_stream; /* a hipStream_t */

/* Largest K accepted by qift_quantize_weights and qift_rotate_quant_act, and
 * largest Hadamard block. */
#define QIFT_MAX_ROW 16384
#define QIFT_MAX_HAD_BLOCK 4096

/*
 * qift_quantize_weights -- offline weight quantizer (Qift abstract: a fixed
 * two-bit code-to-level mapping with the standard per-channel scale, no zero
 * point, applied after the Hadamard rotation).
 *
 * For each row n of W [N, K]: rotate along K in blocks of had_block; take
 * a = max_k |w'| (float32); s_n = a / 1.5 (MNZ), a / 4 (POT) or a / 7 (INT4)
 * in float32, then rounded to scale_dtype (round to nearest even); codes are
 * decided against that stored scale:
 *   MNZ: outer level iff |w'| > s_n; POT: outer iff 2|w'| > 5 s_n (exact);
 *        sign from w' < 0 (so -0 and ties go to the positive/inner level);
 *   INT4: q = clamp(rint(w' / s_n), -7, 7), IEEE float32 division.
 * A row with s_n == 0 gets code 0 (MNZ/POT: +inner) or q = 0 everywhere.
 *
 *   W       [N, K] float32 (QIFT_F32) or bfloat16 (QIFT_BF16)
 *   K       multiple of 64, K <= QIFT_MAX_ROW; had_block | K
 *   codes   out: Np*K/16 uint32 (MNZ, POT) or Np*K/8 uint32 (INT4), tiled
 *           layout, Np = ceil(N/16)*16 (padding channels are written as 0);
 *           16-byte aligned
 *   scales  out: [N] float32 (QIFT_F32) or float16 (QIFT_F16); [2N] for
 *           QIFT_LEVELS_ASYM (the steps, then the zero points)
 * N = 0 is a no-op.
 */
qift_status qift_quantize_weights(const void* W, qift_dtype w_dtype, int64_t N, int64_t K,
                                  int32_t had_block, qift_levels levels, uint32_t* codes,
                                  void* scales, qift_dtype scale_dtype, qift_stream stream);

/*
 * qift_quantize_weights_ex -- qift_quantize_weights with a level table and a
 * scale rule (Qift abstract: the inner/outer ratio analysis, the standard
 * two-bit set as the baseline, and a scale-invariant comparison of level
 * sets, i.e. each set at its best scale).
 *
 *   levels       any qift_levels value; QIFT_LEVELS_LUT uses level_table
 *   level_table  QIFT_LEVELS_LUT: byte c = L[c] (signed, |L| <= 15, not all
 *                zero); must be 0 for the other levels
 *   scale_rule   QIFT_SCALE_ABSMAX: s = absmax / outer, outer = 1.5 (MNZ),
 *                4 (POT), 7 (INT4), max |L| (LUT), as qift_quantize_weights.
 *                QIFT_SCALE_MSE: the candidates
 *                  s_j = store(fl32(fl32(absmax / outer) * (64 - j) / 64)),
 *                j = 0..63 (store = rounding to scale_dtype), are each tried
 *                with codes decided against s_j, and the one with the
 *                smallest sum over the row of (w' - level * s_j)^2 (float64
 *                sums) is kept, the largest on ties (up to the order of the
 *                float64 sum, which may decide between candidates whose errors
 *                differ in the last bits).
 * LUT codes: the level nearest to w' (distances |w' - L[c] * s| in float64),
 * ties to the smaller |L[c]|, then the non-negative level, then the lower
 * code.
 * QIFT_LEVELS_ASYM (the min-max grid; scale_rule must be QIFT_SCALE_ABSMAX,
 * else QIFT_ERR_INVALID_ARG): over the rotated float32 row,
 *   lo = min(min w', 0), hi = max(max w', 0), s = fl32(fl32(hi - lo) / 3)
 *   rounded to scale_dtype, z = clamp(rint(fl32(-lo / s)), 0, 3),
 *   c = clamp(rint(fl32(w' / s)) + z, 0, 3)
 * (IEEE float32 division, round half to even, the stored s); s = 0 gives
 * z = 0 and c = 0. scales receives s_n at n and z_n at N + n.
 * Other arguments, layouts and errors as qift_quantize_weights.
 */
qift_status qift_quantize_weights_ex(const void* W, qift_dtype w_dtype, int64_t N, int64_t K,
                                     int32_t had_block, qift_levels levels, uint32_t level_table,
                                     qift_scale_rule scale_rule, uint32_t* codes, void* scales,
                                     qift_dtype scale_dtype, qift_stream stream);

/*
 * qift_rotate_quant_act -- online activation path (Qift abstract: rotated
 * W2A4 inference, 4-bit activations): rotate each token along K in blocks of
 * had_block (float32 butterflies), then per token
 *   s_a = max_k |x'| / 7 (IEEE float32), q = clamp(rint(x' / s_a), -7, 7)
 * (round half to even, IEEE division; the clamp binds only when s_a is
 * subnormal, whose rounding can put |x' / s_a| above 7.5). A token whose s_a
 * is 0 gets q = 0: an all-zero token, or one whose max |x'| is at most
 * 3 * 2^-149, so that max |x'| / 7 rounds to 0.
 *
 *   X      [M, K] float32 (QIFT_F32) or bfloat16 (QIFT_BF16)
 *   K      even, K <= QIFT_MAX_ROW; had_block | K
 *   xq     out: [M, K/2] int4 pairs (layout above)
 *   s_a    out: [M] float32
 *   x_rot  out, optional (may be NULL): [M, K] float32 rotated activations
 *          (a value that is exactly zero is written as +0)
 * M = 0 is a no-op.
 */
qift_status qift_rotate_quant_act(const void* X, qift_dtype x_dtype, int64_t M, int64_t K,
                                  int32_t had_block, uint8_t* xq, float* s_a, float* x_rot,
                                  qift_stream stream);

/*
 * qift_rotate_quant_act_batched -- qift_rotate_quant_act on up to
 * QIFT_MAX_ROTATE_BATCH independent activation matrices in one call (the
 * same online activation path; meant for the inputs of all linears of a
 * decode step, a few token rows each, which cannot fill the GPU one by one).
 * Each descriptor has the meaning, limits and results of the arguments of
 * qift_rotate_quant_act (the shared launch sums every butterfly stage in
 * float32 registers, where qift_rotate_quant_act sums the first five stages
 * of bfloat16 rows with blocks of 256 or more on the matrix cores: the two
 * agree bit for bit whenever those 32-element sums are exact in float32,
 * and otherwise differ by float32 rounding in the rotated values, within the
 * rotation's tolerance, and in a code only where such a difference meets a
 * rounding near-tie); every descriptor is validated before anything is
 * launched. Descriptors with K % 16 == 0, had_block >= 16 and 16-byte aligned
 * X, xq (and x_rot if given) share one launch with one workgroup per row; any
 * other descriptor gets a launch of its own. Outputs of different
 * descriptors must not overlap.
 *
 *   descs  HOST array of count descriptors, read during the call only
 *   count  0 .. QIFT_MAX_ROTATE_BATCH (0 is a no-op)
 */
#define QIFT_MAX_ROTATE_BATCH 8
typedef struct {
  const void* X;      /* [M, K] float32 or bfloat16 */
  qift_dtype x_dtype; /* QIFT_F32 or QIFT_BF16 */
  int32_t had_block;
  int64_t M;
  int64_t K;
  uint8_t* xq;        /* out: [M, K/2] int4 pairs */
  float* s_a;         /* out: [M] */
  float* x_rot;       /* out, optional: [M, K] float32 */
} qift_rotate_desc;

qift_status qift_rotate_quant_act_batched(const qift_rotate_desc* descs, int32_t count,
                                          qift_stream stream);

/*
 * qift_w2a4_linear -- the linear layer with decoded two-bit weights (Qift
 * abstract: the power-of-two set is applied by sign and shift, the main set
 * in its half-scale integer form):
 *   acc[m, n] = sum_k q[m, k] * level[n, k]            (exact, int32)
 *   Y[m, n]   = acc[m, n] * s_a[m] * s_w[n] * kappa    (float32)
 * with level the integer level of the code (half-scale for MNZ) and
 * kappa = 1/2 for MNZ, 1 for POT and INT4. y_dtype QIFT_I32 stores acc itself.
 * (QIFT_LEVELS_ASYM, through qift_w2a4_linear_ex: level = c - z_n and
 * kappa = 1, i.e. acc = sum q c - z_n sum q; scales holds the 2N steps and
 * zero points.)
 * M <= 16 runs the weight-streaming decode kernel, M > 16 the matrix-core
 * prefill kernel; both give identical results.
 *
 *   xq, s_a   [M, K/2] int4, [M] float32 (as written by qift_rotate_quant_act)
 *   K         multiple of 64, K <= 65536
 *   codes     Np*K/16 (2-bit) or Np*K/8 (INT4) uint32 in the tiled layout
 *             written by qift_quantize_weights; 16-byte aligned
 *   scales    [N] float32 or float16 (scale_dtype); [2N] for QIFT_LEVELS_ASYM
 *   Y         out: [M, N] float32, bfloat16 or int32 (y_dtype)
 *   xq must be 16-byte aligned.
 * M = 0 or N = 0 is a no-op.
 */
qift_status qift_w2a4_linear(const uint8_t* xq, const float* s_a, int64_t M, int64_t K,
                             const uint32_t* codes, const void* scales, qift_dtype scale_dtype,
                             qift_levels levels, int64_t N, void* Y, qift_dtype y_dtype,
                             qift_stream stream);

/*
 * qift_w2a4_linear_ex -- qift_w2a4_linear for any qift_levels value,
 * including a level table (the level-set comparisons of the Qift abstract run
 * through the same decoded linear): with QIFT_LEVELS_LUT,
 *   acc[m, n] = sum_k q[m, k] * L[code[n, k]]   (exact, int32)
 *   Y[m, n]   = acc[m, n] * s_a[m] * s_w[n]
 * level_table as in qift_quantize_weights_ex (0 for the other levels). K is
 * limited to 65536 as for the other levels (|sum| <= 7 * 15 * 65536).
 */
qift_status qift_w2a4_linear_ex(const uint8_t* xq, const float* s_a, int64_t M, int64_t K,
                                const uint32_t* codes, const void* scales, qift_dtype scale_dtype,
                                qift_levels levels, uint32_t level_table, int64_t N, void* Y,
                                qift_dtype y_dtype, qift_stream stream);

/*
 * qift_rotate_w2a4_linear -- the online activation path and the linear in
 * one call (Qift abstract: rotated W2A4 inference), for a layer whose input
 * is not yet quantized: exactly qift_rotate_quant_act(X, x_dtype, M, K,
 * had_block, xq, s_a, NULL) followed by qift_w2a4_linear_ex(xq, s_a, M, K,
 * codes, scales, scale_dtype, levels, level_table, N, Y, y_dtype), with the
 * same results (xq and s_a are written too). A single token row (M = 1) with
 * K % 16 == 0, had_block >= 16 and 16-byte aligned X and xq runs as one
 * launch in which every workgroup rotates and quantizes the row itself while
 * its weights stream in (summing every butterfly stage in float32 registers:
 * for a bfloat16 row with a block of 256 or more, which qift_rotate_quant_act
 * rotates partly on the matrix cores, the results agree bit for bit whenever
 * the 32-element sums of the first five stages are exact in float32, and
 * otherwise may differ in a code only where a float32 rounding difference
 * meets a rounding near-tie); other calls run the two launches.
 *   X, x_dtype, had_block, xq, s_a  as qift_rotate_quant_act (x_rot omitted)
 *   the rest                        as qift_w2a4_linear_ex
 * K must satisfy both calls' limits (a multiple of 64, at most
 * QIFT_MAX_ROW). Errors as either call; M = 0 is a no-op, and N = 0 only
 * writes xq and s_a.
 */
qift_status qift_rotate_w2a4_linear(const void* X, qift_dtype x_dtype, int64_t M, int64_t K,
                                    int32_t had_block, uint8_t* xq, float* s_a,
                                    const uint32_t* codes, const void* scales,
                                    qift_dtype scale_dtype, qift_levels levels,
                                    uint32_t level_table, int64_t N, void* Y, qift_dtype y_dtype,
                                    qift_stream stream);

/*
 * qift_kv4_quant -- KV4 (Qift abstract: rotated W2A4/KV4 inference): each
 * head vector KV[t, h, :] is rotated in blocks of had_block along D, then
 * quantized to int4 with its own scale s = max|v'| / 7, exactly as the
 * activation path.
 *
 *   KV      [T, H, D] bfloat16 or float32; D in {16, 32, 64, 128, 256};
 *           had_block | D
 *   kvq     out: [T, H, D/2] int4 pairs
 *   scales  out: [T, H] float32
 * T*H = 0 is a no-op.
 */
qift_status qift_kv4_quant(const void* KV, qift_dtype dtype, int64_t T, int64_t H, int64_t D,
                           int32_t had_block, uint8_t* kvq, float* scales, qift_stream stream);

/*
 * qift_kv4_quant_kv -- qift_kv4_quant on the K and V caches of one layer in
 * one call (the KV4 of rotated W2A4/KV4 inference, Qift abstract): K and V
 * are quantized exactly as two qift_kv4_quant calls would, with the same
 * results. On the matrix-core path (bfloat16, D = 64, 128 or 256,
 * had_block >= 32) both tensors share one launch, which pays the ramp at the
 * start and the tail at the end of a launch once instead of twice; other
 * shapes run two launches.
 *
 *   K, V      [T, H, D], both of dtype (bfloat16 or float32), 16-byte aligned
 *   kq, vq    out: [T, H, D/2] int4 pairs of K and of V, 16-byte aligned
 *   ks, vs    out: [T, H] float32 scales of K and of V
 * Limits and errors as qift_kv4_quant; in addition kq and vq must not
 * overlap, nor ks and vs (QIFT_ERR_INVALID_ARG), and no output may overlap
 * K or V (not checked). T*H = 0 is a no-op.
 */
qift_status qift_kv4_quant_kv(const void* K, const void* V, qift_dtype dtype, int64_t T,
                              int64_t H, int64_t D, int32_t had_block, uint8_t* kq, float* ks,
                              uint8_t* vq, float* vs, qift_stream stream);

/*
 * qift_kv4_attention_decode -- decode attention over a KV4 cache (the
 * consumer of the 4-bit KV cache of rotated W2A4/KV4 inference, Qift
 * abstract). The cache holds every head vector rotated by H_B / sqrt(B) and
 * quantized (qift_kv4_quant); the query is rotated by the same orthogonal
 * map, so for each sequence s and head h
 *   score[t] = softmax_scale * sum_d q'[s,h,d] * kcode[s,t,h,d] * ks[s,t,h]
 *   p        = softmax over t = 0 .. T-1 of score
 *   o'[d]    = sum_t p[t] * vcode[s,t,h,d] * vs[s,t,h]
 *   out[s,h] = o' rotated back by H_B / sqrt(B)
 * in float32, q' = q rotated in blocks of had_block along D.
 *
 *   q          [S, H, D] float32 or bfloat16 (one query token per sequence)
 *   kq, vq     [S, T, H, D/2] int4 pairs (per sequence, the layout
 *              qift_kv4_quant writes for [T, H, D]); 16-byte aligned
 *   ks, vs     [S, T, H] float32
 *   had_block  the block the cache was rotated with (power of two, divides D)
 *   out        [S, H, D] float32 or bfloat16
 *   workspace  device memory of at least the size that
 *              qift_kv4_attention_workspace_bytes returns, 256-byte aligned,
 *              caller-owned; it holds partial results during the call
 * Limits: D = 128, 1 <= H <= 64, T >= 1, S <= 65535 (outside them:
 * QIFT_ERR_UNSUPPORTED). S = 0 is a no-op.
 */
qift_status qift_kv4_attention_workspace_bytes(int64_t S, int64_t T, int64_t H, int64_t D,
                                               size_t* bytes);
qift_status qift_kv4_attention_decode(const void* q, qift_dtype q_dtype, int64_t S, int64_t T,
                                      int64_t H, int64_t D, int32_t had_block,
                                      const uint8_t* kq, const float* ks, const uint8_t* vq,
                                      const float* vs, float softmax_scale, void* out,
                                      qift_dtype out_dtype, void* workspace,
                                      size_t workspace_bytes, qift_stream stream);

/*
 * qift_kv4_attention_decode_noalloc -- qift_kv4_attention_decode for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): no workspace argument,
 * and the call allocates nothing. Its partial results go to a fixed array of
 * QIFT_ATTENTION_SCRATCH_BYTES in device memory, one per GPU, which the
 * library holds from its first use on that GPU until the process ends; the
 * array used is the current device's (the device of `stream` and of every
 * buffer must be current). A call whose partial results need more
 * (qift_kv4_attention_workspace_bytes above QIFT_ATTENTION_SCRATCH_BYTES,
 * e.g. S * H beyond about 32000 (sequence, head) pairs) returns
 * QIFT_ERR_UNSUPPORTED without launching. Every call on one GPU shares that
 * GPU's array: calls ordered on one stream are safe, calls that overlap on
 * one GPU (other streams, or host threads without ordering) race and give
 * undefined results. Arguments, limits, results and errors otherwise as
 * qift_kv4_attention_decode, whose kernels it runs.
 */
#define QIFT_ATTENTION_SCRATCH_BYTES (16u * 1024u * 1024u)
qift_status qift_kv4_attention_decode_noalloc(const void* q, qift_dtype q_dtype, int64_t S,
                                              int64_t T, int64_t H, int64_t D, int32_t had_block,
                                              const uint8_t* kq, const float* ks,
                                              const uint8_t* vq, const float* vs,
                                              float softmax_scale, void* out,
                                              qift_dtype out_dtype, qift_stream stream);

/*
 * Error-compensated weight quantization with the fixed levels (GPTQ's
 * column-by-column quantization, in which quantizing one column updates the
 * columns after it: QTEA abstract; the Qift abstract reports the "GPTQ
 * residual behavior" of its level sets). Offline, two calls:
 *
 * qift_gptq_hessian -- H (+)= X'^T X' for calibration activations X [S, K]
 * (float32 or bfloat16), X' = X rotated along K in blocks of had_block
 * (float64 butterflies), products and sums in float64 on the matrix cores.
 * accumulate = 0 writes H, 1 adds to it (H summed over calibration batches).
 *   H          [K, K] float64, symmetric (both triangles written), 8-byte aligned
 *   workspace  device memory of qift_gptq_hessian_workspace_bytes(S, K)
 *              bytes, 256-byte aligned, caller-owned (the rotated activations
 *              of up to 4096 tokens at a time)
 * Limits as qift_quantize_weights for K and had_block; S >= 0 (S = 0 with
 * accumulate = 0 writes H = 0).
 *
 * qift_gptq_quantize_weights -- codes and scales of W [N, K] in the layout of
 * qift_quantize_weights_ex (same levels except QIFT_LEVELS_ASYM, which is
 * QIFT_ERR_INVALID_ARG here; same level_table, scale_rule, scale_dtype and
 * limits; the result feeds qift_w2a4_linear unchanged):
 *   1. W' = W rotated (float64 butterflies), rounded to float32;
 *   2. s_n by scale_rule from the rows of W' (the plain quantizer's scales);
 *   3. a feature k with H[k][k] = 0 gets H[k][k] = 1 and weight 0; then
 *      damp * mean(diag H) is added to every diagonal entry;
 *   4. U, upper triangular with U^T U = H^-1 (float64);
 *   5. for k = 0 .. K-1 in order, per channel n: the code of the current
 *      weight w[n][k] rounded to float32, decided against the stored s_n as
 *      in qift_quantize_weights_ex; e = (w[n][k] - level * s_n) / U[k][k];
 *      w[n][j] -= e * U[k][j] for every j > k (float64).
 *   H          [K, K] float64 from qift_gptq_hessian (or any symmetric
 *              positive semi-definite matrix); read only
 *   damp       > 0 and finite (0.01 is customary)
 *   workspace  qift_gptq_workspace_bytes(N, K) bytes of device memory,
 *              256-byte aligned, caller-owned (float64 copies of W' and two
 *              K x K matrices: 2.1 GB for N = 11008, K = 4096)
 * The updates are blocked (64 features at a time) so their float64 rounding
 * differs from the unblocked order; a code can then differ only where a
 * weight lies within that rounding of a decision boundary. N = 0 is a no-op;
 * N * K / 64 above 2^31 - 1 is QIFT_ERR_UNSUPPORTED. H must be positive
 * definite after the damping (true for X'^T X' with damp > 0); otherwise
 * the codes are undefined.
 */
qift_status qift_gptq_hessian_workspace_bytes(int64_t S, int64_t K, size_t* bytes);
qift_status qift_gptq_hessian(const void* X, qift_dtype x_dtype, int64_t S, int64_t K,
                              int32_t had_block, int32_t accumulate, double* H, void* workspace,
                              size_t workspace_bytes, qift_stream stream);
qift_status qift_gptq_workspace_bytes(int64_t N, int64_t K, size_t* bytes);
qift_status qift_gptq_quantize_weights(const void* W, qift_dtype w_dtype, int64_t N, int64_t K,
                                       const double* H, int32_t had_block, qift_levels levels,
                                       uint32_t level_table, qift_scale_rule scale_rule,
                                       double damp, uint32_t* codes, void* scales,
                                       qift_dtype scale_dtype, void* workspace,
                                       size_t workspace_bytes, qift_stream stream);

/*
 * Grouped linear: many independent W2A4 linears (for example every linear of
 * a decoder stack) in one launch. Each descriptor is one qift_w2a4_linear
 * call with M <= 16; levels may differ between descriptors.
 *
 * 1. qift_linear_group_workspace_bytes(descs, count, &bytes) gives the size
 *    of the device workspace the plan needs (it checks each descriptor by
 *    the rules that do not depend on the scale and output dtypes; prepare
 *    checks those too).
 * 2. qift_linear_group_prepare validates every descriptor (same rules as
 *    qift_w2a4_linear), builds the plan on the host and copies it into
 *    `workspace` (device memory, 256-byte aligned, caller-owned) on `stream`,
 *    then waits for that copy; the host array may be freed afterwards. It
 *    writes to *launch_tiles the number of workgroup tiles of the plan.
 *    Linears with larger K come first in the plan, so that the longest tiles
 *    are dispatched first.
 * 3. qift_w2a4_linear_grouped(workspace, launch_tiles, stream) runs every
 *    linear of the plan; launch_tiles must be the value prepare returned.
 *    The plan stays valid while the buffers it names stay allocated; their
 *    contents may change between runs.
 */
typedef struct qift_linear_desc {
  const uint8_t* xq;      /* [M, K/2] int4                         */
  const float* s_a;       /* [M] float32                           */
  const uint32_t* codes;  /* tiled, Np*K/16 or Np*K/8 uint32       */
  const void* scales;     /* [N], dtype given to prepare           */
  void* Y;                /* [M, N], dtype given to prepare        */
  int64_t M, K, N;
  int32_t levels;         /* a qift_levels value                   */
  int32_t reserved;       /* QIFT_LEVELS_LUT: the level table;     */
                          /* other levels: must be 0               */
} qift_linear_desc;

qift_status qift_linear_group_workspace_bytes(const qift_linear_desc* descs, int32_t count,
                                              size_t* bytes);
qift_status qift_linear_group_prepare(const qift_linear_desc* descs, int32_t count,
                                      qift_dtype scale_dtype, qift_dtype y_dtype,
                                      void* workspace, size_t workspace_bytes,
                                      int64_t* launch_tiles, qift_stream stream);
qift_status qift_w2a4_linear_grouped(const void* workspace, int64_t launch_tiles,
                                     qift_stream stream);

/* Human-readable name of a status, and the detail of this thread's last
 * error (empty string if none). Both return static or thread-local storage. */
const char* qift_status_string(qift_status s);
const char* qift_last_error(void);
int32_t qift_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QIFT_H */
