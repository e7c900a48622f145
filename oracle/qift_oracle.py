"""Plain CPU oracle for the rotated W2A4 linear and the KV4 quantizer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. It shares no code with the HIP path (its own
Hadamard matrix, its own packers, dense matmuls instead of butterflies) and is
deliberately slow and literal. Arithmetic is float64 except where a floating
point value decides an integer (a code, a rounding): there both sides take the
decision in float32, the precision of the kernels.

What the method computes comes from one source, the abstract of
"Qift: Shift-Friendly No-Zero W2 Post-Training Quantization for Rotated
W2A4/KV4 LLM Inference" (arXiv 2606.02823, abstract page). The abstract fixes:

* weights and activations pass through a Hadamard rotation before scalar
  quantization;
* the main two-bit level set is {+-0.5, +-1.5} (half-scale {+-1, +-3}); a
  power-of-two variant uses {+-1, +-4}, applied by sign and shift;
* one per-output-channel scale, no zero point, no groups, no learned codebook;
* activations are 4-bit ("W2A4") and so is the KV cache ("KV4");
* an inner/outer level ratio between 0.25 and 0.33 works well, {+-1, +-2}
  does not; the standard two-bit set is {-2, -1, 0, +1}.

It leaves open, and this oracle takes the plainest reading of:

* Hadamard kind: Sylvester order, normalized by 1/sqrt(B) per block of B;
* activation granularity: per token, symmetric, codes in [-7, 7], round half
  to even, s_a = absmax / 7;
* weight scale rule: s_n = absmax_n / 1.5 (MNZ), absmax_n / 4 (PoT),
  absmax_n / 7 (4-bit layers of a mixed stack), rounded to the stored scale
  dtype; codes are decided against the stored scale;
* nearest level by exhaustive comparison; ties go to the inner level and a
  zero weight goes to the positive inner level;
* code bits: for MNZ the 2-bit code read as a two's-complement integer t gives
  the half-scale level 2t+1; for PoT bit 1 is the sign and bit 0 selects the
  shift by two (level +-(1 << 2*bit0));
* packing layouts (the ``pack*`` functions below).

Level tables and the searched scale (the abstract compares level sets: the
no-zero sets against the standard {-2, -1, 0, +1} set, the Lloyd-optimal
inner/outer ratio near 0.30, and a scale-invariant analysis, i.e. each set at
its best scale). Readings taken here:

* a level table is four integers L[c] in [-15, 15], one per 2-bit code, and
  the weight of code c is L[c] * s (so {1, 3, -3, -1} decodes MNZ codes and
  {1, 4, -1, -4} PoT codes, with s the step);
* nearest level as above, ties to the smaller |L|, then to the positive level,
  then to the lower code;
* the absmax scale rule divides by max |L|; the searched ("mse") rule tries
  the 64 stored scales s_j = store(fl32(fl32(absmax / outer) * (64 - j) / 64)),
  j = 0..63, codes decided against each, and keeps the one with the smallest
  sum of squared errors (float64; the first on ties).

The conventional asymmetric two-bit grid with a zero point (the Qift abstract
names it as the baseline that improves on the standard set and whose zero
point Qift removes; it gives no formula). Readings taken here, the usual
min-max uniform quantizer:

* per channel, a 4-point uniform grid s * (c - z), c in {0, 1, 2, 3}, with an
  integer zero point z;
* the range of the rotated float32 row is widened to contain 0:
  lo = min(min w, 0), hi = max(max w, 0); s = fl32(fl32(hi - lo) / 3),
  rounded to the stored scale dtype; z = clip(rint(fl32(-lo / s)), 0, 3);
* c = clip(rint(fl32(w / s)) + z, 0, 3), round half to even in float32;
  s = 0 (an all-zero row, or a step below the stored dtype's range) gives
  z = 0 and c = 0;
* s and z are stored side by side: the 2N scale entries hold s_0..s_{N-1}
  then z_0..z_{N-1} (z as a value of the scale dtype, exact).

Error-compensated quantization with the fixed levels (the Qift abstract
reports the "GPTQ residual behavior" of its level sets; the QTEA abstract
describes GPTQ-style column-by-column quantization, in which quantizing one
column updates the ones after it; the algorithm itself is GPTQ's, restated
here). Readings taken here:

* H = X'^T X' from the calibration activations rotated like the weights (no
  1/S or factor 2: a common factor of H changes nothing below); dead
  features (H[k, k] = 0) get H[k, k] = 1 and weight 0; then
  damp * mean(diag H) is added to the diagonal (damp = 0.01 by default);
* the scales are fixed before the loop, by the plain quantizer's rule on the
  rotated weights; features in natural order (no reordering by H);
* each decision is the plain quantizer's on the current weight rounded to
  float32; updates in float64.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, brute force and the values the abstract prints. The
end-to-end accuracy of a quantized linear against the unquantized one has no
value on the pages: parity unpinned (reported, not asserted).
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# level sets (Qift abstract: the main set, its half-scale form, the PoT variant)
# ---------------------------------------------------------------------------

#: per level kind: integer level for each 2-bit code, the factor kappa that
#: turns the integer level into a multiple of the scale, and the divisor of
#: the absmax scale rule (the outer real level).
LEVEL_KINDS = {
    # code t (two's complement 2-bit) -> half-scale level 2t+1; real = level/2
    "mnz": {"code_to_int": (1, 3, -3, -1), "kappa": 0.5, "outer": 1.5},
    # bit1 = sign, bit0 = shift by two: +1, +4, -1, -4
    "pot": {"code_to_int": (1, 4, -1, -4), "kappa": 1.0, "outer": 4.0},
    # 4-bit symmetric per-channel weights of the W4 layers of a mixed stack
    "int4": {"code_to_int": None, "kappa": 1.0, "outer": 7.0},
}

#: preference order of codes for the nearest-level rule: inner before outer,
#: positive before negative
_PREFERENCE = {"mnz": (0, 3, 1, 2), "pot": (0, 2, 1, 3)}


def real_levels(kind: str) -> np.ndarray:
    """Real levels (multiples of the scale s) indexed by 2-bit code."""
    info = LEVEL_KINDS[kind]
    return np.array(info["code_to_int"], dtype=np.float64) * info["kappa"]


#: largest |level| of a level table
LUT_MAX_LEVEL = 15


def check_table(table) -> tuple:
    """A level table: four integers in [-15, 15], not all zero."""
    t = tuple(int(v) for v in table)
    if len(t) != 4 or any(abs(v) > LUT_MAX_LEVEL for v in t) or all(v == 0 for v in t):
        raise ValueError(f"bad level table {table!r}")
    return t


def table_preference(table) -> tuple:
    """Codes in tie-break order: smaller |level| first, then positive (and
    zero) before negative, then the lower code."""
    t = check_table(table)
    return tuple(sorted(range(4), key=lambda c: (abs(t[c]), t[c] < 0, c)))


def _kind_levels(kind: str, table=None):
    """(real level by code, tie-break order, outer level) of a 2-bit kind."""
    if kind == "lut":
        t = check_table(table)
        return np.array(t, dtype=np.float64), table_preference(t), float(max(abs(v) for v in t))
    return real_levels(kind), _PREFERENCE[kind], LEVEL_KINDS[kind]["outer"]


# ---------------------------------------------------------------------------
# Hadamard rotation
# ---------------------------------------------------------------------------

def hadamard(B: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_B (int64), H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]], built by Kronecker products."""
    if B < 1 or (B & (B - 1)) != 0:
        raise ValueError("Hadamard block must be a power of two")
    H = np.ones((1, 1), dtype=np.int64)
    base = np.array([[1, 1], [1, -1]], dtype=np.int64)
    while H.shape[0] < B:
        H = np.kron(base, H)
    return H


def rotate(x: np.ndarray, B: int) -> np.ndarray:
    """Block-diagonal rotation along the last axis: each run of B consecutive
    features is multiplied by H_B / sqrt(B). float64, dense matmul."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % B != 0:
        raise ValueError("block must divide K")
    Q = hadamard(B).astype(np.float64) / math.sqrt(B)
    lead = x.shape[:-1]
    xb = x.reshape(-1, K // B, B)
    return (xb @ Q).reshape(*lead, K)


# ---------------------------------------------------------------------------
# per-token symmetric 4-bit quantization (A4 and KV4)
# ---------------------------------------------------------------------------

def quant_sym4(xr32: np.ndarray):
    """Per row: s = float32(absmax) / float32(7); q = clip(rint(x / s), -7, 7)
    with float32 IEEE division and round half to even. A row whose scale is 0
    gets q = 0: an all-zero row, and also a row whose absmax is at most
    3 * 2^-149, for which absmax / 7 rounds to 0 (the zero-scale rule is
    about the scale, not only about all-zero input).
    Returns (q int8 [R, K], s float32 [R])."""
    xr32 = np.asarray(xr32, dtype=np.float32)
    R, K = xr32.shape
    q = np.zeros((R, K), dtype=np.int8)
    s = np.zeros(R, dtype=np.float32)
    for r in range(R):
        a = np.float32(np.max(np.abs(xr32[r]))) if K > 0 else np.float32(0)
        sr = np.float32(a) / np.float32(7.0)
        if sr == 0:
            continue
        s[r] = sr
        q[r] = np.clip(np.rint(xr32[r] / sr), -7, 7).astype(np.int8)
    return q, s


def rotate_quant_act(X: np.ndarray, B: int):
    """Online activation path: rotate along K in blocks of B (float64), round
    the rotated values to float32, then quantize per token to int4.
    Returns (q int8 [M, K], s_a float32 [M], x_rot float32 [M, K],
    x_rot64 float64 [M, K])."""
    xr64 = rotate(X, B)
    xr32 = xr64.astype(np.float32)
    q, s = quant_sym4(xr32)
    return q, s, xr32, xr64


# ---------------------------------------------------------------------------
# offline weight quantization
# ---------------------------------------------------------------------------

def _store_scale(s32: np.ndarray, scale_dtype: str) -> np.ndarray:
    if scale_dtype == "f32":
        return s32.astype(np.float32)
    if scale_dtype == "f16":
        return s32.astype(np.float16)
    raise ValueError(scale_dtype)


def _outer(kind: str, table=None) -> float:
    return LEVEL_KINDS["int4"]["outer"] if kind == "int4" else _kind_levels(kind, table)[2]


def absmax_scales(wr32: np.ndarray, kind: str, scale_dtype: str, table=None) -> np.ndarray:
    """s_n = float32(absmax_n) / float32(outer level), rounded to the stored
    dtype (float16 round-to-nearest-even, or float32)."""
    a = np.max(np.abs(wr32.astype(np.float32)), axis=1).astype(np.float32)
    s32 = a / np.float32(_outer(kind, table))
    return _store_scale(s32.astype(np.float32), scale_dtype)


#: candidates of the searched scale: factors (64 - j) / 64 of the absmax scale
MSE_GRID = 64


def scale_candidates(wr32: np.ndarray, kind: str, scale_dtype: str, table=None) -> np.ndarray:
    """[N, 64] stored candidate scales s_j = store(fl32(fl32(absmax / outer)
    * (64 - j) / 64)), j = 0..63 (the factors are exact in float32)."""
    a = np.max(np.abs(wr32.astype(np.float32)), axis=1).astype(np.float32)
    base = (a / np.float32(_outer(kind, table))).astype(np.float32)
    f = ((MSE_GRID - np.arange(MSE_GRID)) / MSE_GRID).astype(np.float32)
    s32 = (base[:, None] * f[None, :]).astype(np.float32)
    return _store_scale(s32, scale_dtype)


def row_sq_error(w32: np.ndarray, s, kind: str, table=None) -> float:
    """Sum over the row of (w - level(code) * s)^2 in float64, the codes
    decided against the stored scale s."""
    w32 = np.asarray(w32, dtype=np.float32)[None, :]
    sv = np.asarray([s])
    if kind == "int4":
        lv = int4_weight_codes(w32, sv).astype(np.float64)
    else:
        codes = nearest_codes(w32, sv, kind, table)
        lv = _kind_levels(kind, table)[0][codes]
    d = w32.astype(np.float64) - lv * float(np.float64(sv[0]))
    return float(np.sum(d * d))


def weight_scales(wr32: np.ndarray, kind: str, scale_dtype: str, table=None,
                  rule: str = "absmax") -> np.ndarray:
    """Per-channel stored scales by the absmax rule, or by the searched rule:
    the candidate of scale_candidates with the smallest row_sq_error (the
    first one on ties)."""
    if rule == "absmax":
        return absmax_scales(wr32, kind, scale_dtype, table)
    if rule != "mse":
        raise ValueError(rule)
    cand = scale_candidates(wr32, kind, scale_dtype, table)
    out = cand[:, 0].copy()
    for n in range(wr32.shape[0]):
        errs = [row_sq_error(wr32[n], cand[n, j], kind, table) for j in range(MSE_GRID)]
        out[n] = cand[n, int(np.argmin(errs))]
    return out


def nearest_codes(wr32: np.ndarray, s_stored: np.ndarray, kind: str, table=None) -> np.ndarray:
    """2-bit code of each weight: the code whose level * s is closest to w,
    found by comparing all four distances (float64, exact for float32 w and a
    float16/float32 s). Ties go to the earlier code in the preference order
    (inner before outer, positive before negative)."""
    w = wr32.astype(np.float32).astype(np.float64)
    s = s_stored.astype(np.float64)[:, None]
    lv, order, _ = _kind_levels(kind, table)
    d = np.stack([np.abs(w - lv[c] * s) for c in order], axis=0)
    pick = np.argmin(d, axis=0)  # first minimum = preferred code on ties
    return np.asarray(order, dtype=np.int64)[pick]


def int4_weight_codes(wr32: np.ndarray, s_stored: np.ndarray) -> np.ndarray:
    """4-bit symmetric weight codes q = clip(rint(w / s), -7, 7) in float32
    with the stored scale; s = 0 gives q = 0."""
    w = wr32.astype(np.float32)
    s = s_stored.astype(np.float32)
    q = np.zeros(w.shape, dtype=np.int64)
    for n in range(w.shape[0]):
        if s[n] == 0:
            continue
        q[n] = np.clip(np.rint(w[n] / s[n]), -7, 7).astype(np.int64)
    return q


def asym_minmax_params(wr32: np.ndarray, scale_dtype: str):
    """Step and zero point of the asymmetric min-max grid, per channel:
    lo = min(min w, 0), hi = max(max w, 0) over the float32 row,
    s = store(fl32(fl32(hi - lo) / 3)), z = clip(rint(fl32(-lo / s)), 0, 3)
    (z = 0 where s = 0). Returns (s [N] stored dtype, z [N] int64)."""
    w = np.asarray(wr32, dtype=np.float32)
    lo = np.minimum(w.min(axis=1), np.float32(0)).astype(np.float32)
    hi = np.maximum(w.max(axis=1), np.float32(0)).astype(np.float32)
    rng = (hi - lo).astype(np.float32)
    s = _store_scale((rng / np.float32(3)).astype(np.float32), scale_dtype)
    z = np.zeros(w.shape[0], dtype=np.int64)
    for n in range(w.shape[0]):
        sn = np.float32(s[n])
        if sn == 0:
            continue
        z[n] = int(np.clip(np.rint(np.float32(-lo[n]) / sn), 0, 3))
    return s, z


def asym_codes(wr32: np.ndarray, s_stored: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Codes of the asymmetric grid: c = clip(rint(fl32(w / s)) + z, 0, 3),
    decided in float32 with the stored step; 0 where s = 0."""
    w = np.asarray(wr32, dtype=np.float32)
    c = np.zeros(w.shape, dtype=np.int64)
    for n in range(w.shape[0]):
        sn = np.float32(s_stored[n])
        if sn == 0:
            continue
        c[n] = np.clip(np.rint(w[n] / sn).astype(np.int64) + int(z[n]), 0, 3)
    return c


def split_asym_scales(s_w: np.ndarray):
    """The 2N scale entries of the asymmetric grid -> (s [N], z [N] int64)."""
    s_w = np.asarray(s_w)
    N = s_w.shape[0] // 2
    return s_w[:N], s_w[N:].astype(np.int64)


def quantize_weights(W: np.ndarray, B: int, kind: str, scale_dtype: str, table=None,
                     rule: str = "absmax"):
    """Offline path for one linear W [N, K]: rotate each row along K in blocks
    of B (float64), round to float32, scale rule, nearest code. kind 'lut'
    takes a level table; kind 'asym' is the min-max grid with a zero point
    (absmax rule only: its step comes from the range).
    Returns (codes int64 [N, K] (2-bit codes, or int4 values for 'int4'),
    scales [N] in the stored dtype ([2N] for 'asym': the steps, then the zero
    points), rotated float32 weights)."""
    wr32 = rotate(W, B).astype(np.float32)
    if kind == "asym":
        if rule != "absmax":
            raise ValueError("the asymmetric grid takes its step from the range")
        s, z = asym_minmax_params(wr32, scale_dtype)
        codes = asym_codes(wr32, s, z)
        return codes, np.concatenate([s, z.astype(s.dtype)]), wr32
    s = weight_scales(wr32, kind, scale_dtype, table, rule)
    if kind == "int4":
        codes = int4_weight_codes(wr32, s)
    else:
        codes = nearest_codes(wr32, s, kind, table)
    return codes, s, wr32


def gptq_hessian(X: np.ndarray, B: int, damp: float):
    """Second-order statistics of the layer input for error-compensated
    quantization (GPTQ, the column-by-column quantizer the QTEA abstract
    builds on and the Qift abstract evaluates): the calibration activations
    X [S, K] rotated like the weights (float64), H = X'^T X'. A feature whose
    diagonal entry is 0 never reaches the output: its diagonal becomes 1.
    Then the mean of the diagonal times ``damp`` is added to every diagonal
    entry. Returns (damped H [K, K] float64, dead feature mask [K])."""
    xr = rotate(X, B)
    H = xr.T @ xr
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H = H + float(damp) * float(np.mean(np.diag(H))) * np.eye(H.shape[0])
    return H, dead


def gptq_factor(H: np.ndarray) -> np.ndarray:
    """U, the upper triangular matrix with U^T U = H^-1 (Cholesky factor of
    the inverse, transposed)."""
    return np.linalg.cholesky(np.linalg.inv(H)).T


def gptq_columns(wr32: np.ndarray, s: np.ndarray, U: np.ndarray, dead: np.ndarray, kind: str,
                 table=None) -> np.ndarray:
    """The column loop. Features are quantized one at a time in their natural
    order. Feature k takes, per channel, the nearest level of its current
    weight rounded to float32 (the decision of the plain quantizer); the
    rounding error divided by U[k, k] is removed from the later features
    along row k of U. Weights of dead features start at 0. float64 updates.
    Returns codes int64 [N, K]."""
    w = np.asarray(wr32, dtype=np.float32).astype(np.float64)
    w[:, dead] = 0.0
    N, K = w.shape
    sd = np.asarray(s).astype(np.float64)
    codes = np.zeros((N, K), dtype=np.int64)
    for k in range(K):
        col32 = w[:, k].astype(np.float32)[:, None]
        if kind == "int4":
            c = int4_weight_codes(col32, s)[:, 0]
            deq = c.astype(np.float64) * sd
        else:
            c = nearest_codes(col32, s, kind, table)[:, 0]
            deq = _kind_levels(kind, table)[0][c] * sd
        codes[:, k] = c
        err = (w[:, k] - deq) / U[k, k]
        w[:, k + 1:] -= np.outer(err, U[k, k + 1:])
    return codes


def gptq_quantize_weights(W: np.ndarray, X: np.ndarray, B: int, kind: str, scale_dtype: str,
                          table=None, rule: str = "absmax", damp: float = 0.01, rows=None,
                          factor=None):
    """Error-compensated quantization with the fixed levels. The per-channel
    scales are those of ``quantize_weights`` (from the rotated float32
    weights, before any update); H and its factor U come from the rotated
    calibration activations X [S, K]; then ``gptq_columns``.
    ``rows`` (optional indices) restricts the work to a few channels: every
    channel is processed independently once U is known. ``factor`` = a
    (U, dead) pair from an earlier call, reused.
    Returns (codes int64 [R, K], scales [R] stored dtype, (U, dead))."""
    if kind == "asym":
        raise ValueError("error-compensated quantization takes the fixed level sets only")
    W = np.asarray(W)
    if rows is not None:
        W = W[np.asarray(rows)]
    wr32 = rotate(W, B).astype(np.float32)
    s = weight_scales(wr32, kind, scale_dtype, table, rule)
    if factor is None:
        H, dead = gptq_hessian(X, B, damp)
        factor = (gptq_factor(H), dead)
    U, dead = factor
    return gptq_columns(wr32, s, U, dead, kind, table), s, factor


def code_levels(codes: np.ndarray, kind: str, table=None) -> np.ndarray:
    """Integer level of each code (half-scale for MNZ, the table's entry for
    a level table): int64."""
    if kind == "int4":
        return np.asarray(codes, dtype=np.int64)
    if kind == "lut":
        lut = np.array(check_table(table), dtype=np.int64)
    else:
        lut = np.array(LEVEL_KINDS[kind]["code_to_int"], dtype=np.int64)
    return lut[np.asarray(codes, dtype=np.int64)]


def level_kappa(kind: str) -> float:
    """Factor from the integer level to the multiple of the scale."""
    return 1.0 if kind in ("lut", "asym") else LEVEL_KINDS[kind]["kappa"]


# ---------------------------------------------------------------------------
# packing (the oracle's own; the layouts are part of the interface)
# ---------------------------------------------------------------------------

def bit_offset_2b(i: int) -> int:
    """Bit offset of the code of feature k = 16*j + i inside 32-bit word j:
    byte b = (i >> 1) & 3 holds features 2b, 2b+1, 8+2b, 9+2b at bit pairs
    0-1, 2-3, 4-5, 6-7."""
    return 8 * ((i >> 1) & 3) + 4 * (i >> 3) + 2 * (i & 1)


def pack_codes2(codes: np.ndarray) -> np.ndarray:
    """int codes in [0, 4) [N, K] -> uint32 [N, K/16]."""
    codes = np.asarray(codes, dtype=np.uint64)
    N, K = codes.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    words = np.zeros((N, K // 16), dtype=np.uint64)
    for i in range(16):
        words |= (codes[:, i::16] & 3) << np.uint64(bit_offset_2b(i))
    return words.astype(np.uint32)


def unpack_codes2(words: np.ndarray) -> np.ndarray:
    """uint32 [N, K/16] -> int64 codes [N, K]."""
    words = np.asarray(words, dtype=np.uint64)
    N, W = words.shape
    codes = np.zeros((N, W * 16), dtype=np.int64)
    for i in range(16):
        codes[:, i::16] = ((words >> np.uint64(bit_offset_2b(i))) & np.uint64(3)).astype(np.int64)
    return codes


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int values in [-8, 8) [R, K] -> uint8 [R, K/2]: element 2j in the low
    nibble of byte j, element 2j+1 in the high nibble, two's complement."""
    q = np.asarray(q, dtype=np.int64)
    if q.shape[-1] % 2:
        raise ValueError("K must be even")
    nib = (q & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(b: np.ndarray) -> np.ndarray:
    """uint8 [R, K/2] -> int64 [R, K] sign-extended."""
    b = np.asarray(b, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return np.where(out >= 8, out - 16, out)


def pack_int4_words(q: np.ndarray) -> np.ndarray:
    """4-bit weight codes [N, K] -> uint32 [N, K/8] in row order (the int4
    byte layout read as little-endian 32-bit words: element i of a word at
    bits 4i..4i+3)."""
    b = pack_int4(q)
    N = b.shape[0]
    b = np.ascontiguousarray(b).reshape(N, -1, 4).astype(np.uint32)
    return (b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)).astype(np.uint32)


def unpack_int4_words(words: np.ndarray) -> np.ndarray:
    """uint32 [N, K/8] row-order words -> int64 [N, K]."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    return unpack_int4(w.view(np.uint8).reshape(w.shape[0], -1))


# Weight codes in device memory are stored in tiles of 16 output channels,
# chunk-major. With W the 32-bit words of one channel row in row order (K/16
# words for 2-bit codes, K/8 for 4-bit), T = Np/16 tiles, and the row cut into
# chunks of 16 words (u_c = min(16, W - 16c) words in chunk c):
#   tile r = channel // 16, lane-row i = channel % 16,
#   chunk c, unit-group g (0..3) and word j (0..3) of the feature's word,
#   tiled word index = c * 256 * T + r * 16 * u_c + (16 * g + i) * 4 + j
# i.e. chunk c of all tiles precedes chunk c + 1; a full chunk of a tile is
# 1 KB holding 16 channels x 16 words, unit u = 16g + i at byte 16u; a short
# last chunk holds only its first groups. Channels are padded with zero codes
# to a multiple of 16.

def _tiled_index(Np: int, W: int) -> np.ndarray:
    """tiled word index of (channel n, row-order word w), [Np, W]."""
    n = np.arange(Np)[:, None]
    w = np.arange(W)[None, :]
    r, i = n // 16, n % 16
    c, rem = w // 16, w % 16
    g, j = rem // 4, rem % 4
    T = Np // 16
    uc = np.minimum(16, W - 16 * c)
    return c * 256 * T + r * 16 * uc + (16 * g + i) * 4 + j


def tile_weight_words(rows: np.ndarray) -> np.ndarray:
    """Row-order words [N, W] (W a multiple of 4) -> tiled words
    [ceil(N/16)*16, W] (same words, tile order)."""
    rows = np.asarray(rows, dtype=np.uint32)
    N, W = rows.shape
    if W % 4:
        raise ValueError("words per row must be a multiple of 4")
    Np = -(-N // 16) * 16
    pad = np.zeros((Np, W), dtype=np.uint32)
    pad[:N] = rows
    out = np.zeros(Np * W, dtype=np.uint32)
    out[_tiled_index(Np, W)] = pad
    return out.reshape(Np, W)


def untile_weight_words(tiled: np.ndarray, N: int) -> np.ndarray:
    """Inverse of tile_weight_words: tiled [Np, W] -> row-order words [N, W]."""
    tiled = np.asarray(tiled, dtype=np.uint32)
    Np, W = tiled.shape
    return tiled.reshape(-1)[_tiled_index(Np, W)][:N]


def pack_weights(codes: np.ndarray, kind: str) -> np.ndarray:
    """Codes [N, K] -> device layout: row-order words, then 16-channel tiles."""
    rows = pack_int4_words(codes) if kind == "int4" else pack_codes2(codes)
    return tile_weight_words(rows)


def unpack_weights(tiled: np.ndarray, N: int, kind: str) -> np.ndarray:
    rows = untile_weight_words(tiled, N)
    return unpack_int4_words(rows) if kind == "int4" else unpack_codes2(rows)


# ---------------------------------------------------------------------------
# the linear (decoded weight application)
# ---------------------------------------------------------------------------

def int_matmul(q: np.ndarray, lv: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * lv[n, k], exactly (int64 result). Uses a
    float64 matmul: every term and partial sum is an integer below 2**53, so
    the result does not depend on summation order."""
    a = np.asarray(q, dtype=np.float64) @ np.asarray(lv, dtype=np.float64).T
    return np.rint(a).astype(np.int64)


def linear(q: np.ndarray, s_a: np.ndarray, codes: np.ndarray, s_w: np.ndarray, kind: str,
           table=None):
    """y = x_q W_q^T with integer accumulation: acc = q . level^T, then
    y[m, n] = acc[m, n] * s_a[m] * s_w[n] * kappa (kappa = 1/2 for the
    half-scale MNZ levels, 1 otherwise). For 'asym', s_w holds the 2N steps
    and zero points and the level of code c in channel n is c - z_n.
    Returns (acc int64, y float64)."""
    if kind == "asym":
        s_w, z = split_asym_scales(s_w)
        lv = np.asarray(codes, dtype=np.int64) - z[:, None]
    else:
        lv = code_levels(codes, kind, table)
    acc = int_matmul(q, lv)
    kappa = level_kappa(kind)
    y = acc.astype(np.float64) * np.asarray(s_a, np.float64)[:, None] \
        * np.asarray(s_w, np.float64)[None, :] * kappa
    return acc, y


# ---------------------------------------------------------------------------
# KV4
# ---------------------------------------------------------------------------

def kv4_quant(KV: np.ndarray, B: int):
    """KV [T, H, D]: rotate each head vector by H_B / sqrt(B) (B | D), then
    per (token, head) symmetric int4 as for activations.
    Returns (q int8 [T, H, D], s float32 [T, H], rotated float32)."""
    KV = np.asarray(KV, dtype=np.float64)
    T, H, D = KV.shape
    q, s, xr32, _ = rotate_quant_act(KV.reshape(T * H, D), B)
    return q.reshape(T, H, D), s.reshape(T, H), xr32.reshape(T, H, D)


def kv4_attention_decode(q: np.ndarray, k_codes: np.ndarray, k_scales: np.ndarray,
                         v_codes: np.ndarray, v_scales: np.ndarray, B: int,
                         softmax_scale: float) -> np.ndarray:
    """Decode attention over a KV4 cache (the consumer of the 4-bit KV cache of
    rotated W2A4/KV4 inference). The cache holds each head vector rotated by
    H_B / sqrt(B) and quantized; the query is rotated by the same orthogonal
    map, so q' . k' = q . k, scores are softmax_scale * (q' . k_hat'), the
    output is the softmax-weighted sum of the dequantized rotated values,
    rotated back (H_B / sqrt(B) is its own inverse). float64.

    q [S, H, D]; codes [S, T, H, D] integers; scales [S, T, H].
    Returns out [S, H, D]."""
    q = np.asarray(q, dtype=np.float64)
    kd = np.asarray(k_codes, np.float64) * np.asarray(k_scales, np.float64)[..., None]
    vd = np.asarray(v_codes, np.float64) * np.asarray(v_scales, np.float64)[..., None]
    qr = rotate(q, B)
    s = np.einsum("shd,sthd->sht", qr, kd) * float(softmax_scale)
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=2, keepdims=True)
    o_rot = np.einsum("sht,sthd->shd", p, vd)
    return rotate(o_rot, B)


# ---------------------------------------------------------------------------
# level-set analysis on a Gaussian source (Qift abstract: ratio analysis,
# Lloyd, the standard set and {+-1, +-2})
# ---------------------------------------------------------------------------

def _phi(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x: float) -> float:
    if x == math.inf:
        return 1.0
    if x == -math.inf:
        return 0.0
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def gaussian_mse(levels, s: float = 1.0) -> float:
    """Mean squared error of nearest-level quantization of a standard normal
    with reconstruction points s * levels, exactly from Phi and phi: on each
    cell [a, b] around point c, the integral of (x - c)^2 phi(x) is
    (Phi(b) - Phi(a)) + a phi(a) - b phi(b) - 2c (phi(a) - phi(b))
    + c^2 (Phi(b) - Phi(a))."""
    pts = sorted(float(v) * s for v in levels)
    edges = [-math.inf] + [(pts[i] + pts[i + 1]) / 2 for i in range(len(pts) - 1)] + [math.inf]
    total = 0.0
    for c, a, b in zip(pts, edges[:-1], edges[1:]):
        P = _Phi(b) - _Phi(a)
        aphi = 0.0 if math.isinf(a) else a * _phi(a)
        bphi = 0.0 if math.isinf(b) else b * _phi(b)
        total += P + aphi - bphi - 2.0 * c * (_phi(a) - _phi(b)) + c * c * P
    return total


def best_scale_mse(levels, lo: float = 1e-3, hi: float = 5.0):
    """(s*, MSE(s*)) minimising gaussian_mse(levels, s) over s (bounded scalar
    minimisation, scipy)."""
    from scipy.optimize import minimize_scalar
    r = minimize_scalar(lambda s: gaussian_mse(levels, s), bounds=(lo, hi),
                        method="bounded", options={"xatol": 1e-10})
    return float(r.x), float(r.fun)


def lloyd_gaussian(n_levels: int = 4, iters: int = 2000, tol: float = 1e-13):
    """Lloyd iteration on a standard normal: cells at midpoints, each point
    moved to the conditional mean (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    Returns the sorted reconstruction points."""
    pts = list(np.linspace(-1.5, 1.5, n_levels))
    for _ in range(iters):
        edges = [-math.inf] + [(pts[i] + pts[i + 1]) / 2 for i in range(n_levels - 1)] + [math.inf]
        new = []
        for a, b in zip(edges[:-1], edges[1:]):
            P = _Phi(b) - _Phi(a)
            new.append((_phi(a) - _phi(b)) / P)
        delta = max(abs(u - v) for u, v in zip(new, pts))
        pts = new
        if delta < tol:
            break
    return np.array(pts)


def inner_outer_ratio(levels) -> float:
    """min |level| / max |level| of a symmetric no-zero set."""
    m = np.abs(np.asarray(levels, dtype=np.float64))
    return float(m.min() / m.max())


def excess_kurtosis(x: np.ndarray) -> np.ndarray:
    """Per-row excess kurtosis E[(x-mu)^4]/var^2 - 3."""
    x = np.asarray(x, dtype=np.float64)
    d = x - x.mean(axis=-1, keepdims=True)
    v = (d ** 2).mean(axis=-1)
    return (d ** 4).mean(axis=-1) / (v ** 2) - 3.0
