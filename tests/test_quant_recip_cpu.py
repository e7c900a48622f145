"""Host check of the argument behind the GPU's reciprocal shortcut for
symmetric int4 quantization: the code of rint(x * (1/s)), rounded by adding
1.5 * 2^23 in float32, with an exact division (clamped to [-7, 7]) only
within 1e-5 of a half-integer (or for non-finite products), equals the code
of clamp(rint(x / s), -7, 7) with the IEEE float32 quotient, for
s = absmax / 7 and |x| <= absmax. Emulated in numpy float32 (IEEE, with
subnormals). Both forms the kernels use are checked: the product rounded to
float32 before the adder (code_int4_recip), and the exact product rounded
once inside a fused multiply-add (int4x8_rint_fma)."""
import numpy as np
import pytest

from oracle import qift_oracle as O

MAGIC = np.float32(12582912.0)  # 1.5 * 2^23
MAGIC8 = np.float32(12582920.0)  # 1.5 * 2^23 + 8
TINY = np.float32(2.0 ** -149)  # the smallest positive subnormal float32


def shortcut(x, s, clamp_exact=True):
    """The kernel's code decision (code_int4_recip / int4x8_rint with the
    int4x8_exact fallback), emulated in float32."""
    if s == 0:  # the kernels take r = 0 (every product 0) and code 0
        return np.zeros(np.shape(x), np.int64)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        r = np.float32(1) / s
        y = (x * r).astype(np.float32)
        ym = (y + MAGIC).astype(np.float32)
        t = (ym - MAGIC).astype(np.float32)
        code = ym.view(np.uint32).astype(np.int64) & 0xF
        exact = ~(np.abs(y - t) <= np.float32(0.49999))
        q_div = np.rint(x / s).astype(np.int64)
        if clamp_exact:
            q_div = np.clip(q_div, -7, 7)
        code_div = q_div & 0xF
    return np.where(exact, code_div, code)


def shortcut_fma(x, s, clamp_exact=True):
    """int4x8_rint_fma with the int4x8_exact fallback, emulated: the exact
    float32 x float32 product in float64 (48 significant bits, exact), plus
    the constant, rounded once to float32 (a float64 rounding first can only
    differ within 2^-29 of a half-integer, which the 0.49999 margin sends to
    the exact division anyway); the margin from a second fused multiply-add,
    P - rint(P), rounded once to float32."""
    if s == 0:
        return np.zeros(np.shape(x), np.int64)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        r = np.float32(1) / s
        P = x.astype(np.float64) * np.float64(r)
        ym = (P + np.float64(MAGIC8)).astype(np.float32)
        t = (ym - MAGIC8).astype(np.float32)
        d = (P - t.astype(np.float64)).astype(np.float32)
        code = (ym.view(np.uint32).astype(np.int64) & 0xF) ^ 0x8
        exact = ~(np.abs(d) <= np.float32(0.49999)) | ~np.isfinite(np.float32(r))
        q_div = np.rint(x / s).astype(np.int64)
        if clamp_exact:
            q_div = np.clip(q_div, -7, 7)
        code_div = q_div & 0xF
    return np.where(exact, code_div, code)


DECISIONS = {"rounded_product": shortcut, "fused": shortcut_fma}


@pytest.mark.parametrize("form", sorted(DECISIONS))
def test_reciprocal_shortcut_matches_ieee_division(form):
    shortcut = DECISIONS[form]
    rng = np.random.default_rng(0)
    total = 0
    for _ in range(60):
        amax = np.float32(10 ** rng.uniform(-37, 37))
        s = np.float32(amax) / np.float32(7)
        x = (rng.uniform(-1, 1, 100_000) * amax).astype(np.float32)
        ties = ((rng.integers(-7, 7, 1000) + 0.5).astype(np.float32) * s).astype(np.float32)
        x = np.concatenate([x, ties, np.array([amax, -amax, 0.0], np.float32)])
        with np.errstate(over="ignore", invalid="ignore"):
            ref = np.clip(np.rint(x / s), -7, 7).astype(np.int64) & 0xF
        assert np.array_equal(shortcut(x, s), ref)
        total += x.size
    assert total > 5_000_000


def subnormal_rows(seed=0):
    """Rows whose absmax is m * 2^-149 for m = 1..64 (every value an integer
    multiple of 2^-149, the largest +-m), plus rows at the top of the
    subnormal range and just above it."""
    rng = np.random.default_rng(seed)
    rows = []
    for m in range(1, 65):
        k = rng.integers(-m, m + 1, 64)
        k[rng.integers(0, 64)] = m if m % 2 else -m
        rows.append(k.astype(np.float32) * TINY)
    for a in (np.float32(2.0 ** -127), np.float32(2.0 ** -126), np.float32(2.0 ** -124)):
        rows.append((rng.uniform(-1, 1, 64).astype(np.float32) * a).astype(np.float32))
        rows[-1][0] = a
    return np.stack(rows)


@pytest.mark.parametrize("form", sorted(DECISIONS))
def test_subnormal_scales_clamp_to_seven(form):
    """With absmax = m * 2^-149, s = fl(absmax / 7) is subnormal and its
    rounding can put |x / s| above 7.5 (m = 8: s = 2^-149, x / s = 8); the
    oracle clamps to 7, and so must the kernel's exact-division fallback."""
    shortcut = DECISIONS[form]
    X = subnormal_rows()
    q_o, s_o = O.quant_sym4(X)
    clamp_bound = 0
    for r in range(X.shape[0]):
        s = np.float32(np.max(np.abs(X[r]))) / np.float32(7)
        assert s == s_o[r]
        got = shortcut(X[r], s)
        assert np.array_equal(got, q_o[r].astype(np.int64) & 0xF), r
        with np.errstate(divide="ignore", invalid="ignore"):
            clamp_bound += int(np.any(np.abs(np.rint(X[r] / s)) > 7))
    # the rows do reach the clamp, and without it the codes would differ
    assert clamp_bound >= 5
    unclamped = np.stack([shortcut(X[r], np.float32(np.max(np.abs(X[r]))) / np.float32(7),
                                   clamp_exact=False) for r in range(X.shape[0])])
    assert not np.array_equal(unclamped, q_o.astype(np.int64) & 0xF)
    # absmax 8 * 2^-149: the oracle gives +-7 where an unclamped 8 would read as -8
    row8 = np.array([8, -8, 7, 1], np.float32) * TINY
    q8, s8 = O.quant_sym4(row8[None])
    assert s8[0] == TINY and q8[0].tolist() == [7, -7, 7, 1]
