"""Host check of the argument behind the GPU's reciprocal shortcut for
symmetric int4 quantization: the code of rint(x * (1/s)), rounded by adding
1.5 * 2^23 in float32, with an exact division only within 1e-5 of a
half-integer (or for non-finite products), equals the code of
clamp(rint(x / s), -7, 7) with the IEEE float32 quotient, for s = absmax / 7
and |x| <= absmax. Emulated in numpy float32 (IEEE)."""
import numpy as np


MAGIC = np.float32(12582912.0)  # 1.5 * 2^23


def shortcut(x, s):
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.float32(1) / s
        y = (x * r).astype(np.float32)
        ym = (y + MAGIC).astype(np.float32)
        t = (ym - MAGIC).astype(np.float32)
        code = ym.view(np.uint32).astype(np.int64) & 0xF
        exact = ~(np.abs(y - t) <= np.float32(0.49999))
        code_div = np.rint(x / s).astype(np.int64) & 0xF
    return np.where(exact, code_div, code)


def test_reciprocal_shortcut_matches_ieee_division():
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
