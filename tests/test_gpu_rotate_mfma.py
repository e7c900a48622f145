"""The matrix-core rotation of bfloat16 rows: K = 4096 with one block of 4096
(the inputs of the K = 4096 linears of LLaMA-shaped prefill), and blocks of
256, 512 and 1024 for any K (the K = 11008 and K = 14336 inputs): rotated
values against the float64 oracle, the quantizer bit-exact on the kernel's
own rotated values, exact rounding ties and degenerate rows against the
oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_fwht_amd as q
from oracle import qift_oracle as O
import synth_inputs as si
from gpu_util import DEV, say, check_act_codes, guarded, check_guard

pytestmark = pytest.mark.gpu
K = B = 4096


def sync():
    torch.cuda.synchronize()


def rotate(Xt, want_rot=True):
    M = Xt.shape[0]
    xq, gq = guarded((M, K // 2), torch.uint8)
    s_a, gs = guarded((M,), torch.float32)
    xr, gx = guarded((M, K), torch.float32) if want_rot else (None, None)
    q.qift_rotate_quant_act(Xt, B, xq=xq, s_a=s_a, x_rot=xr)
    sync()
    check_guard(gq, "xq")
    check_guard(gs, "s_a")
    if want_rot:
        check_guard(gx, "x_rot")
    return (O.unpack_int4(xq.cpu().numpy()), s_a.cpu().numpy(),
            xr.cpu().numpy() if want_rot else None)


def test_mfma_rotation_prefill_rows():
    """2048 bfloat16 rows with outlier channels: rotated values within 1e-5
    of the float64 rotation on sampled rows, codes equal to the oracle's
    except at rounding near-ties, and the codes and scales bit-exact against
    the oracle's quantizer applied to the kernel's own rotated values; the
    call without the rotated output gives the same codes and scales."""
    M = 2048
    Xt = si.device_activations(M, K, seed=6, device=DEV)
    say("matrix-core rotation 2048 x 4096")
    qg, sg, xg = rotate(Xt)
    qn, sn, _ = rotate(Xt, want_rot=False)
    assert np.array_equal(qn, qg) and np.array_equal(sn.view(np.uint32), sg.view(np.uint32))
    qo_self, so_self = O.quant_sym4(xg)
    assert np.array_equal(sg.view(np.uint32), so_self.view(np.uint32))
    assert np.array_equal(qg, qo_self.astype(np.int64))
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(3).choice(M, 40, replace=False)]))
    Xv = Xt[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    qo, so, _, xo64 = O.rotate_quant_act(Xv, B)
    for i in range(len(rows)):
        assert np.abs(xg[rows[i]] - xo64[i]).max() <= 1e-5 * np.abs(xo64[i]).max()
    assert np.allclose(sg[rows], so, rtol=1e-6, atol=0)
    check_act_codes(qg[rows], qo, xo64, so)


def hadamard_row(i):
    e = np.arange(K)
    pc = np.array([bin(int(v)).count("1") for v in (e & i)])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def test_mfma_rotation_exact_ties():
    """Rows alpha h_i + beta h_j of two Hadamard rows (bfloat16-exact, every
    partial sum exact) rotate to exactly 64 alpha at i and 64 beta at j: with
    alpha = 7 the scale is 64 and the code at j is rint(beta), half to even,
    through every stage of the kernel (matrix core, lanes, LDS)."""
    cases = [(7.0, 1.5, 5, 77), (7.0, 2.5, 100, 3000), (7.0, -0.5, 4095, 0), (7.0, 3.5, 31, 32),
             (-7.0, -2.5, 1234, 2048), (7.0, 0.5, 511, 1536), (7.0, -3.5, 2, 4094), (7.0, 6.5, 64, 65)]
    X = np.stack([a * hadamard_row(i) + b * hadamard_row(j) for a, b, i, j in cases])
    assert np.array_equal(X.astype(np.float32), X)
    Xt = torch.from_numpy(X.astype(np.float32)).to(DEV).to(torch.bfloat16)
    assert np.array_equal(Xt.float().cpu().numpy(), X)  # bfloat16-exact
    say("matrix-core rotation exact ties")
    qg, sg, xg = rotate(Xt)
    qo, so, xo32, xo64 = O.rotate_quant_act(X, B)
    assert np.array_equal(xg, xo32)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo.astype(np.int64))
    for r, (a, b, i, j) in enumerate(cases):
        assert sg[r] == 64.0 and qg[r, i] == (7 if a > 0 else -7)
        assert qg[r, j] == int(np.rint(b))


def test_mfma_rotation_degenerate_rows():
    """A zero row (scale 0, codes 0), a constant row (one nonzero rotated
    value), rows of the smallest normal and of subnormal bfloat16 values
    (bfloat16 subnormals are multiples of 2^-133): codes, scales and
    rotated values equal to the oracle's."""
    rng = np.random.default_rng(11)
    tiny = 2.0 ** -133
    rows = [np.zeros(K), np.full(K, 3.0), 2.0 ** -126 * hadamard_row(9),
            tiny * rng.integers(-100, 101, K).astype(np.float64),
            tiny * hadamard_row(700) * 5.0, tiny * rng.integers(-3, 4, K).astype(np.float64)]
    X = np.stack(rows)
    Xt = torch.from_numpy(X.astype(np.float32)).to(DEV).to(torch.bfloat16)
    Xv = Xt.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(Xv, X)  # exact in bfloat16
    say("matrix-core rotation degenerate rows")
    qg, sg, xg = rotate(Xt)
    qo, so, xo32, xo64 = O.rotate_quant_act(Xv, B)
    assert sg[0] == 0 and np.all(qg[0] == 0)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo.astype(np.int64))
    assert np.array_equal(xg, xo32)


# ---------------------------------------------------------------------------
# blocks of 256, 512 and 1024 (rotate_quant_act_mfma_groups_kernel): K up to
# 16384, one to four groups of 1024 elements per wave, rows ending in a
# partial group (K = 11008 and 2816 with blocks of 256, 1536 and 11264 with
# blocks of 512), K = 13312 with waves of three and four groups
# ---------------------------------------------------------------------------

def rotate_kb(Xt, Bk, want_rot=True):
    M, Kk = Xt.shape
    xq, gq = guarded((M, Kk // 2), torch.uint8)
    s_a, gs = guarded((M,), torch.float32)
    xr, gx = guarded((M, Kk), torch.float32) if want_rot else (None, None)
    q.qift_rotate_quant_act(Xt, Bk, xq=xq, s_a=s_a, x_rot=xr)
    sync()
    check_guard(gq, "xq")
    check_guard(gs, "s_a")
    if want_rot:
        check_guard(gx, "x_rot")
    return (O.unpack_int4(xq.cpu().numpy()), s_a.cpu().numpy(),
            xr.cpu().numpy() if want_rot else None)


@pytest.mark.parametrize("M,Kk,Bk", [(2048, 11008, 256), (1024, 14336, 1024), (64, 4096, 512),
                                     (33, 2048, 1024), (5, 256, 256), (9, 16384, 256),
                                     (7, 16384, 1024), (3, 13312, 1024), (5, 1536, 512),
                                     (3, 11264, 512), (4, 2816, 256)])
def test_mfma_group_rotation_rows(M, Kk, Bk):
    """bfloat16 rows with outlier channels: rotated values within 1e-5 of the
    float64 rotation on sampled rows, codes equal to the oracle's except at
    near-ties, codes and scales bit-exact against the oracle's quantizer on
    the kernel's own rotated values, with and without the rotated output."""
    Xt = si.device_activations(M, Kk, seed=M + Kk + Bk, device=DEV)
    say(f"matrix-core group rotation M={M} K={Kk} B={Bk}")
    qg, sg, xg = rotate_kb(Xt, Bk)
    qn, sn, _ = rotate_kb(Xt, Bk, want_rot=False)
    assert np.array_equal(qn, qg) and np.array_equal(sn.view(np.uint32), sg.view(np.uint32))
    qo_self, so_self = O.quant_sym4(xg)
    assert np.array_equal(sg.view(np.uint32), so_self.view(np.uint32))
    assert np.array_equal(qg, qo_self.astype(np.int64))
    rng = np.random.default_rng(M + Bk)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 24), replace=False)]))
    Xv = Xt[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    qo, so, _, xo64 = O.rotate_quant_act(Xv, Bk)
    for i in range(len(rows)):
        assert np.abs(xg[rows[i]] - xo64[i]).max() <= 1e-5 * np.abs(xo64[i]).max()
    assert np.allclose(sg[rows], so, rtol=1e-6, atol=0)
    check_act_codes(qg[rows], qo, xo64, so)


def block_hadamard_row(Kk, Bk, blk, i):
    """Row with H_B row i in block blk and zeros elsewhere."""
    r = np.zeros(Kk)
    e = np.arange(Bk)
    pc = np.array([bin(int(v)).count("1") for v in (e & i)])
    r[blk * Bk:(blk + 1) * Bk] = np.where(pc % 2 == 0, 1.0, -1.0)
    return r


@pytest.mark.parametrize("Kk,Bk", [(11008, 256), (14336, 1024), (4096, 256), (16384, 1024)])
def test_mfma_group_rotation_exact_ties(Kk, Bk):
    """alpha h_i + beta h_j inside one block (the last block of the row
    among them) rotates to exactly sqrt(B) alpha and sqrt(B) beta (blocks
    whose sqrt is a power of two, so the normalization is exact); with
    alpha = 7 the scale is sqrt(B) and the code at j is rint(beta), half to
    even; zero, constant and subnormal rows equal the oracle's too."""
    nb = Kk // Bk
    cases = [(7.0, 1.5, 0, 5, 77), (7.0, 2.5, nb - 1, 100, 3), (-7.0, -0.5, nb // 2, 0, Bk - 1),
             (7.0, 3.5, nb - 1, Bk - 2, 1), (7.0, -6.5, 1, 64, 65)]
    rows = [a * block_hadamard_row(Kk, Bk, blk, i) + b * block_hadamard_row(Kk, Bk, blk, j)
            for a, b, blk, i, j in cases]
    rng = np.random.default_rng(Kk)
    tiny = 2.0 ** -133
    rows += [np.zeros(Kk), np.full(Kk, 3.0), tiny * rng.integers(-100, 101, Kk).astype(np.float64)]
    X = np.stack(rows)
    Xt = torch.from_numpy(X.astype(np.float32)).to(DEV).to(torch.bfloat16)
    assert np.array_equal(Xt.float().cpu().numpy(), X)  # bfloat16-exact
    say(f"matrix-core group rotation exact ties K={Kk} B={Bk}")
    qg, sg, xg = rotate_kb(Xt, Bk)
    qo, so, xo32, _ = O.rotate_quant_act(X, Bk)
    assert np.array_equal(xg, xo32)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo.astype(np.int64))
    for r, (a, b, blk, i, j) in enumerate(cases):
        assert qg[r, blk * Bk + i] == (7 if a > 0 else -7)
        assert qg[r, blk * Bk + j] == int(np.rint(b))
