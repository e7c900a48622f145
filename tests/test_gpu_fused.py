"""GPU parity of qift_rotate_w2a4_linear (the rotation and the linear in one
call) through the C ABI.

Contract: the same results, bit for bit, as qift_rotate_quant_act followed
by qift_w2a4_linear_ex (Y, and the xq and s_a it also writes), both for the
single-launch path (one token row, K % 16 == 0, block >= 16) and for the
two-launch path of every other call; and, end to end, the oracle's bar.
"""
import numpy as np
import pytest
import torch

import bit_quantized_fwht_amd as q
from oracle import qift_oracle as O
import synth_inputs as si
from gpu_util import DEV, say, to_dev, guarded, check_guard, rel_l2

pytestmark = pytest.mark.gpu

TABLE = (3, 10, -3, -10)


def device_weights(N, K, kind, seed):
    """Random code words (every bit pattern is a valid 2-bit code; int4 words
    are drawn nibble by nibble in [-7, 7]) and float16 scales, on the GPU."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    Np = q.padded_channels(N)
    W = q.code_words_per_row(K, kind)
    if kind == "int4":
        nib = torch.randint(-7, 8, (Np * W, 8), device=DEV, generator=g, dtype=torch.int32) & 0xF
        words = (nib << (4 * torch.arange(8, device=DEV, dtype=torch.int32))).sum(1, dtype=torch.int64)
        codes = (words - ((words >> 31) << 32)).to(torch.int32).view(Np, W)
    else:
        codes = torch.randint(-2 ** 31, 2 ** 31 - 1, (Np, W), device=DEV, generator=g,
                              dtype=torch.int32)
    scales = (torch.rand((N,), device=DEV, generator=g) * 0.1 + 0.01).to(torch.float16)
    return codes, scales


def run_both(X, B, codes, scales, kind, y_dtype, N, table=None):
    M, K = X.shape
    Yf, gy = guarded((M, N), y_dtype)
    xqf, gq = guarded((M, K // 2), torch.uint8)
    saf, gs = guarded((M,), torch.float32)
    q.qift_rotate_w2a4_linear(X, B, codes, scales, kind, Y=Yf, N=N, xq=xqf, s_a=saf, table=table)
    xq2, sa2, _ = q.qift_rotate_quant_act(X, B)
    Y2 = q.qift_w2a4_linear(xq2, sa2, codes, scales, kind, y_dtype, N=N, table=table)
    torch.cuda.synchronize()
    for g_, name in ((gy, "Y"), (gq, "xq"), (gs, "s_a")):
        check_guard(g_, name)
    return (Yf, xqf, saf), (Y2, xq2, sa2)


def assert_same(a, b, what):
    for x, y, name in zip(a, b, ("Y", "xq", "s_a")):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{what}: {name} differs"


# single-launch path: K, block (register and LDS rotation stages), N (one,
# two and four tiles per workgroup, ragged), level kinds, dtypes
FUSED_CASES = [
    (192, 64, 40, "mnz"), (256, 256, 17, "mnz"), (1024, 16, 300, "pot"), (2048, 64, 4100, "lut"),
    (4096, 4096, 4096, "mnz"), (4096, 4096, 12288, "mnz"), (4096, 4096, 22016, "mnz"),
    (4096, 4096, 22010, "int4"), (11008, 256, 4096, "mnz"), (14336, 1024, 4096, "pot"),
    (16384, 4096, 1000, "int4"), (16384, 4096, 513, "mnz"),
]


@pytest.mark.parametrize("x_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("y_dtype", [torch.bfloat16, torch.float32, torch.int32])
@pytest.mark.parametrize("K,B,N,kind", FUSED_CASES)
def test_fused_single_row_equals_two_calls(K, B, N, kind, y_dtype, x_dtype):
    X = si.device_activations(1, K, seed=K + N, device=DEV).to(x_dtype)
    codes, scales = device_weights(N, K, kind, seed=3 * K + N)
    table = TABLE if kind == "lut" else None
    say(f"fused M=1 K={K} B={B} N={N} {kind} {x_dtype} -> {y_dtype}")
    a, b = run_both(X, B, codes, scales, kind, y_dtype, N, table)
    assert_same(a, b, "fused vs two calls")


@pytest.mark.parametrize("M,K,B,N", [(2, 4096, 4096, 4096), (5, 11008, 256, 300),
                                     (16, 4096, 4096, 1000), (40, 2048, 2048, 500),
                                     (1, 512, 8, 64), (3, 192, 32, 40)])
def test_two_launch_path_equals_two_calls(M, K, B, N):
    """More than one row, a block below 16, or K not a multiple of 256: the
    call runs the rotation and the linear as two launches."""
    X = si.device_activations(M, K, seed=M + K, device=DEV)
    codes, scales = device_weights(N, K, "mnz", seed=M * K + N)
    say(f"rotate+linear two launches M={M} K={K} B={B} N={N}")
    a, b = run_both(X, B, codes, scales, "mnz", torch.float32, N)
    assert_same(a, b, "two-launch path vs two calls")


def test_fused_misaligned_input_takes_two_launches():
    """X one element into its buffer (not 16-byte aligned): the same results
    through the two-launch path."""
    K, N = 4096, 512
    buf = si.device_activations(1, K + 8, seed=9, device=DEV).reshape(-1)
    X = buf[1:K + 1].view(1, K)
    codes, scales = device_weights(N, K, "mnz", seed=10)
    say("fused misaligned X")
    a, b = run_both(X, 4096, codes, scales, "mnz", torch.bfloat16, N)
    assert_same(a, b, "misaligned X")


def test_fused_end_to_end_against_oracle():
    """The 16 x 256 case, one token row at a time through the single-launch
    path: W2A4 output within 1e-3 relative L2 of the oracle, codes only
    flipped at rounding near-ties."""
    W, X, _ = si.small_linear_case()
    cw, sw = q.qift_quantize_weights(to_dev(W), 256, "mnz", torch.float32)
    qo, so, _, xo64 = O.rotate_quant_act(X.astype(np.float64), 256)
    co, swo, _ = O.quantize_weights(W.astype(np.float64), 256, "mnz", "f32")
    _, yo = O.linear(qo, so, co, swo.astype(np.float64), "mnz")
    say("fused end to end 16x256, row by row")
    rows = []
    for m in range(16):
        Y, xq, sa = q.qift_rotate_w2a4_linear(to_dev(X[m:m + 1]), 256, cw, sw, "mnz")
        rows.append(Y)
    torch.cuda.synchronize()
    y = torch.cat(rows).cpu().numpy()
    assert rel_l2(y, yo) <= 1e-3
