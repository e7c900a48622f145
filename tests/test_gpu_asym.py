"""GPU parity of the asymmetric min-max two-bit grid with a zero point
(QIFT_LEVELS_ASYM, the baseline the Qift abstract compares its no-zero sets
with) against the oracle.

Bar: the quantizer's steps, zero points and codes bit-exact on identical
rotated input (and on the hand-worked fixture); with the rotation inside,
steps within float32 rounding and codes flipped only at rounding near-ties.
The linear's int32 accumulator bit-exact through every kernel that runs it
(split-K and wide decode, the grouped launch, the one-call rotation +
linear, the general and the direct-to-LDS prefill), float32 / bfloat16
outputs within one rounding of the exact value.
"""
import json
import os

import numpy as np
import pytest
import torch

import bit_quantized_fwht_amd as q
from oracle import qift_oracle as O
import synth_inputs as si
from gpu_util import DEV, say, to_dev, u32_to_dev, dev_u32, rel_l2, guarded, check_guard

pytestmark = pytest.mark.gpu

SCALE_T = {"f16": torch.float16, "f32": torch.float32}


def skewed_weights(N, K, seed):
    """Gaussian rows shifted by a per-row offset (so that lo and hi differ and
    the zero points spread over 0..3), with an all-positive, an all-negative
    and an all-zero row when N allows."""
    W = si.weights(N, K, seed=seed, sigma=0.02).astype(np.float64)
    W += ((np.arange(N) % 7) - 3)[:, None] * 0.012
    if N >= 3:
        W[0] = np.abs(W[0]) + 0.001
        W[1] = -np.abs(W[1]) - 0.001
        W[2] = 0.0
    return W.astype(np.float32)


def gpu_quant_asym(W_t, B, sdt):
    N, K = W_t.shape
    codes, gc = guarded((q.padded_channels(N), K // 16), torch.int32)
    scales, gs = guarded((2, N), SCALE_T[sdt])
    q.qift_quantize_weights(W_t, B, "asym", SCALE_T[sdt], codes=codes, scales=scales)
    torch.cuda.synchronize()
    check_guard(gc, "codes")
    check_guard(gs, "scales")
    words = dev_u32(codes)
    return O.unpack_weights(words, N, "asym"), scales.float().cpu().numpy(), words


def test_asym_quantizer_hand_example():
    """tests/golden/asym_minmax.json (rows repeated to K = 64, which keeps
    each row's range): steps, zero points and codes as worked by hand."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "asym_minmax.json")))
    W = np.array([r["row"] * 8 for r in g["rows"]], np.float32)
    for sdt in ("f16", "f32"):
        say(f"asym quantizer fixture {sdt}")
        cg, sg, _ = gpu_quant_asym(to_dev(W), 1, sdt)
        for i, r in enumerate(g["rows"]):
            assert float(sg[0, i]) == r["scale"][sdt], r["name"]
            assert float(sg[1, i]) == r["zero"], r["name"]
            assert cg[i].tolist() == r["codes"] * 8, r["name"]


@pytest.mark.parametrize("sdt", ["f16", "f32"])
@pytest.mark.parametrize("N,K", [(1, 64), (37, 256), (130, 4096), (5, 11008), (19, 16384)])
def test_asym_quantizer_bitexact_given_rotated_input(sdt, N, K):
    B = 256 if K % 256 == 0 else 64
    W = skewed_weights(N, K, seed=N * 13 + K)
    wr32 = O.rotate(W.astype(np.float64), B).astype(np.float32)
    say(f"asym quantizer bitexact {sdt} N={N} K={K}")
    cg, sg, words = gpu_quant_asym(to_dev(wr32), 1, sdt)
    co, so, _ = O.quantize_weights(wr32.astype(np.float64), 1, "asym", sdt)
    assert np.array_equal(sg[0].astype(np.float32).view(np.uint32),
                          so[:N].astype(np.float32).view(np.uint32))
    assert np.array_equal(sg[1], so[N:].astype(np.float32))
    assert np.array_equal(cg, co)
    assert np.array_equal(words, O.pack_weights(co, "asym"))


def test_asym_quantizer_rotated():
    """With the rotation inside (float32 butterflies against the oracle's
    float64 rotation): steps within float32 rounding, zero points equal
    except at a near-tie of -lo / s, codes equal except +-1 at near-ties of
    w / s, at most 1e-4 of them."""
    N, K, B = 48, 4096, 4096
    W = skewed_weights(N, K, seed=5)
    say("asym quantizer rotated 48 x 4096")
    cg, sg, _ = gpu_quant_asym(to_dev(W), B, "f32")
    co, so, wr32 = O.quantize_weights(W.astype(np.float64), B, "asym", "f32")
    w64 = O.rotate(W.astype(np.float64), B)
    s_o, z_o = so[:N].astype(np.float64), so[N:].astype(np.int64)
    assert np.allclose(sg[0], s_o, rtol=2e-6, atol=0)
    bad = 0
    for n in range(N):
        lo = min(w64[n].min(), 0.0)
        if sg[1, n] != z_o[n]:
            t = -lo / s_o[n]
            assert abs(t - np.floor(t) - 0.5) < 1e-4, n
            continue
        diff = cg[n] != co[n]
        if not diff.any():
            continue
        assert np.all(np.abs(cg[n] - co[n])[diff] == 1)
        r = w64[n] / s_o[n]
        assert np.all(np.abs(r - np.floor(r) - 0.5)[diff] < 1e-4)
        bad += int(diff.sum())
    assert bad <= max(1, 1e-4 * N * K)


# ---------------------------------------------------------------------------
# the linear
# ---------------------------------------------------------------------------

def asym_linear_inputs(M, K, N, seed):
    qa = si.uniform_int4((M, K), seed=seed)
    codes = si.uniform_codes((N, K), 4, seed=seed + 1)
    s_a = si.positive_scales(M, seed + 2)
    s_w = si.positive_scales(N, seed + 3).astype(np.float16)
    z = si.uniform_codes((N,), 4, seed=seed + 4)
    return qa, codes, s_a, s_w, z


def asym_scales(s_w, z):
    return np.concatenate([s_w.astype(np.float64), z.astype(np.float64)])


def run_asym(qa, codes, s_a, s_w, z, out_dtype):
    xq = torch.from_numpy(O.pack_int4(qa)).to(DEV)
    cw = u32_to_dev(O.pack_weights(codes, "asym"))
    sc = to_dev(asym_scales(s_w, z), torch.float16)
    Y, gy = guarded((qa.shape[0], codes.shape[0]), out_dtype)
    q.qift_w2a4_linear(xq, to_dev(s_a), cw, sc, "asym", out_dtype, Y=Y, N=codes.shape[0])
    torch.cuda.synchronize()
    check_guard(gy, "Y")
    return Y


# decode: split-K (few tiles) and 64-channel waves ((2, 256, 131100));
# prefill: general kernel (K % 256 != 0: 576, 320) and direct-to-LDS kernel
# with 64- and 128-row tiles
ASYM_SHAPES = [(1, 64, 1), (1, 256, 17), (4, 4096, 257), (16, 1024, 129), (2, 8448, 33),
               (3, 3072, 4100), (2, 256, 131100), (1, 2048, 20000), (17, 256, 130),
               (31, 320, 63), (129, 576, 200), (200, 2048, 385), (1000, 256, 8200)]


@pytest.mark.parametrize("M,K,N", ASYM_SHAPES)
def test_asym_linear_int32_bitexact(M, K, N):
    qa, codes, s_a, s_w, z = asym_linear_inputs(M, K, N, seed=M * 1000 + K + N)
    say(f"asym linear i32 M={M} K={K} N={N}")
    Y = run_asym(qa, codes, s_a, s_w, z, torch.int32).cpu().numpy()
    acc, _ = O.linear(qa, s_a, codes, asym_scales(s_w, z), "asym")
    assert np.array_equal(Y.astype(np.int64), acc)


@pytest.mark.parametrize("M,K,N", [(1, 256, 33), (16, 512, 100), (2, 256, 131100), (40, 1024, 150),
                                   (130, 768, 136), (1000, 256, 8200)])
def test_asym_linear_float_epilogue(M, K, N):
    qa, codes, s_a, s_w, z = asym_linear_inputs(M, K, N, seed=5 + M + N)
    say(f"asym linear f32/bf16 M={M} K={K} N={N}")
    _, y = O.linear(qa, s_a, codes, asym_scales(s_w, z), "asym")
    Yf = run_asym(qa, codes, s_a, s_w, z, torch.float32).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Yf - y) <= 4e-7 * np.abs(y) + 1e-30)
    Yb = run_asym(qa, codes, s_a, s_w, z, torch.bfloat16).float().cpu().numpy()
    assert np.all(np.abs(Yb - y) <= 2 ** -8 * np.abs(y) + 1e-30)


@pytest.mark.parametrize("y_dtype", [torch.int32, torch.bfloat16])
def test_asym_in_grouped_launch(y_dtype):
    shapes = [(1, 4096, 1000, "mnz"), (4, 512, 300, "asym"), (16, 256, 64, "asym"),
              (2, 1024, 200, "pot"), (1, 11008, 4096, "asym")]
    items, refs = [], []
    for i, (M, K, N, kind) in enumerate(shapes):
        if kind == "asym":
            qa, codes, s_a, s_w, z = asym_linear_inputs(M, K, N, seed=970 + i)
            sc = asym_scales(s_w, z)
        else:
            qa = si.uniform_int4((M, K), seed=970 + i)
            codes = si.uniform_codes((N, K), 4, seed=971 + i)
            s_a = si.positive_scales(M, 972 + i)
            sc = si.positive_scales(N, 973 + i).astype(np.float16).astype(np.float64)
        Y, gy = guarded((M, N), y_dtype)
        items.append(dict(xq=torch.from_numpy(O.pack_int4(qa)).to(DEV), s_a=to_dev(s_a),
                          codes=u32_to_dev(O.pack_weights(codes, kind)),
                          scales=to_dev(sc, torch.float16), Y=Y, levels=kind, N=N, guard=gy))
        refs.append(O.linear(qa, s_a, codes, sc, kind))
    say(f"grouped linear with asymmetric items -> {y_dtype}")
    grp = q.LinearGroup(items, scale_dtype=torch.float16, y_dtype=y_dtype)
    grp.run()
    torch.cuda.synchronize()
    for it, (acc, y) in zip(items, refs):
        check_guard(it["guard"], "Y")
        if y_dtype == torch.int32:
            assert np.array_equal(it["Y"].cpu().numpy().astype(np.int64), acc)
        else:
            Yb = it["Y"].float().cpu().numpy()
            assert np.all(np.abs(Yb - y) <= 2 ** -8 * np.abs(y) + 1e-30)


@pytest.mark.parametrize("K,B,N", [(4096, 4096, 4096), (11008, 256, 4096), (1024, 16, 300),
                                   (4096, 4096, 22016)])
def test_asym_rotate_linear_one_call_equals_two_calls(K, B, N):
    """The rotation folded into the single-row linear gives the two calls'
    results bit for bit with asymmetric weights."""
    X = si.device_activations(1, K, seed=K + N, device=DEV)
    W = skewed_weights(N, K, seed=N + 3)
    codes, scales = q.qift_quantize_weights(to_dev(W), B, "asym", torch.float16)
    say(f"asym rotate+linear one call K={K} B={B} N={N}")
    Y1, gy = guarded((1, N), torch.bfloat16)
    xq1 = torch.empty((1, K // 2), dtype=torch.uint8, device=DEV)
    sa1 = torch.empty((1,), dtype=torch.float32, device=DEV)
    q.qift_rotate_w2a4_linear(X, B, codes, scales, "asym", Y=Y1, xq=xq1, s_a=sa1)
    xq2, sa2, _ = q.qift_rotate_quant_act(X, B)
    Y2 = q.qift_w2a4_linear(xq2, sa2, codes, scales, "asym", torch.bfloat16)
    torch.cuda.synchronize()
    check_guard(gy, "Y")
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(xq1, xq2) and torch.equal(sa1, sa2)


def test_asym_end_to_end_against_oracle():
    """16 x 256 weights and tokens, everything on the GPU (quantizer, rotation,
    linear) against the oracle's pipeline: within 1e-3 relative L2."""
    W = skewed_weights(64, 256, seed=11)
    _, X, _ = si.small_linear_case()
    say("asym end to end 16 x 256 x 64")
    cw, sw = q.qift_quantize_weights(to_dev(W), 256, "asym", torch.float32)
    xq, sa, _ = q.qift_rotate_quant_act(to_dev(X), 256)
    Y = q.qift_w2a4_linear(xq, sa, cw, sw, "asym").cpu().numpy()
    co, so, _ = O.quantize_weights(W.astype(np.float64), 256, "asym", "f32")
    qo, sao, _, _ = O.rotate_quant_act(X.astype(np.float64), 256)
    _, yo = O.linear(qo, sao, co, so.astype(np.float64), "asym")
    assert rel_l2(Y, yo) <= 1e-3
