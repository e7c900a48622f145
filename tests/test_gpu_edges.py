"""GPU parity at the edges of the contract, through the C ABI, against the CPU
oracle:

* activation and KV rows at the bottom of the float32 range, where the
  scale fl(absmax / 7) is subnormal (its rounding can put |x / s| above 7.5,
  so the clamp to [-7, 7] binds) or rounds to 0 (codes 0);
* exact half-integer ties of 4-bit weights (round half to even), through
  the plain and the error-compensated quantizer;
* the float32 and bfloat16 epilogues of the grouped decode launch, the
  single-call decode kernels and the wide single-call kernel, at LLaMA-7B
  shapes, with ragged N, misaligned outputs and sentinel bytes after every
  output.

Bars: codes, scales and rotated values bit-exact where both sides see the
same exact values; float32 outputs within 4e-7 relative of the float64
oracle, bfloat16 outputs within 2^-8 relative.
"""
import json
import os

import numpy as np
import pytest
import torch

import bit_quantized_fwht_amd as q
from oracle import qift_oracle as O
import synth_inputs as si
from gpu_util import (DEV, say, to_dev, u32_to_dev, dev_u32, check_act_codes, guarded,
                      check_guard)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE_T = {"f16": torch.float16, "f32": torch.float32}


def sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# subnormal scales: clamp and zero-scale rule
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,K,batched", [(1, 256, False), (16, 256, False), (256, 256, False),
                                         (4096, 4096, False), (256, 512, True)])
def test_rotate_subnormal_rows(B, K, batched):
    """Rows of integer multiples of 2^-149: the butterfly sums are exact and
    1/sqrt(B) is a power of two, so both sides round the same exact rotated
    values once; scales, codes and rotated values must agree bit for bit,
    including rows where the clamp binds and rows whose scale rounds to 0.
    B = 1 runs the general kernel, B >= 16 the register kernel (B = 4096
    through its LDS stage), batched the multi-matrix launch."""
    M = 70
    X = si.subnormal_rows(M, K, seed=B + K)
    qo, so, xo32, _ = O.rotate_quant_act(X.astype(np.float64), B)
    hits = sum(int(so[r] > 0 and np.abs(np.rint(xo32[r] / so[r])).max() > 7) for r in range(M))
    assert hits >= 3 and np.any(so == 0)  # the case reaches the clamp and the zero scale
    say(f"rotate subnormal rows B={B} K={K} batched={batched}")
    xq, gq = guarded((M, K // 2), torch.uint8)
    s_a, gs = guarded((M,), torch.float32)
    xr, gx = guarded((M, K), torch.float32)
    if batched:
        q.qift_rotate_quant_act_batched([(to_dev(X), B, xq, s_a, xr)])
    else:
        q.qift_rotate_quant_act(to_dev(X), B, xq=xq, s_a=s_a, x_rot=xr)
    sync()
    for g, name in ((gq, "xq"), (gs, "s_a"), (gx, "x_rot")):
        check_guard(g, name)
    assert np.array_equal(s_a.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(xr.cpu().numpy(), xo32)
    assert np.array_equal(O.unpack_int4(xq.cpu().numpy()), qo.astype(np.int64))


@pytest.mark.parametrize("D,B", [(128, 16), (128, 64), (64, 64), (128, 128)])
def test_kv4_subnormal_rows(D, B):
    """KV head vectors of integer multiples of 2^-149. With 1/sqrt(B) a power
    of two both sides round the same exact values (bit-exact codes); for
    B = 128 the kernel multiplies by fl(1/sqrt(128)), so a code may differ
    only at a rounding near-tie."""
    T, H = 64, 2
    KV = si.subnormal_rows(T * H, D, seed=D + B).reshape(T, H, D)
    qo, so, _ = O.kv4_quant(KV.astype(np.float64), B)
    say(f"kv4 subnormal rows D={D} B={B}")
    kvq, gk = guarded((T, H, D // 2), torch.uint8)
    sc, gsc = guarded((T, H), torch.float32)
    q.qift_kv4_quant(to_dev(KV), B, kvq=kvq, scales=sc)
    sync()
    check_guard(gk, "kvq")
    check_guard(gsc, "scales")
    qg = O.unpack_int4(kvq.cpu().numpy())
    sg = sc.cpu().numpy()
    if B in (16, 64):
        assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
        assert np.array_equal(qg, qo.astype(np.int64))
    else:
        assert np.array_equal(sg == 0, so == 0)
        assert np.allclose(sg, so, rtol=2 ** -20, atol=2.0 ** -149)
        xo64 = O.rotate(KV.reshape(T * H, D).astype(np.float64), B).reshape(T, H, D)
        live = (sg == so)  # rows whose scale agrees: codes differ only at near-ties
        check_act_codes(qg[live], qo[live], xo64[live], so[live], frac=1e-2)


# ---------------------------------------------------------------------------
# 4-bit weight ties (round half to even)
# ---------------------------------------------------------------------------

def int4_tie_rows():
    g = json.load(open(os.path.join(GOLDEN, "int4_weight_ties.json")))
    rows, codes = [], []
    for case in g["rows"]:
        r = np.tile(np.array(case["row"], np.float32), 4)  # 64 features
        c = np.tile(np.array(case["codes"], np.int64), 4)
        rows += [r, -r]
        codes += [c, -c]
    return np.stack(rows), np.stack(codes)


@pytest.mark.parametrize("sdt", ["f16", "f32"])
def test_int4_weight_ties_plain_quantizer(sdt):
    W, expect = int4_tie_rows()
    N, K = W.shape
    say(f"int4 weight ties, plain quantizer {sdt}")
    codes, gc = guarded((q.padded_channels(N), K // 8), torch.int32)
    scales, gs = guarded((N,), SCALE_T[sdt])
    q.qift_quantize_weights(to_dev(W), 1, "int4", SCALE_T[sdt], codes=codes, scales=scales)
    sync()
    check_guard(gc, "codes")
    check_guard(gs, "scales")
    got = O.unpack_weights(dev_u32(codes), N, "int4")
    assert np.array_equal(got, expect)
    co, so, _ = O.quantize_weights(W.astype(np.float64), 1, "int4", sdt)
    assert np.array_equal(got, co)


@pytest.mark.parametrize("sdt", ["f16", "f32"])
def test_int4_weight_ties_error_compensated(sdt):
    """With H = I every update term vanishes (U is diagonal), so the
    error-compensated quantizer decides each weight as it stands: the ties
    must round half to even there too."""
    W, expect = int4_tie_rows()
    N, K = W.shape
    H = torch.eye(K, dtype=torch.float64, device=DEV)
    say(f"int4 weight ties, error-compensated quantizer {sdt}")
    codes, scales = q.qift_gptq_quantize_weights(to_dev(W), H, 1, "int4", SCALE_T[sdt])
    sync()
    assert np.array_equal(O.unpack_weights(dev_u32(codes), N, "int4"), expect)


# ---------------------------------------------------------------------------
# float epilogues of the decode kernels
# ---------------------------------------------------------------------------

def make_weights(K, N, kind, seed):
    codes = si.uniform_int4((N, K), seed=seed) if kind == "int4" \
        else si.uniform_codes((N, K), 4, seed=seed)
    s_w = si.positive_scales(N, seed + 1).astype(np.float16)
    return codes, s_w, u32_to_dev(O.pack_weights(codes, kind)), \
        to_dev(s_w.astype(np.float32), torch.float16)


def check_float(Y, y, y_dtype, what):
    got = Y.float().cpu().numpy().astype(np.float64)
    tol = 4e-7 if y_dtype == torch.float32 else 2.0 ** -8
    bad = np.abs(got - y) > tol * np.abs(y) + 1e-30
    assert not np.any(bad), f"{what}: {int(bad.sum())} outputs outside {tol:g} relative"


@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_grouped_float_epilogue_llama_shapes(y_dtype):
    """The grouped launch the decode benchmark times (float16 scales, float
    outputs) at the LLaMA-7B shapes for M = 1, 4, 8, 16, plus ragged N
    (N % 4 != 0) and outputs misaligned by 1-3 elements (the element-wise
    store path), every output guarded; two consecutive runs."""
    shapes = {(4096, 4096): "mnz", (4096, 11008): "mnz", (11008, 4096): "mnz",
              (4096, 4099): "mnz", (1024, 1001): "pot", (2048, 777): "int4", (512, 130): "lut"}
    table = (3, 10, -3, -10)
    wts = {kn: make_weights(kn[0], kn[1], kind, seed=11 * kn[0] + kn[1])
           for kn, kind in shapes.items()}
    items, refs, guards = [], [], []
    for M in (1, 4, 8, 16):
        for (K, N), kind in shapes.items():
            codes, s_w, cw, swt = wts[(K, N)]
            qa = si.uniform_int4((M, K), seed=M * 7 + K)
            s_a = si.positive_scales(M, seed=M + N)
            off = (M + N) % 4 if N % 4 else 0  # misaligned outputs for the ragged shapes
            Y, gy = guarded((M, N), y_dtype, offset=off)
            tb = table if kind == "lut" else None
            items.append(dict(xq=torch.from_numpy(O.pack_int4(qa)).to(DEV), s_a=to_dev(s_a),
                              codes=cw, scales=swt, Y=Y, levels=kind, table=tb))
            refs.append(O.linear(qa, s_a, codes, s_w.astype(np.float64), kind, tb)[1])
            guards.append(gy)
    say(f"grouped float epilogue {y_dtype} ({len(items)} linears)")
    grp = q.LinearGroup(items, scale_dtype=torch.float16, y_dtype=y_dtype)
    for rep in range(2):
        for it in items:  # every run must write every output element
            it["Y"].view(torch.uint8).fill_(0x5C)
        grp.run()
        sync()
        for it, y, g in zip(items, refs, guards):
            check_guard(g, f"Y M={it['Y'].shape[0]} N={it['Y'].shape[1]}")
            check_float(it["Y"], y, y_dtype, f"grouped M={it['Y'].shape[0]} N={it['Y'].shape[1]}")


@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,K,N,kind,off", [
    (1, 4096, 4096, "mnz", 0), (16, 11008, 4096, "mnz", 0), (4, 4096, 11008, "pot", 0),
    (8, 4096, 4099, "mnz", 1), (16, 2048, 1001, "int4", 3), (2, 4096, 22010, "mnz", 2),
    (2, 256, 131100, "mnz", 0), (16, 256, 131104, "mnz", 0), (3, 512, 131101, "pot", 1)])
def test_single_call_float_epilogue(y_dtype, M, K, N, kind, off):
    """One linear per call (M <= 16): the split-K decode kernel at LLaMA-7B
    shapes (one, two and four 16-channel tiles per workgroup; N = 22010 ends
    in a workgroup whose last tile is partial) and, for N >= 131072, the
    64-channel-wave kernel, with float outputs (ragged N and misaligned
    outputs included), guarded."""
    codes, s_w, cw, swt = make_weights(K, N, kind, seed=K + N + M)
    qa = si.uniform_int4((M, K), seed=M + 3 * K)
    s_a = si.positive_scales(M, seed=M + 5)
    say(f"single-call float epilogue {y_dtype} M={M} K={K} N={N} {kind} offset {off}")
    Y, gy = guarded((M, N), y_dtype, offset=off)
    q.qift_w2a4_linear(torch.from_numpy(O.pack_int4(qa)).to(DEV), to_dev(s_a), cw, swt, kind,
                       y_dtype, Y=Y)
    sync()
    check_guard(gy, "Y")
    _, y = O.linear(qa, s_a, codes, s_w.astype(np.float64), kind)
    check_float(Y, y, y_dtype, "single call")
