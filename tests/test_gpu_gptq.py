"""GPU parity of the error-compensated (GPTQ-style) weight quantizer against
the CPU oracle, through the C ABI.

Bar: H within 1e-12 of the largest entry (float64 sums in a different order);
scales bit-exact; codes bit-exact. Both sides decide each code on the current
weight rounded to float32 against the same stored scale, and the weights they
decide on differ only by float64 rounding (blocked against unblocked update
order), so a code could differ only for a weight within ~1e-16 of a decision
boundary; none occurs in these seeded cases. The full up_proj shape is checked
on sampled channel rows (every row is independent given H).
"""
import numpy as np
import pytest
import torch

import bit_quantized_fwht_amd as q
from oracle import qift_oracle as O
import synth_inputs as si
from gpu_util import DEV, say, to_dev, dev_u32, rel_l2

pytestmark = pytest.mark.gpu

SCALE_T = {"f16": torch.float16, "f32": torch.float32}


def sync():
    torch.cuda.synchronize()


def oracle_hessian(X, B):
    xr = O.rotate(np.asarray(X, np.float64), B)
    return xr.T @ xr


@pytest.mark.parametrize("S,K,B,dt", [(300, 256, 64, "f32"), (100, 320, 64, "bf16"),
                                      (5000, 128, 128, "f32"), (1, 64, 1, "f32"),
                                      (77, 1024, 1024, "bf16"), (64, 11008, 256, "bf16")])
def test_hessian_matches_oracle(S, K, B, dt):
    X = si.calibration_activations(S, K, seed=S + K)
    say(f"gptq hessian S={S} K={K} B={B} {dt}")
    if dt == "bf16":
        Xt = si.to_bf16(X).to(DEV)
        Xv = si.bf16_values(Xt)
    else:
        Xt = to_dev(X)
        Xv = X.astype(np.float64)
    H = q.qift_gptq_hessian(Xt, B)
    sync()
    Hg = H.cpu().numpy()
    Ho = oracle_hessian(Xv, B)
    assert np.array_equal(Hg, Hg.T)
    assert np.max(np.abs(Hg - Ho)) <= 1e-12 * np.max(np.abs(Ho))


def test_hessian_accumulates_and_zero():
    K, B = 256, 256
    X1 = si.calibration_activations(120, K, seed=1)
    X2 = si.calibration_activations(50, K, seed=2)
    say("gptq hessian accumulate")
    H = q.qift_gptq_hessian(to_dev(X1), B)
    q.qift_gptq_hessian(to_dev(X2), B, H=H, accumulate=True)
    sync()
    Ho = oracle_hessian(X1, B) + oracle_hessian(X2, B)
    assert np.max(np.abs(H.cpu().numpy() - Ho)) <= 1e-12 * np.max(np.abs(Ho))
    H0 = q.qift_gptq_hessian(torch.empty((0, K), device=DEV), B)
    sync()
    assert np.all(H0.cpu().numpy() == 0)


def gpu_gptq(W, X, B, kind, sdt, table=None, rule="absmax", damp=0.01):
    Xt = X if isinstance(X, torch.Tensor) else to_dev(X)
    Wt = W if isinstance(W, torch.Tensor) else to_dev(W)
    H = q.qift_gptq_hessian(Xt, B)
    codes, scales = q.qift_gptq_quantize_weights(Wt, H, B, kind, SCALE_T[sdt], table=table,
                                                 scale_rule=rule, damp=damp)
    sync()
    return O.unpack_weights(dev_u32(codes), Wt.shape[0], kind), scales.float().cpu().numpy()


CASES = [("mnz", None, "f16", "absmax"), ("pot", None, "f16", "absmax"),
         ("int4", None, "f32", "absmax"), ("lut", (0, 2, -1, -4), "f32", "absmax"),
         ("mnz", None, "f32", "mse"), ("pot", None, "f16", "mse"), ("int4", None, "f16", "mse")]


@pytest.mark.parametrize("kind,table,sdt,rule", CASES)
@pytest.mark.parametrize("N,K,S,B", [(40, 256, 300, 64), (300, 1024, 2048, 1024),
                                     (21, 768, 500, 256)])
def test_gptq_codes_match_oracle(kind, table, sdt, rule, N, K, S, B):
    W = si.weights(N, K, seed=3 * N + K)
    X = si.calibration_activations(S, K, seed=5 * S + K)
    say(f"gptq {kind} {table} {sdt} {rule} N={N} K={K} S={S} B={B}")
    cg, sg = gpu_gptq(W, X, B, kind, sdt, table, rule)
    co, so, _ = O.gptq_quantize_weights(W, X, B, kind, sdt, table, rule)
    assert np.array_equal(sg.astype(np.float32).view(np.uint32),
                          so.astype(np.float32).view(np.uint32))
    plain, _, _ = O.quantize_weights(W, B, kind, sdt, table, rule)
    assert np.any(plain != co)  # the case exercises the compensation
    assert np.array_equal(cg, co), f"{int(np.sum(cg != co))} of {co.size} codes differ"


@pytest.mark.parametrize("kind,table", [("mnz", None), ("pot", None), ("int4", None),
                                        ("lut", (1, 3, -3, -1))])
def test_identity_hessian_equals_plain_quantizer(kind, table):
    """H proportional to I passes no error on: the codes and scales are the
    GPU plain quantizer's, bit for bit (had_block 1: both read the same
    float32 weights)."""
    N, K = 50, 512
    W = si.weights(N, K, seed=91)
    say(f"gptq identity H {kind}")
    Wt = to_dev(W)
    X = to_dev(3.0 * np.eye(K, dtype=np.float32))
    H = q.qift_gptq_hessian(X, 1)
    cg, sg = q.qift_gptq_quantize_weights(Wt, H, 1, kind, torch.float16, table=table)
    cp, sp = q.qift_quantize_weights(Wt, 1, kind, torch.float16, table=table)
    sync()
    assert torch.equal(sg, sp)
    assert np.array_equal(dev_u32(cg), dev_u32(cp))


def test_dead_feature():
    N, K, S = 33, 256, 200
    W = si.weights(N, K, seed=92)
    X = si.calibration_activations(S, K, seed=93)
    X[:, [5, 100]] = 0.0
    say("gptq dead features")
    for kind, table in (("mnz", None), ("pot", None), ("int4", None), ("lut", (0, 2, -1, -4))):
        cg, sg = gpu_gptq(W, X, 1, kind, "f16", table)
        co, so, _ = O.gptq_quantize_weights(W, X, 1, kind, "f16", table)
        assert np.array_equal(cg, co), kind
        zero_code = O.quantize_weights(np.zeros((1, 64)), 1, kind, "f16", table)[0][0, 0] \
            if kind != "int4" else 0
        assert np.all(cg[:, 5] == zero_code) and np.all(cg[:, 100] == zero_code)


def test_up_proj_full_size_sampled_rows():
    """LLaMA-7B up_proj (11008 x 4096, block 4096) with 2048 calibration
    tokens: the GPU quantizes every channel; the oracle recomputes 8 sampled
    channels from its own H and factor."""
    N, K, S, B = 11008, 4096, 2048, 4096
    say("gptq up_proj full size")
    W = si.weights(N, K, seed=2024)
    X = si.calibration_activations(S, K, seed=2025)
    rows = np.array([0, 1, 15, 16, 4097, 7001, 11000, 11007])
    cg, sg = gpu_gptq(W, X, B, "mnz", "f16")
    co, so, _ = O.gptq_quantize_weights(W, X, B, "mnz", "f16", rows=rows)
    assert np.array_equal(sg[rows].astype(np.float32), so.astype(np.float32))
    assert np.array_equal(cg[rows], co)


def test_codes_lower_linear_error():
    """End to end through the W2A4 linear: on tokens from the calibration
    distribution, the error-compensated codes give a smaller output error
    against the unquantized product than the plain codes (MNZ and PoT)."""
    N, K, B, S, M = 512, 1024, 1024, 2048, 64
    W = si.weights(N, K, seed=94)
    Xall = si.calibration_activations(S + M, K, seed=95)  # one distribution
    X, Xe = Xall[:S], Xall[S:]
    ref = Xe.astype(np.float64) @ W.astype(np.float64).T
    say("gptq end to end linear")
    Wt, Xet = to_dev(W), to_dev(Xe)
    H = q.qift_gptq_hessian(to_dev(X), B)
    xq, s_a, _ = q.qift_rotate_quant_act(Xet, B)
    for kind in ("mnz", "pot"):
        errs = []
        for cs in (q.qift_quantize_weights(Wt, B, kind, torch.float16),
                   q.qift_gptq_quantize_weights(Wt, H, B, kind, torch.float16)):
            Y = q.qift_w2a4_linear(xq, s_a, cs[0], cs[1], kind, N=N)
            sync()
            errs.append(rel_l2(Y.cpu().numpy(), ref))
        say(f"  {kind}: plain {errs[0]:.4f}, compensated {errs[1]:.4f}")
        assert errs[1] < 0.9 * errs[0], (kind, errs)


def test_bfloat16_weights_and_tokens():
    N, K, S, B = 37, 512, 400, 512
    W = si.weights(N, K, seed=97)
    X = si.calibration_activations(S, K, seed=98)
    Wt, Xt = si.to_bf16(W).to(DEV), si.to_bf16(X).to(DEV)
    say("gptq bf16 weights and tokens")
    for kind, table in (("mnz", None), ("int4", None)):
        cg, sg = gpu_gptq(Wt, Xt, B, kind, "f16", table)
        co, so, _ = O.gptq_quantize_weights(si.bf16_values(Wt), si.bf16_values(Xt), B, kind,
                                            "f16", table)
        assert np.array_equal(sg.astype(np.float32), so.astype(np.float32))
        assert np.array_equal(cg, co), kind


def test_longest_k_lowers_output_error():
    """LLaMA-3.1-8B down_proj rows (K = 14336, block 1024: 224 factorization
    steps): the compensated codes give a smaller output error on the
    calibration tokens than the plain codes (the property that defines the
    method; the oracle's float64 inverse at this size is too slow for a
    test). Errors are measured by the oracle's rotation and unpacking."""
    N, K, S, B = 256, 14336, 4096, 1024
    W = si.weights(N, K, seed=99, sigma=0.015)
    X = si.calibration_activations(S, K, seed=100)
    say("gptq K=14336 output error")
    Wt, Xt = to_dev(W), si.to_bf16(X).to(DEV)
    H = q.qift_gptq_hessian(Xt, B)
    cg, sg = q.qift_gptq_quantize_weights(Wt, H, B, "pot", torch.float16)
    cp, sp = q.qift_quantize_weights(Wt, B, "pot", torch.float16)
    sync()
    wr = O.rotate(W.astype(np.float64), B)
    xr = O.rotate(si.bf16_values(Xt), B)
    errs = []
    for codes, scales in ((cp, sp), (cg, sg)):
        c = O.unpack_weights(dev_u32(codes), N, "pot")
        deq = O._kind_levels("pot")[0][c] * scales.double().cpu().numpy()[:, None]
        errs.append(float(np.sum(((wr - deq) @ xr.T) ** 2)))
    say(f"  plain {errs[0]:.4g}, compensated {errs[1]:.4g}")
    assert np.isfinite(errs[1]) and errs[1] < 0.5 * errs[0]
