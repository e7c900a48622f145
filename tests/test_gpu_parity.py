"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs.

Bar (from the method's contract): packed codes, int4 activations and int32
accumulators bit-exact when both sides see identical rotated inputs; rotated
activations within 1e-5 relative; end-to-end float32 outputs within 1e-3
relative L2, with at most 1e-4 of the codes flipped and only at rounding
near-ties. Sizes span several tiles with ragged tails; the full LLaMA shapes
are checked on sampled outputs.
"""
import numpy as np
import pytest
import torch

import bit_quantized_fwht_amd as q
from oracle import qift_oracle as O
import synth_inputs as si
from gpu_util import (DEV, say, to_dev, u32_to_dev, dev_u32, rel_l2, check_act_codes,
                      check_weight_codes, guarded, check_guard)

pytestmark = pytest.mark.gpu

SCALE_T = {"f16": torch.float16, "f32": torch.float32}


def sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# rotate + per-token int4 (qift_rotate_quant_act)
# ---------------------------------------------------------------------------

def gpu_rotate(X_t, B, want=True):
    """The rotation through the C ABI into guarded outputs (sentinel bytes
    after xq, s_a and x_rot must stay untouched)."""
    M, K = X_t.shape
    xq, gq = guarded((M, K // 2), torch.uint8)
    s_a, gs = guarded((M,), torch.float32)
    xr, gx = guarded((M, K), torch.float32) if want else (None, None)
    q.qift_rotate_quant_act(X_t, B, xq=xq, s_a=s_a, x_rot=xr)
    sync()
    check_guard(gq, "xq")
    check_guard(gs, "s_a")
    if want:
        check_guard(gx, "x_rot")
    return O.unpack_int4(xq.cpu().numpy()), s_a.cpu().numpy(), (xr.cpu().numpy() if want else None)


def test_rotate_small_linear_case():
    W, X, _ = si.small_linear_case()
    say("rotate small case M=16 K=256 B=256")
    qg, sg, xg = gpu_rotate(to_dev(X), 256)
    qo, so, xo32, xo64 = O.rotate_quant_act(X.astype(np.float64), 256)
    for r in range(16):
        row_err = np.abs(xg[r].astype(np.float64) - xo64[r])
        assert row_err.max() <= 1e-5 * np.abs(xo64[r]).max()
        assert rel_l2(xg[r], xo64[r]) <= 1e-5
    assert np.allclose(sg, so, rtol=1e-6, atol=0)
    check_act_codes(qg, qo, xo64, so)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_rotate_every_block_size(B):
    M, K = 3, max(2 * B, 256)
    X = si.activations(M, K, seed=100 + B, n_outliers=4)
    say(f"rotate M={M} K={K} B={B}")
    Xt = si.to_bf16(X).to(DEV)
    qg, sg, xg = gpu_rotate(Xt, B)
    Xv = si.bf16_values(Xt)
    qo, so, xo32, xo64 = O.rotate_quant_act(Xv, B)
    for r in range(M):
        assert np.abs(xg[r] - xo64[r]).max() <= 1e-5 * np.abs(xo64[r]).max()
    assert np.allclose(sg, so, rtol=1e-6, atol=0)
    check_act_codes(qg, qo, xo64, so)


@pytest.mark.parametrize("M,K", [(1, 64), (5, 10), (17, 256), (33, 4096), (7, 11008), (2, 14336),
                                 (3, 16384), (4, 18), (2, 2)])
def test_rotate_quant_bitexact_given_rotated_input(M, K):
    """had_block = 1 and the oracle's float32 rotated values as input: the
    quantizer must reproduce the oracle's codes and scales bit for bit."""
    B = 256 if K % 256 == 0 else 2
    X = si.activations(M, K, seed=7 * K + M, n_outliers=min(4, K // 2))
    _, _, xr32, _ = O.rotate_quant_act(X.astype(np.float64), B)
    say(f"bitexact quant M={M} K={K}")
    qg, sg, xg = gpu_rotate(to_dev(xr32), 1)
    qo, so = O.quant_sym4(xr32)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo.astype(np.int64))
    assert np.array_equal(xg.view(np.uint32), xr32.view(np.uint32))


# rows of 1, 2, 3 and 4 groups of 16 per thread (K up to 4096, 8192, 12288,
# 16384; 4112 = 257 groups leaves one thread a second group)
@pytest.mark.parametrize("M,K,B", [(3, 16, 16), (5, 256, 64), (17, 4096, 256), (2, 4096, 1024),
                                   (4, 4096, 4096), (3, 11008, 256), (2, 14336, 1024),
                                   (1, 16384, 4096), (33, 1024, 16), (5, 4112, 16),
                                   (3, 6144, 1024), (2, 8192, 4096), (2, 12288, 4096)])
def test_rotate_quant_bitexact_exact_rotation(M, K, B):
    """Integer-valued inputs with an even log2(block): every butterfly sum is
    an exact small integer and 1/sqrt(B) is a power of two, so the rotated
    values are exact on both sides and codes, scales and rotated values must
    agree bit for bit (this exercises the register-first kernel used for
    blocks of 16 and more)."""
    X = si.uniform_int4((M, K), seed=K + B + M, lo=-8, hi=8).astype(np.float32)
    X[0, :3] = 0.0
    say(f"bitexact exact-rotation M={M} K={K} B={B}")
    for dt in (torch.float32, torch.bfloat16):
        qg, sg, xg = gpu_rotate(to_dev(X, dt), B)
        qo, so, xo32, _ = O.rotate_quant_act(X.astype(np.float64), B)
        assert np.array_equal(xg.view(np.uint32), xo32.view(np.uint32))
        assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
        assert np.array_equal(qg, qo.astype(np.int64))


def test_rotate_batched_matches_single_calls():
    """One batched call over matrices of different K, block, dtype and row
    count (one outside the shared launch's conditions, one empty) gives the
    same bytes as one call per matrix."""
    cases = [(3, 4096, 4096, torch.bfloat16, False), (5, 11008, 256, torch.float32, True),
             (2, 256, 16, torch.bfloat16, True), (0, 512, 64, torch.bfloat16, False),
             (4, 10, 2, torch.float32, True), (2, 16384, 4096, torch.bfloat16, False)]
    say("rotate batched vs single")
    items, refs = [], []
    for i, (M, K, B, dt, want) in enumerate(cases):
        X = torch.from_numpy(si.activations(M, K, seed=300 + i, n_outliers=min(3, K))).to(dt).to(DEV)
        refs.append(q.qift_rotate_quant_act(X, B, want_x_rot=want))
        x_rot = torch.full((M, K), 7.0, device=DEV) if want else None
        items.append((X, B, None, None, x_rot))
    outs = q.qift_rotate_quant_act_batched(items)
    sync()
    for (xq, sa, xr), (rxq, rsa, rxr), c in zip(outs, refs, cases):
        assert torch.equal(xq, rxq), c
        assert torch.equal(sa, rsa), c
        if c[4]:
            assert torch.equal(xr, rxr), c


def test_rotate_rne_ties_and_zero_rows():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rne_ties.json")))
    row = np.array(g["row"] + [0.0] * 6, dtype=np.float32)  # pad to 16
    X = np.stack([row, np.zeros(16, np.float32), -row])
    say("rne ties")
    qg, sg, _ = gpu_rotate(to_dev(X), 1, want=False)
    assert qg[0, :10].tolist() == g["codes"]
    assert qg[2, :10].tolist() == [-c for c in g["codes"]]
    assert sg[0] == 1.0 and sg[1] == 0.0 and np.all(qg[1] == 0)


def exact_tie_rows(D, B, seed):
    """Rows z of rounding ties (half-integers times 2^e, max |z| = 7 * 2^e)
    and inputs x with x = H_B z / sqrt(B) blockwise, which float32
    butterflies map back to z exactly (every partial sum is a short dyadic
    number; 1/sqrt(B) is a power of two for even log2 B)."""
    base = np.array([7.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 6.5, -7.0, 4.5, 5.5, -3.5, -4.5,
                     -5.5, -6.5])
    rng = np.random.default_rng(seed)
    rows = []
    for e in (-3, 0, 5):
        for _ in range(3):
            rows.append(np.concatenate([rng.permutation(base) for _ in range(D // 16)]) * 2.0 ** e)
    Z = np.stack(rows)
    Hb = np.array([[(-1) ** bin(i & j).count("1") for j in range(B)] for i in range(B)], float)
    X = (Z.reshape(len(rows), D // B, B) @ Hb.T).reshape(len(rows), D) / np.sqrt(B)
    assert np.array_equal(X.astype(np.float32).astype(np.float64), X)  # exact in float32
    expect = np.rint(Z / (Z.max(axis=1, keepdims=True) / 7.0))  # numpy rint: half to even
    return X.astype(np.float32), Z, expect.astype(np.int64)


@pytest.mark.parametrize("K,B", [(64, 16), (256, 64), (512, 256), (2048, 1024)])
def test_rotate_exact_ties_after_rotation(K, B):
    """Rotated values that are exact rounding ties, through the in-lane,
    cross-lane and (B = 1024) LDS stages: codes round half to even."""
    X, Z, expect = exact_tie_rows(K, B, seed=K + B)
    say(f"rotate exact ties K={K} B={B}")
    qg, sg, xg = gpu_rotate(to_dev(X), B)
    assert np.array_equal(xg.astype(np.float64), Z)
    assert np.array_equal(sg, (Z.max(axis=1) / 7.0).astype(np.float32))
    assert np.array_equal(qg, expect)


def test_rotate_one_hot_closed_form():
    B, j, c = 4096, 1234, 2.5
    X = np.zeros((2, 2 * B), np.float32)
    X[1, B + j] = c
    say("rotate one-hot B=4096")
    qg, sg, xg = gpu_rotate(to_dev(X), B)
    popc = np.array([bin(i & j).count("1") for i in range(B)])
    expect = np.where(popc % 2 == 0, 7, -7)
    assert np.array_equal(qg[1, B:], expect) and np.all(qg[1, :B] == 0)
    assert np.all(qg[0] == 0) and sg[0] == 0


# ---------------------------------------------------------------------------
# weight quantizer (qift_quantize_weights)
# ---------------------------------------------------------------------------

def gpu_quant_weights(W_t, B, kind, sdt):
    N, K = W_t.shape
    codes, gc = guarded((q.padded_channels(N), q.code_words_per_row(K, kind)), torch.int32)
    scales, gsc = guarded((N,), SCALE_T[sdt])
    q.qift_quantize_weights(W_t, B, kind, SCALE_T[sdt], codes=codes, scales=scales)
    sync()
    check_guard(gc, "codes")
    check_guard(gsc, "scales")
    words = dev_u32(codes)
    c = O.unpack_weights(words, W_t.shape[0], kind)
    return c, scales.float().cpu().numpy(), words


@pytest.mark.parametrize("kind", ["mnz", "pot", "int4"])
@pytest.mark.parametrize("sdt", ["f16", "f32"])
@pytest.mark.parametrize("N,K", [(1, 64), (37, 256), (130, 4096), (5, 11008)])
def test_quantize_weights_bitexact_given_rotated_input(kind, sdt, N, K):
    B = 256 if K % 256 == 0 else 64
    W = si.weights(N, K, seed=N * 31 + K, sigma=0.02)
    wr32 = O.rotate(W.astype(np.float64), B).astype(np.float32)
    say(f"bitexact weights {kind} {sdt} N={N} K={K}")
    cg, sg, words = gpu_quant_weights(to_dev(wr32), 1, kind, sdt)
    co, so, _ = O.quantize_weights(wr32.astype(np.float64), 1, kind, sdt)
    assert np.array_equal(sg.astype(np.float32).view(np.uint32),
                          so.astype(np.float32).view(np.uint32))
    assert np.array_equal(cg, co)
    assert np.array_equal(words, O.pack_weights(co, kind))


@pytest.mark.parametrize("kind", ["mnz", "pot"])
def test_quantize_weights_ties_and_zero_rows(kind):
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "weight_ties.json")))[kind]
    row = np.array(g["row"] * 4, np.float32)  # 64 features
    W = np.stack([row, np.zeros(64, np.float32), -row, np.full(64, 1e-30, np.float32)])
    say(f"weight ties {kind}")
    for sdt in ("f16", "f32"):
        cg, sg, _ = gpu_quant_weights(to_dev(W), 1, kind, sdt)
        co, so, _ = O.quantize_weights(W.astype(np.float64), 1, kind, sdt)
        assert cg[0, :16].tolist() == g["codes"]
        assert np.array_equal(cg, co) and np.array_equal(sg, so.astype(np.float32))


@pytest.mark.parametrize("kind", ["mnz", "pot", "int4"])
def test_quantize_weights_rotated_small_case(kind):
    W, _, _ = si.small_linear_case()
    say(f"weights small case {kind}")
    cg, sg, _ = gpu_quant_weights(to_dev(W), 256, kind, "f32")
    co, so, wr32 = O.quantize_weights(W.astype(np.float64), 256, kind, "f32")
    assert np.allclose(sg, so, rtol=1e-6, atol=0)
    w64 = O.rotate(W.astype(np.float64), 256)
    check_weight_codes(O.code_levels(cg, kind), O.code_levels(co, kind), w64, so, kind, s_gpu=sg)


# ---------------------------------------------------------------------------
# the linear (qift_w2a4_linear): int32 bit-exact on oracle-packed inputs
# ---------------------------------------------------------------------------

def random_linear_inputs(M, K, N, kind, seed):
    qa = si.uniform_int4((M, K), seed=seed)
    codes = si.uniform_int4((N, K), seed=seed + 1) if kind == "int4" \
        else si.uniform_codes((N, K), 4, seed=seed + 1)
    s_a = si.positive_scales(M, seed + 2)
    s_w = si.positive_scales(N, seed + 3).astype(np.float16)
    return qa, codes, s_a, s_w


def run_linear(qa, codes, s_a, s_w, kind, out_dtype):
    """The linear through the C ABI into a guarded Y (sentinel bytes after
    it must stay untouched)."""
    xq = torch.from_numpy(O.pack_int4(qa)).to(DEV)
    cw = u32_to_dev(O.pack_weights(codes, kind))
    Y, gy = guarded((qa.shape[0], codes.shape[0]), out_dtype)
    q.qift_w2a4_linear(xq, to_dev(s_a), cw, to_dev(s_w.astype(np.float32), torch.float16),
                       kind, out_dtype, Y=Y)
    sync()
    check_guard(gy, "Y")
    return Y


# M <= 16: decode with K split over 4, 8 or 16 waves (by the number of K
# chunks: up to 8, 16, more) when 64-channel waves would give fewer than 512
# workgroups, else
# 64-channel waves ((2, 256, 131100): 513 workgroups, ragged N); M > 16 with
# K % 256 == 0: prefill with 64-row tiles when 128-row tiles number fewer than
# 512 (two per CU), else 128-row tiles ((1000, 256, 8200): 8 x 65 tiles,
# ragged in M and N); other K: the general prefill kernel
LIN_SHAPES = [(1, 64, 1), (1, 256, 17), (3, 320, 64), (4, 4096, 257), (8, 192, 300),
              (16, 1024, 129), (5, 2304, 40), (2, 8448, 33), (3, 3072, 4100), (2, 256, 131100),
              (17, 256, 130), (31, 128, 63), (64, 4096, 256), (129, 576, 200),
              (200, 2048, 385), (1000, 256, 8200), (1050, 256, 7300), (1, 2048, 20000)]


@pytest.mark.parametrize("kind", ["mnz", "pot", "int4"])
@pytest.mark.parametrize("M,K,N", LIN_SHAPES)
def test_linear_int32_bitexact(kind, M, K, N):
    qa, codes, s_a, s_w = random_linear_inputs(M, K, N, kind, seed=M * 1000 + K + N)
    say(f"linear i32 {kind} M={M} K={K} N={N}")
    Y = run_linear(qa, codes, s_a, s_w, kind, torch.int32).cpu().numpy()
    acc, _ = O.linear(qa, s_a, codes, s_w.astype(np.float64), kind)
    assert np.array_equal(Y.astype(np.int64), acc)


@pytest.mark.parametrize("kind", ["mnz", "pot", "int4"])
@pytest.mark.parametrize("M,K,N", [(1, 256, 33), (16, 512, 100), (40, 1024, 150), (48, 512, 256),
                                   (130, 768, 136), (33, 256, 1000), (1000, 256, 8200)])
def test_linear_float_epilogue(kind, M, K, N):
    qa, codes, s_a, s_w = random_linear_inputs(M, K, N, kind, seed=5 + M + N)
    say(f"linear f32/bf16 {kind} M={M} K={K} N={N}")
    _, y = O.linear(qa, s_a, codes, s_w.astype(np.float64), kind)
    Yf = run_linear(qa, codes, s_a, s_w, kind, torch.float32).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Yf - y) <= 4e-7 * np.abs(y) + 1e-30)
    Yb = run_linear(qa, codes, s_a, s_w, kind, torch.bfloat16).float().cpu().numpy()
    assert np.all(np.abs(Yb - y) <= 2 ** -8 * np.abs(y) + 1e-30)


@pytest.mark.parametrize("M", [7, 40])  # decode and prefill kernels
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_linear_unaligned_output(out_dtype, M):
    """An output view that starts one element into its buffer (not 16-byte
    aligned) is written element by element, with the same values."""
    K, N = 512, 256
    qa, codes, s_a, s_w = random_linear_inputs(M, K, N, "mnz", seed=77)
    say(f"linear unaligned output {out_dtype} M={M}")
    ref = run_linear(qa, codes, s_a, s_w, "mnz", out_dtype)
    xq = torch.from_numpy(O.pack_int4(qa)).to(DEV)
    cw = u32_to_dev(O.pack_weights(codes, "mnz"))
    buf = torch.full((M * N + 1,), 3, dtype=out_dtype, device=DEV)
    Y = buf[1:].view(M, N)
    q.qift_w2a4_linear(xq, to_dev(s_a), cw, to_dev(s_w.astype(np.float32), torch.float16), "mnz",
                       out_dtype, Y=Y)
    sync()
    assert torch.equal(Y, ref)
    assert buf[0].item() == 3


def test_linear_extremes_do_not_overflow():
    """All activations +-7 against all outer levels at the largest K."""
    for kind, code in (("mnz", 1), ("pot", 1), ("int4", 7)):
        M, K, N = 17, 65536, 16
        qa = np.full((M, K), 7)
        qa[1::2] = -7
        codes = np.full((N, K), code)
        s_a = np.ones(M, np.float32)
        s_w = np.ones(N, np.float16)
        say(f"linear extremes {kind}")
        for m_sub in (16, 17):  # decode and prefill kernels
            Y = run_linear(qa[:m_sub], codes, s_a[:m_sub], s_w, kind, torch.int32).cpu().numpy()
            acc, _ = O.linear(qa[:m_sub], s_a[:m_sub], codes, s_w.astype(np.float64), kind)
            assert np.array_equal(Y.astype(np.int64), acc)


def test_linear_empty_batch():
    xq = torch.empty((0, 128), dtype=torch.uint8, device=DEV)
    Y = q.qift_w2a4_linear(xq, torch.empty(0, device=DEV), torch.zeros((16, 16), dtype=torch.int32,
                           device=DEV), torch.ones(8, dtype=torch.float16, device=DEV), "mnz")
    assert Y.shape == (0, 8)


def test_quantize_weights_writes_zero_padding_channels():
    W = si.weights(20, 128, seed=2)
    say("weight padding channels")
    codes = torch.full((32, 8), -1, dtype=torch.int32, device=DEV)
    q.qift_quantize_weights(to_dev(W), 128, "mnz", torch.float16, codes=codes)
    sync()
    rows = O.untile_weight_words(dev_u32(codes), 32)
    assert np.all(rows[20:] == 0) and not np.all(rows[:20] == 0)


# ---------------------------------------------------------------------------
# end to end: quantize weights, rotate + quantize activations, linear
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["mnz", "pot", "int4"])
def test_end_to_end_small_linear_case(kind):
    W, X, _ = si.small_linear_case()
    say(f"end to end small case {kind}")
    cw, sw = q.qift_quantize_weights(to_dev(W), 256, kind, torch.float32)
    xq, s_a, _ = q.qift_rotate_quant_act(to_dev(X), 256)
    Y = q.qift_w2a4_linear(xq, s_a, cw, sw, kind, torch.float32)
    sync()
    qo, so, _, xo64 = O.rotate_quant_act(X.astype(np.float64), 256)
    co, swo, _ = O.quantize_weights(W.astype(np.float64), 256, kind, "f32")
    _, yo = O.linear(qo, so, co, swo.astype(np.float64), kind)
    assert rel_l2(Y.cpu().numpy(), yo) <= 1e-3
    check_act_codes(O.unpack_int4(xq.cpu().numpy()), qo, xo64, so)


# ---------------------------------------------------------------------------
# KV4 (qift_kv4_quant)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D,B", [(128, 128), (128, 64), (128, 32), (128, 1), (64, 64), (64, 32),
                                 (256, 256), (256, 32), (16, 16), (32, 8)])
def test_kv4_matches_oracle(D, B):
    T, H = 37, 5
    KV = si.kv(T, H, D, seed=D + B)
    KVt = si.to_bf16(KV).to(DEV)
    say(f"kv4 T={T} H={H} D={D} B={B}")
    kvq, gk = guarded((T, H, D // 2), torch.uint8)
    sc, gsc = guarded((T, H), torch.float32)
    q.qift_kv4_quant(KVt, B, kvq=kvq, scales=sc)
    sync()
    check_guard(gk, "kvq")
    check_guard(gsc, "scales")
    qo, so, xr = O.kv4_quant(si.bf16_values(KVt), B)
    qg = O.unpack_int4(kvq.cpu().numpy())
    sg = sc.cpu().numpy()
    assert np.allclose(sg, so, rtol=1e-6, atol=0)
    xo64 = O.rotate(si.bf16_values(KVt).reshape(T * H, D), B).reshape(T, H, D)
    check_act_codes(qg, qo, xo64, so)
    if B == 1:
        assert np.array_equal(qg, qo.astype(np.int64))


@pytest.mark.parametrize("D,B,dt", [(128, 128, "bf16"), (128, 32, "bf16"), (64, 64, "bf16"),
                                    (256, 64, "bf16"), (128, 64, "f32"), (32, 8, "bf16")])
def test_kv4_pair_matches_two_calls_and_oracle(D, B, dt):
    """qift_kv4_quant_kv: K and V of one layer in one call (one launch on the
    matrix-core path, bfloat16 with a block of at least 32; two otherwise)
    give exactly the codes and scales of two qift_kv4_quant calls, and the
    oracle's. T * H = 185 vectors: the last 16-vector tile of each tensor is
    partial. K's and V's codes sit back to back in one buffer, and so do
    their scales (adjacent outputs), with canaries after V's."""
    T, H = 37, 5
    cast = si.to_bf16 if dt == "bf16" else (lambda a: torch.from_numpy(a))
    Kt = cast(si.kv(T, H, D, seed=3 * D + B)).to(DEV)
    Vt = cast(si.kv(T, H, D, seed=3 * D + B + 1)).to(DEV)
    say(f"kv4 pair T={T} H={H} D={D} B={B} {dt}")
    n = T * H
    codes, gq = guarded((2 * n, D // 2), torch.uint8)
    scs, gs = guarded((2 * n,), torch.float32)
    kq, vq = codes[:n].view(T, H, D // 2), codes[n:].view(T, H, D // 2)
    ks, vs = scs[:n].view(T, H), scs[n:].view(T, H)
    q.qift_kv4_quant_kv(Kt, Vt, B, kq=kq, ks=ks, vq=vq, vs=vs)
    k1, s1 = q.qift_kv4_quant(Kt, B)
    v1, t1 = q.qift_kv4_quant(Vt, B)
    sync()
    check_guard(gq, "codes")
    check_guard(gs, "scales")
    assert torch.equal(kq, k1) and torch.equal(vq, v1)
    assert torch.equal(ks, s1) and torch.equal(vs, t1)
    for X, cq, sc in ((Kt, kq, ks), (Vt, vq, vs)):
        xv = si.bf16_values(X) if dt == "bf16" else X.cpu().numpy().astype(np.float64)
        qo, so, _ = O.kv4_quant(xv, B)
        assert np.allclose(sc.cpu().numpy(), so, rtol=1e-6, atol=0)
        xo64 = O.rotate(xv.reshape(T * H, D), B).reshape(T, H, D)
        check_act_codes(O.unpack_int4(cq.cpu().numpy()), qo, xo64, so)


@pytest.mark.parametrize("D", [16, 64, 256])
def test_kv4_exact_ties_after_rotation(D):
    """Head vectors whose rotated values are exact rounding ties: z holds
    half-integers times 2^e with max |z| = 7 * 2^e, and the input is
    x = H_D z / sqrt(D), which the float32 butterflies map back to z exactly
    (every partial sum is a short dyadic number; 1/sqrt(D) is a power of two
    for D = 16, 64, 256). So s = 2^e exactly and x'/s are the ties, which
    round half to even; D = 64 and 256 run the cross-lane stages."""
    X, Z, expect = exact_tie_rows(D, D, seed=D)
    KV = X.reshape(len(Z), 1, D)
    say(f"kv4 exact ties D={D}")
    kvq, sc = q.qift_kv4_quant(to_dev(KV), D)
    sync()
    qg = O.unpack_int4(kvq.cpu().numpy()).reshape(len(Z), D)
    assert np.array_equal(qg, expect)
    assert np.array_equal(sc.cpu().numpy().reshape(-1), Z.max(axis=1) / 7.0)
    qo, so, _ = O.kv4_quant(KV.astype(np.float64), D)
    assert np.array_equal(qg, qo.reshape(len(Z), D).astype(np.int64))


def sparse_tie_rows_bf16(D, B, seed):
    """Head vectors z of rounding ties (half-integers times 2^e, max |z| =
    7 * 2^e) with at most three nonzeros per block of B, and x = H_B z /
    sqrt(B) blockwise: every x is a sum of at most three such values, a
    number of at most 6 significant bits, so x is exact in bfloat16 and
    the matrix-core transform (bfloat16 products, float32 sums) returns z
    exactly (1/sqrt(B) is a power of two for even log2 B)."""
    rng = np.random.default_rng(seed)
    ties = np.array([0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5])
    Hb = np.array([[(-1) ** bin(i & j).count("1") for j in range(B)] for i in range(B)], float)
    rows = []
    for e in (-3, 0, 5):
        for _ in range(4):
            z = np.zeros(D)
            for b in range(D // B):
                pos = rng.choice(B, 3, replace=False)
                z[b * B + pos] = rng.choice(ties, 3) * rng.choice([-1.0, 1.0], 3)
            z[rng.integers(D)] = 7.0 * rng.choice([-1.0, 1.0])
            rows.append(z * 2.0 ** e)
    Z = np.stack(rows)
    X = (Z.reshape(len(rows), D // B, B) @ Hb.T).reshape(len(rows), D) / np.sqrt(B)
    assert np.array_equal(si.bf16_values(si.to_bf16(X)), X)  # exact in bfloat16
    expect = np.rint(Z / (np.abs(Z).max(axis=1, keepdims=True) / 7.0))  # half to even
    return X, Z, expect.astype(np.int64)


@pytest.mark.parametrize("D,B", [(64, 64), (128, 64), (256, 256), (256, 64)])
def test_kv4_exact_ties_bf16_matrix_core(D, B):
    """bfloat16 head vectors with a block of at least 32 take the matrix-core
    transform; exact ties after it round half to even, as the oracle does."""
    X, Z, expect = sparse_tie_rows_bf16(D, B, seed=D + B)
    KV = si.to_bf16(X.reshape(len(Z), 1, D)).to(DEV)
    say(f"kv4 bf16 exact ties D={D} B={B}")
    kvq, sc = q.qift_kv4_quant(KV, B)
    sync()
    qg = O.unpack_int4(kvq.cpu().numpy()).reshape(len(Z), D)
    assert np.array_equal(qg, expect)
    assert np.array_equal(sc.cpu().numpy().reshape(-1), np.abs(Z).max(axis=1) / 7.0)
    qo, so, _ = O.kv4_quant(X.reshape(len(Z), 1, D), B)
    assert np.array_equal(qg, qo.reshape(len(Z), D).astype(np.int64))


def test_kv4_bitexact_given_rotated_input():
    T, H, D = 9, 4, 128
    KV = si.kv(T, H, D, seed=3)
    _, _, xr32 = O.kv4_quant(KV.astype(np.float64), 128)
    say("kv4 bitexact")
    kvq, sc = q.qift_kv4_quant(to_dev(xr32), 1)
    sync()
    qo, so, _ = O.kv4_quant(xr32.astype(np.float64), 1)
    assert np.array_equal(O.unpack_int4(kvq.cpu().numpy()), qo.astype(np.int64))
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), so.view(np.uint32))


# ---------------------------------------------------------------------------
# level tables (QIFT_LEVELS_LUT) and the searched scale
# ---------------------------------------------------------------------------

TABLES = [(-2, -1, 0, 1), (3, 10, -3, -10), (15, -15, 1, -1)]


def run_linear_lut(qa, codes, s_a, s_w, table, out_dtype):
    xq = torch.from_numpy(O.pack_int4(qa)).to(DEV)
    cw = u32_to_dev(O.pack_weights(codes, "lut"))
    Y, gy = guarded((qa.shape[0], codes.shape[0]), out_dtype)
    q.qift_w2a4_linear(xq, to_dev(s_a), cw, to_dev(s_w.astype(np.float32), torch.float16),
                       "lut", out_dtype, Y=Y, table=table)
    sync()
    check_guard(gy, "Y")
    return Y


# decode with K split over 4, 16 and 8 waves, 64-channel decode waves, prefill
# with 64- and 128-row tiles, the general prefill kernel (K % 256 != 0)
LUT_SHAPES = [(1, 256, 17), (4, 4096, 257), (3, 3072, 4100), (2, 256, 131100), (17, 256, 130),
              (64, 4096, 256), (1000, 256, 8200), (129, 576, 200)]


@pytest.mark.parametrize("table", TABLES)
@pytest.mark.parametrize("M,K,N", LUT_SHAPES)
def test_lut_linear_int32_bitexact(table, M, K, N):
    qa, codes, s_a, s_w = random_linear_inputs(M, K, N, "lut", seed=M * 7 + K + N)
    say(f"linear lut {table} M={M} K={K} N={N}")
    Y = run_linear_lut(qa, codes, s_a, s_w, table, torch.int32).cpu().numpy()
    acc, _ = O.linear(qa, s_a, codes, s_w.astype(np.float64), "lut", table)
    assert np.array_equal(Y.astype(np.int64), acc)


@pytest.mark.parametrize("M", [3, 40])  # decode and prefill kernels
def test_lut_linear_float_epilogue(M):
    K, N, table = 512, 200, (3, 10, -3, -10)
    qa, codes, s_a, s_w = random_linear_inputs(M, K, N, "lut", seed=61 + M)
    say(f"linear lut float M={M}")
    _, y = O.linear(qa, s_a, codes, s_w.astype(np.float64), "lut", table)
    Yf = run_linear_lut(qa, codes, s_a, s_w, table, torch.float32).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Yf - y) <= 4e-7 * np.abs(y) + 1e-30)


def test_lut_extremes_do_not_overflow():
    """All activations +-7 against levels +-15 at the largest K."""
    M, K, N = 17, 65536, 16
    qa = np.full((M, K), 7)
    qa[1::2] = -7
    codes = np.zeros((N, K), np.int64)
    codes[1::2] = 1
    table = (15, -15, 1, -1)
    s_a = np.ones(M, np.float32)
    s_w = np.ones(N, np.float16)
    say("linear lut extremes")
    for m_sub in (16, 17):
        Y = run_linear_lut(qa[:m_sub], codes, s_a[:m_sub], s_w, table, torch.int32).cpu().numpy()
        acc, _ = O.linear(qa[:m_sub], s_a[:m_sub], codes, s_w.astype(np.float64), "lut", table)
        assert np.array_equal(Y.astype(np.int64), acc)


@pytest.mark.parametrize("kind,table", [("mnz", (1, 3, -3, -1)), ("pot", (1, 4, -1, -4))])
def test_lut_decodes_mnz_and_pot_codes(kind, table):
    """MNZ (PoT) codes read through the table {1, 3, -3, -1} ({1, 4, -1, -4})
    give the MNZ (PoT) integer sums."""
    for M, K, N in ((2, 1024, 100), (48, 512, 256)):
        qa, codes, s_a, s_w = random_linear_inputs(M, K, N, kind, seed=71 + M)
        say(f"lut decodes {kind} M={M}")
        a = run_linear(qa, codes, s_a, s_w, kind, torch.int32)
        b = run_linear_lut(qa, codes, s_a, s_w, table, torch.int32)
        assert torch.equal(a, b)


def test_lut_in_grouped_launch():
    shapes = [(1, 4096, 1000, "mnz", None), (4, 512, 300, "lut", (3, 10, -3, -10)),
              (16, 256, 64, "lut", (-2, -1, 0, 1)), (2, 1024, 200, "pot", None)]
    items, refs = [], []
    for i, (M, K, N, kind, table) in enumerate(shapes):
        qa, codes, s_a, s_w = random_linear_inputs(M, K, N, kind, seed=950 + i)
        Y = torch.full((M, N), -1, dtype=torch.int32, device=DEV)
        items.append(dict(xq=torch.from_numpy(O.pack_int4(qa)).to(DEV), s_a=to_dev(s_a),
                          codes=u32_to_dev(O.pack_weights(codes, kind)),
                          scales=to_dev(s_w.astype(np.float32), torch.float16), Y=Y, levels=kind,
                          table=table))
        refs.append(O.linear(qa, s_a, codes, s_w.astype(np.float64), kind, table)[0])
    say("grouped linear with level tables")
    grp = q.LinearGroup(items, scale_dtype=torch.float16, y_dtype=torch.int32)
    grp.run()
    sync()
    for it, ref in zip(items, refs):
        assert np.array_equal(it["Y"].cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("table", TABLES + [(0, 5, -5, 1), (2, 2, -2, -2)])
@pytest.mark.parametrize("sdt", ["f16", "f32"])
def test_lut_quantizer_bitexact_given_rotated_input(table, sdt):
    N, K = 37, 512
    W = si.weights(N, K, seed=81, sigma=0.02)
    wr32 = O.rotate(W.astype(np.float64), 256).astype(np.float32)
    # exact midpoints between levels (ties) in the first row, a zero row
    s0 = O.absmax_scales(wr32[:1], "lut", sdt, table).astype(np.float64)[0]
    mids = np.array([(a + b) / 2 * s0 for a in table for b in table], np.float32)
    wr32[0, :mids.size] = mids
    wr32[0, mids.size] = max(abs(v) for v in table) * s0  # keeps the absmax
    wr32[1] = 0.0
    say(f"lut weights {table} {sdt}")
    codes, scales = q.qift_quantize_weights(to_dev(wr32), 1, "lut", SCALE_T[sdt], table=table)
    sync()
    co, so, _ = O.quantize_weights(wr32.astype(np.float64), 1, "lut", sdt, table)
    assert np.array_equal(scales.float().cpu().numpy().view(np.uint32),
                          so.astype(np.float32).view(np.uint32))
    assert np.array_equal(O.unpack_weights(dev_u32(codes), N, "lut"), co)


@pytest.mark.parametrize("kind,table", [("mnz", None), ("pot", None), ("int4", None),
                                        ("lut", (-2, -1, 0, 1)), ("lut", (3, 10, -3, -10))])
@pytest.mark.parametrize("sdt", ["f16", "f32"])
def test_mse_scale_quantizer(kind, table, sdt):
    """Searched scale: the GPU's choice is the oracle's least-squares
    candidate (or one whose float64 error ties it to 1e-12), and the codes are
    exactly the oracle's nearest codes for the GPU's scale."""
    N, K = 24, 1024
    W = si.heavy_tailed_weights(N, K, seed=83)
    W[3] = 0.0
    wr32 = O.rotate(W.astype(np.float64), 1024).astype(np.float32)
    say(f"mse scale {kind} {table} {sdt}")
    codes, scales = q.qift_quantize_weights(to_dev(wr32), 1, kind, SCALE_T[sdt], table=table,
                                            scale_rule="mse")
    sync()
    sg = scales.cpu().numpy()
    co, so, _ = O.quantize_weights(wr32.astype(np.float64), 1, kind, sdt, table, "mse")
    cg = O.unpack_weights(dev_u32(codes), N, kind)
    cand = O.scale_candidates(wr32, kind, sdt, table)
    levels = (O.real_levels(kind) if kind in ("mnz", "pot") else
              np.array(table, np.float64) if kind == "lut" else None)

    def sq_error(n, codes_n, s):  # the row's squared error for the given codes and scale
        lv = codes_n.astype(np.float64) if kind == "int4" else levels[codes_n]
        d = wr32[n].astype(np.float64) - lv * float(s)
        return float(np.sum(d * d))

    for n in range(N):
        assert sg[n] in cand[n]
        if sg[n] == so[n]:
            assert np.array_equal(cg[n], co[n]), n
            continue
        # a float64 near-tie between two candidates: the GPU's codes must be
        # nearest levels for its scale (checked here by brute force) and its
        # error must tie the oracle's best
        s = np.float64(sg[n])
        w = wr32[n].astype(np.float64)
        if kind == "int4":
            assert np.all(np.abs(w - cg[n] * s) <= 0.5 * s * (1 + 1e-9) + (np.abs(cg[n]) == 7) * np.inf)
        else:
            dist = np.abs(w[:, None] - levels[None, :] * s)
            assert np.all(dist[np.arange(K), cg[n]] <= dist.min(axis=1))
        eg, eo = sq_error(n, cg[n], sg[n]), sq_error(n, co[n], so[n])
        assert eg <= eo * (1 + 1e-12), (n, sg[n], so[n], eg, eo)


# ---------------------------------------------------------------------------
# decode attention over the KV4 cache (qift_kv4_attention_decode)
# ---------------------------------------------------------------------------

def attention_inputs(S, T, H, D, seed):
    rng = np.random.default_rng(seed)
    qv = rng.standard_normal((S, H, D)).astype(np.float32)
    kc = si.uniform_int4((S * T * H, D), seed=seed + 1).reshape(S, T, H, D)
    vc = si.uniform_int4((S * T * H, D), seed=seed + 2).reshape(S, T, H, D)
    ks = si.positive_scales(S * T * H, seed + 3, lo=0.01, hi=0.1).reshape(S, T, H).astype(np.float32)
    vs = si.positive_scales(S * T * H, seed + 4, lo=0.01, hi=1.0).reshape(S, T, H).astype(np.float32)
    return qv, kc, ks, vc, vs


def run_attention(qv, kc, ks, vc, vs, B, scale, q_dtype=torch.float32, out_dtype=torch.float32):
    S, T, H, D = kc.shape
    pack = lambda c: torch.from_numpy(O.pack_int4(c.reshape(-1, D)).reshape(S, T, H, D // 2)).to(DEV)
    out = q.qift_kv4_attention_decode(to_dev(qv).to(q_dtype), pack(kc), to_dev(ks), pack(vc),
                                      to_dev(vs), B, scale, out_dtype=out_dtype)
    sync()
    return out.float().cpu().numpy().astype(np.float64)


def check_attention(got, ref, tol):
    err = np.abs(got - ref).max()
    assert err <= tol * np.abs(ref).max(), (err, np.abs(ref).max())


# (1, 3000, 2) and (1, 8192, 1) split each head into 94 and 256 runs of 32
# tokens: the merge then takes its runs in chunks of 64, the last one ragged
@pytest.mark.parametrize("S,T,H,B", [(1, 1, 1, 128), (2, 37, 3, 128), (1, 16, 32, 128),
                                     (3, 100, 32, 64), (1, 1000, 64, 128), (2, 513, 5, 1),
                                     (1, 4096, 32, 128), (1, 3000, 2, 128), (1, 8192, 1, 64)])
def test_kv4_attention(S, T, H, B):
    D = 128
    qv, kc, ks, vc, vs = attention_inputs(S, T, H, D, seed=S * 100 + T + H)
    say(f"kv4 attention S={S} T={T} H={H} B={B}")
    got = run_attention(qv, kc, ks, vc, vs, B, 1 / np.sqrt(D))
    ref = O.kv4_attention_decode(qv.astype(np.float64), kc, ks, vc, vs, B, 1 / np.sqrt(D))
    check_attention(got, ref, 2e-5)


def test_kv4_attention_peaked_and_bf16():
    """A large softmax scale (a few tokens carry all the weight) stays stable;
    bfloat16 query and output."""
    S, T, H, D = 2, 300, 8, 128
    qv, kc, ks, vc, vs = attention_inputs(S, T, H, D, seed=7)
    say("kv4 attention peaked / bf16")
    got = run_attention(qv, kc, ks, vc, vs, 128, 4.0)
    ref = O.kv4_attention_decode(qv.astype(np.float64), kc, ks, vc, vs, 128, 4.0)
    check_attention(got, ref, 5e-5)
    qb = si.bf16_values(torch.from_numpy(qv).to(torch.bfloat16))  # rounded on the host
    gotb = run_attention(qv, kc, ks, vc, vs, 128, 0.0884, torch.bfloat16, torch.bfloat16)
    refb = O.kv4_attention_decode(qb, kc, ks, vc, vs, 128, 0.0884)
    check_attention(gotb, refb, 2 ** -7)


def test_kv4_attention_on_a_quantized_cache():
    """K and V [4096, 32, 128] quantized by the oracle's KV4 (rotated, block
    128), attention by the GPU against the oracle on those codes, and against
    plain float64 attention on the unquantized K and V (reported bound)."""
    T, H, D = 4096, 32, 128
    K = si.kv(T, H, D, seed=31)
    V = si.kv(T, H, D, seed=32)
    qv = np.random.default_rng(33).standard_normal((1, H, D)).astype(np.float32)
    kc, ksc, _ = O.kv4_quant(K.astype(np.float64), 128)
    vc, vsc, _ = O.kv4_quant(V.astype(np.float64), 128)
    say("kv4 attention on a KV4 cache [4096, 32, 128]")
    got = run_attention(qv, kc[None], ksc[None], vc[None], vsc[None], 128, 1 / np.sqrt(D))
    ref = O.kv4_attention_decode(qv.astype(np.float64), kc[None], ksc[None], vc[None], vsc[None],
                                 128, 1 / np.sqrt(D))
    check_attention(got, ref, 2e-5)


# ---------------------------------------------------------------------------
# HIP graph capture of the library's launches
# ---------------------------------------------------------------------------

def test_calls_replay_from_a_hip_graph():
    """Rotation, a single decode call, a prefill call, a grouped launch and
    decode attention captured in one HIP graph: every replay (with eager work
    and synchronizations between replays) equals the eager results."""
    M1, M2, K, N = 2, 40, 1024, 200
    qa1, codes, s_a1, s_w = random_linear_inputs(M1, K, N, "mnz", seed=501)
    X = to_dev(si.activations(M2, K, seed=502))
    cw = u32_to_dev(O.pack_weights(codes, "mnz"))
    sw = to_dev(s_w.astype(np.float32), torch.float16)
    xq1 = torch.from_numpy(O.pack_int4(qa1)).to(DEV)
    sa1 = to_dev(s_a1)
    xq2 = torch.empty((M2, K // 2), dtype=torch.uint8, device=DEV)
    sa2 = torch.empty((M2,), dtype=torch.float32, device=DEV)
    Y1 = torch.empty((M1, N), dtype=torch.bfloat16, device=DEV)
    Y2 = torch.empty((M2, N), dtype=torch.float32, device=DEV)
    Yg = torch.empty((M1, N), dtype=torch.int32, device=DEV)
    grp = q.LinearGroup([dict(xq=xq1, s_a=sa1, codes=cw, scales=sw, Y=Yg, levels="mnz")],
                        scale_dtype=torch.float16, y_dtype=torch.int32)
    qv, kc, ks, vc, vs = attention_inputs(1, 300, 4, 128, seed=503)
    kq = torch.from_numpy(O.pack_int4(kc.reshape(-1, 128)).reshape(1, 300, 4, 64)).to(DEV)
    vq = torch.from_numpy(O.pack_int4(vc.reshape(-1, 128)).reshape(1, 300, 4, 64)).to(DEV)
    qt, kst, vst = to_dev(qv), to_dev(ks), to_dev(vs)
    ao = torch.empty((1, 4, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty((q.qift_kv4_attention_workspace_bytes(1, 300, 4, 128),), dtype=torch.uint8,
                     device=DEV)

    def work():
        q.qift_rotate_quant_act(X, 1024, xq=xq2, s_a=sa2)
        q.qift_w2a4_linear(xq2, sa2, cw, sw, "mnz", Y=Y2)
        q.qift_w2a4_linear(xq1, sa1, cw, sw, "mnz", Y=Y1)
        grp.run()
        q.qift_kv4_attention_decode(qt, kq, kst, vq, vst, 128, out=ao, workspace=ws)

    outs = (xq2, sa2, Y2, Y1, Yg, ao)
    say("graph capture")
    work()
    sync()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    sync()
    for rep in range(3):
        for o in outs:
            o.zero_()
        Y2.add_(1.0)  # eager work between replays
        sync()
        g.replay()
        sync()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), rep


# ---------------------------------------------------------------------------
# grouped launch == single calls
# ---------------------------------------------------------------------------

def test_grouped_matches_single_calls():
    rng_shapes = [(1, 4096, 4096, "mnz"), (4, 11008, 4096, "mnz"), (8, 4096, 1000, "pot"),
                  (16, 256, 300, "int4"), (3, 64, 17, "mnz"), (0, 128, 64, "mnz"),
                  (2, 14336, 512, "pot")]
    items, refs = [], []
    for i, (M, K, N, kind) in enumerate(rng_shapes):
        qa, codes, s_a, s_w = random_linear_inputs(M, K, N, kind, seed=900 + i)
        xq = torch.from_numpy(O.pack_int4(qa)).to(DEV)
        cw = u32_to_dev(O.pack_weights(codes, kind))
        sa = to_dev(s_a)
        swt = to_dev(s_w.astype(np.float32), torch.float16)
        Y = torch.full((M, N), -1, dtype=torch.int32, device=DEV)
        items.append(dict(xq=xq, s_a=sa, codes=cw, scales=swt, Y=Y, levels=kind))
        refs.append(O.linear(qa, s_a, codes, s_w.astype(np.float64), kind)[0])
    say("grouped linear")
    grp = q.LinearGroup(items, scale_dtype=torch.float16, y_dtype=torch.int32)
    for rep in range(3):
        for it in items:
            it["Y"].fill_(-1)
        grp.run()
        sync()
        for it, ref in zip(items, refs):
            assert np.array_equal(it["Y"].cpu().numpy().astype(np.int64), ref)


# ---------------------------------------------------------------------------
# full LLaMA shapes, sampled
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N,kind", [
    (1, 4096, 11008, "mnz"), (8, 11008, 4096, "mnz"), (4, 4096, 4096, "mnz"),
    (1, 14336, 4096, "pot"), (16, 4096, 11008, "int4"),
    (2048, 4096, 11008, "mnz"), (2048, 11008, 4096, "mnz"), (4096, 4096, 1024, "pot"),
    (4096, 14336, 4096, "pot"),
])
def test_full_shape_linear_sampled(M, K, N, kind):
    """Oracle-packed random codes and activations at the full shapes; the
    oracle computes a sample of rows (all columns) and a sample of columns
    (all rows) exactly."""
    rng = np.random.default_rng(M + K + N)
    qa = si.uniform_int4((M, K), seed=K + 1)
    codes = si.uniform_int4((N, K), seed=N + 2) if kind == "int4" \
        else si.uniform_codes((N, K), 4, seed=N + 2)
    s_a = si.positive_scales(M, 3)
    s_w = si.positive_scales(N, 4).astype(np.float16)
    say(f"full shape linear {kind} M={M} K={K} N={N}")
    Y = run_linear(qa, codes, s_a, s_w, kind, torch.int32).cpu().numpy().astype(np.int64)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 24), replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, 24), replace=False)]))
    acc_r, _ = O.linear(qa[rows], s_a[rows], codes, s_w.astype(np.float64), kind)
    assert np.array_equal(Y[rows], acc_r)
    acc_c, _ = O.linear(qa, s_a, codes[cols], s_w[cols].astype(np.float64), kind)
    assert np.array_equal(Y[:, cols], acc_c)


@pytest.mark.parametrize("N,K,B,kind,sigma", [(11008, 4096, 4096, "mnz", 0.02),
                                               (4096, 11008, 256, "mnz", 0.02),
                                               (4096, 14336, 1024, "pot", 0.015),
                                               (1024, 4096, 4096, "int4", 0.02)])
def test_full_shape_weight_quantizer_sampled(N, K, B, kind, sigma):
    W_t = si.device_weights(N, K, seed=17, sigma=sigma, device=DEV)
    say(f"full shape weights {kind} N={N} K={K} B={B}")
    cg_t, sg_t = q.qift_quantize_weights(W_t, B, kind, torch.float16)
    sync()
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(1).choice(N, 30, replace=False)]))
    Wr = W_t[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    co, so, _ = O.quantize_weights(Wr, B, kind, "f16")
    cg = O.unpack_weights(dev_u32(cg_t), N, kind)[rows]
    sg = sg_t.float().cpu().numpy()[rows]
    so32 = so.astype(np.float32)
    assert np.all(np.abs(sg - so32) <= 2 ** -10 * so32)  # at most one float16 ulp
    check_weight_codes(O.code_levels(cg, kind), O.code_levels(co, kind), O.rotate(Wr, B), so,
                       kind, s_gpu=sg)


def test_full_shape_kv4_sampled():
    T, H, D = 4096, 32, 128
    KV_t = si.device_kv(T, H, D, seed=5, device=DEV)
    say("full shape kv4 [4096, 32, 128]")
    kvq, sc = q.qift_kv4_quant(KV_t, 128)
    sync()
    ts = np.random.default_rng(2).choice(T, 64, replace=False)
    sub = KV_t[torch.from_numpy(ts).to(DEV)].float().cpu().numpy().astype(np.float64)
    qo, so, _ = O.kv4_quant(sub, 128)
    qg = O.unpack_int4(kvq.cpu().numpy()[ts])
    assert np.allclose(sc.cpu().numpy()[ts], so, rtol=1e-6, atol=0)
    xo64 = O.rotate(sub.reshape(-1, D), 128).reshape(sub.shape)
    check_act_codes(qg, qo, xo64, so)


def test_full_shape_end_to_end_prefill():
    """LLaMA-7B up_proj at M=2048: GPU weights + activations + GEMM against
    the oracle on sampled tokens and channels (rel L2 <= 1e-3)."""
    M, K, N, B = 2048, 4096, 11008, 4096
    W_t = si.device_weights(N, K, seed=23, sigma=0.02, device=DEV)
    X_t = si.device_activations(M, K, seed=24, device=DEV)
    say("full shape end to end prefill")
    cw, sw = q.qift_quantize_weights(W_t, B, "mnz", torch.float16)
    xq, s_a, _ = q.qift_rotate_quant_act(X_t, B)
    Y = q.qift_w2a4_linear(xq, s_a, cw, sw, "mnz", torch.float32)
    sync()
    rows = np.random.default_rng(3).choice(M, 8, replace=False)
    cols = np.random.default_rng(4).choice(N, 256, replace=False)
    Xs = X_t[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    Ws = W_t[torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
    qo, so, _, xo64 = O.rotate_quant_act(Xs, B)
    co, swo, _ = O.quantize_weights(Ws, B, "mnz", "f16")
    _, yo = O.linear(qo, so, co, swo.astype(np.float64), "mnz")
    yg = Y.cpu().numpy()[np.ix_(rows, cols)]
    assert rel_l2(yg, yo) <= 1e-3
