"""The allocation-free decode attention (qift_kv4_attention_decode_noalloc)
against the workspace entry point (qift_kv4_attention_decode), both through
the C ABI, and both against the CPU oracle.

The two run the same kernels on the same inputs and differ only in where the
partial results live (the library's fixed per-GPU array instead of a
caller-owned workspace), so their outputs must be identical bit for bit; the
oracle bar is that of decode attention (2e-5 of the largest output). Two
calls in a row, the second smaller, so the second reads no stale partial
results of the first.
"""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_fwht_amd as q
from oracle import qift_oracle as O
import synth_inputs as si
from gpu_util import DEV, say, to_dev, guarded, check_guard

pytestmark = pytest.mark.gpu


def cache(S, T, H, D, seed):
    rng = np.random.default_rng(seed)
    qv = rng.standard_normal((S, H, D)).astype(np.float32)
    kc = si.uniform_int4((S * T * H, D), seed=seed + 1)
    vc = si.uniform_int4((S * T * H, D), seed=seed + 2)
    ks = si.positive_scales(S * T * H, seed + 3, lo=0.01, hi=0.1).astype(np.float32)
    vs = si.positive_scales(S * T * H, seed + 4, lo=0.01, hi=1.0).astype(np.float32)
    return (qv, kc.reshape(S, T, H, D), ks.reshape(S, T, H), vc.reshape(S, T, H, D),
            vs.reshape(S, T, H))


def test_noalloc_matches_workspace_entry_point():
    D, B = 128, 128
    # the second call is smaller than the first (fewer sequences, tokens, heads)
    for S, T, H in ((4, 1024, 32), (1, 300, 5)):
        qv, kc, ks, vc, vs = cache(S, T, H, D, seed=S * 1000 + T + H)
        need = q.qift_kv4_attention_workspace_bytes(S, T, H, D)
        assert need <= q.QIFT_ATTENTION_SCRATCH_BYTES
        pack = lambda c: torch.from_numpy(O.pack_int4(c.reshape(-1, D)).reshape(S, T, H, D // 2)).to(DEV)
        qt, kq, kst, vq, vst = to_dev(qv), pack(kc), to_dev(ks), pack(vc), to_dev(vs)
        scale = 1.0 / np.sqrt(D)
        say(f"noalloc attention S={S} T={T} H={H} (partials {need} bytes)")
        ref = q.qift_kv4_attention_decode(qt, kq, kst, vq, vst, B, scale)
        out, g = guarded((S, H, D), torch.float32)
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = q._C.qift_kv4_attention_decode_noalloc(
            ctypes.c_void_p(qt.data_ptr()), q.QIFT_F32, S, T, H, D, B,
            ctypes.c_void_p(kq.data_ptr()), ctypes.c_void_p(kst.data_ptr()),
            ctypes.c_void_p(vq.data_ptr()), ctypes.c_void_p(vst.data_ptr()), float(scale),
            ctypes.c_void_p(out.data_ptr()), q.QIFT_F32, stream)
        assert st == q.QIFT_OK, q.last_error()
        torch.cuda.synchronize()
        check_guard(g, "out")
        assert torch.equal(out, ref)
        o = O.kv4_attention_decode(qv.astype(np.float64), kc, ks, vc, vs, B, scale)
        got = out.cpu().numpy().astype(np.float64)
        assert np.abs(got - o).max() <= 2e-5 * np.abs(o).max()


def test_noalloc_rejects_partials_beyond_the_array():
    """Too many (sequence, head) pairs for the fixed array: rejected with
    QIFT_ERR_UNSUPPORTED before anything runs; the output stays untouched."""
    S, T, H, D = 600, 64, 64, 128
    assert q.qift_kv4_attention_workspace_bytes(S, T, H, D) > q.QIFT_ATTENTION_SCRATCH_BYTES
    qt = torch.zeros((S, H, D), device=DEV)
    kq = torch.zeros((S, T, H, D // 2), dtype=torch.uint8, device=DEV)
    ks = torch.ones((S, T, H), device=DEV)
    out = torch.full((S, H, D), 7.0, device=DEV)
    with pytest.raises(q.QiftError, match="exceed"):
        q.qift_kv4_attention_decode_noalloc(qt, kq, ks, kq, ks, 128, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
