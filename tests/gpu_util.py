"""Helpers shared by the GPU parity tests (comparison rules only; all
expected values come from the CPU oracle)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def u32_to_dev(words: np.ndarray):
    """uint32 words -> int32 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(DEV)


def dev_u32(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    d = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (d if d > 0 else 1.0))


def check_act_codes(q_gpu, q_orc, x_rot64, s_a, frac=1e-4):
    """GPU and oracle int4 codes from independently rotated inputs: every
    mismatch must be +-1 and sit at a rounding near-tie
    (|x'/s - (k + 1/2)| < 1e-4); at most `frac` of the codes may differ."""
    q_gpu = np.asarray(q_gpu, np.int64)
    q_orc = np.asarray(q_orc, np.int64)
    diff = q_gpu != q_orc
    n_bad = int(diff.sum())
    if n_bad == 0:
        return 0
    assert np.all(np.abs(q_gpu - q_orc)[diff] == 1), "code mismatch larger than 1"
    s = np.asarray(s_a, np.float64).reshape(-1, *([1] * (x_rot64.ndim - 1)))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s > 0, x_rot64 / s, 0.0)
    frac_part = np.abs(np.abs(ratio) - np.floor(np.abs(ratio)) - 0.5)
    # a clamp at 7 is also a tie when |x'/s| is within rounding of 7.5
    assert np.all(frac_part[diff] < 1e-4), "code mismatch away from a rounding tie"
    assert n_bad <= max(1, frac * q_orc.size), f"{n_bad} of {q_orc.size} codes flipped"
    return n_bad


def check_weight_codes(lv_gpu, lv_orc, w_rot64, s, kind, frac=1e-4, s_gpu=None):
    """Weight levels from independently rotated weights: mismatches must be
    adjacent levels at a threshold near-tie (widened by any difference of the
    two stored scales); at most `frac` may differ."""
    lv_gpu = np.asarray(lv_gpu, np.int64)
    lv_orc = np.asarray(lv_orc, np.int64)
    diff = lv_gpu != lv_orc
    n_bad = int(diff.sum())
    if n_bad == 0:
        return 0
    s = np.asarray(s, np.float64)[:, None]
    ds = np.zeros_like(s) if s_gpu is None else np.abs(np.asarray(s_gpu, np.float64)[:, None] - s)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel_ds = np.where(s > 0, ds / s, 0.0)
    a = np.abs(w_rot64)
    if kind == "int4":
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(s > 0, a / s, 0)
        near = np.abs(r - np.floor(r) - 0.5) < 1e-4 + 8 * rel_ds
        assert np.all(np.abs(lv_gpu - lv_orc)[diff] == 1)
    else:
        thr = {"mnz": 1.0, "pot": 2.5}[kind]
        near = (np.abs(a - thr * s) <= (1e-5 + 2 * rel_ds) * thr * s) | (a <= 1e-6 * s)
    assert np.all(near[diff]), "weight code mismatch away from a threshold"
    assert n_bad <= max(1, frac * lv_orc.size), f"{n_bad} of {lv_orc.size} weight codes flipped"
    return n_bad


# ---------------------------------------------------------------------------
# guarded output buffers: sentinel bytes before and after every output
# ---------------------------------------------------------------------------

CANARY_ELEMS = 64
CANARY_BYTE = 0xA7


def guarded(shape, dtype, offset=0):
    """An output tensor of ``shape`` placed ``offset`` elements into a device
    buffer that has CANARY_ELEMS more elements after it; every byte of the
    buffer starts as CANARY_BYTE. Returns (view, guard) for check_guard."""
    n = int(np.prod(shape)) if len(shape) else 1
    buf = torch.empty(offset + n + CANARY_ELEMS, dtype=dtype, device=DEV)
    buf.view(torch.uint8).fill_(CANARY_BYTE)
    return buf[offset:offset + n].view(shape), (buf, offset, n)


def check_guard(guard, name="output"):
    """The sentinel bytes before and after the output are untouched."""
    buf, offset, n = guard
    es = buf.element_size()
    b = buf.view(torch.uint8).cpu().numpy()
    head, tail = b[:offset * es], b[(offset + n) * es:]
    assert np.all(head == CANARY_BYTE), f"{name}: write before the start of the buffer"
    assert np.all(tail == CANARY_BYTE), f"{name}: write past the end ({np.count_nonzero(tail != CANARY_BYTE)} bytes)"
