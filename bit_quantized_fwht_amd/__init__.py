"""Python binding of libqift.so: the rotated W2A4 linear and KV4 on MI355X.

The functions keep the names of the C ABI (``include/qift.h``) and do
argument marshalling only: every step of the computation runs in the HIP
kernels of ``libqift.so``. PyTorch provides device memory and the stream;
outputs are allocated with ``torch.empty`` on the input's device unless the
caller passes them. There is no fallback path: if the library has not been
built (``python -m bit_quantized_fwht_amd.build``) every call raises
``QiftUnavailable``, and every call raises ``QiftError`` on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqift.so")

# enums (qift.h)
QIFT_OK, QIFT_ERR_INVALID_ARG, QIFT_ERR_ALIGNMENT, QIFT_ERR_UNSUPPORTED, QIFT_ERR_HIP = range(5)
QIFT_F32, QIFT_BF16, QIFT_F16, QIFT_I32 = range(4)
LEVELS = {"mnz": 0, "pot": 1, "int4": 2, "lut": 3, "asym": 4}
SCALE_RULES = {"absmax": 0, "mse": 1}
QIFT_MAX_ROW = 16384
QIFT_MAX_HAD_BLOCK = 4096
QIFT_ATTENTION_SCRATCH_BYTES = 16 * 1024 * 1024
QIFT_MEASURE_SINK_WORDS = 8192

_TORCH_TO_QIFT = {torch.float32: QIFT_F32, torch.bfloat16: QIFT_BF16,
                  torch.float16: QIFT_F16, torch.int32: QIFT_I32}


class QiftError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_string(status)}: {detail}")
        self.status = status


class QiftUnavailable(ImportError):
    pass


class qift_rotate_desc(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("x_dtype", ctypes.c_int32), ("had_block", ctypes.c_int32),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("xq", ctypes.c_void_p),
                ("s_a", ctypes.c_void_p), ("x_rot", ctypes.c_void_p)]


QIFT_MAX_ROTATE_BATCH = 8


class qift_linear_desc(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("s_a", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("Y", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("K", ctypes.c_int64), ("N", ctypes.c_int64), ("levels", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise QiftUnavailable(f"{LIB_PATH} is not built; run `python -m bit_quantized_fwht_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_st = ctypes.c_int
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sig = {
        "qift_quantize_weights": [vp, c_st, i64, i64, i32, c_st, vp, vp, c_st, vp],
        "qift_quantize_weights_ex": [vp, c_st, i64, i64, i32, c_st, ctypes.c_uint32, c_st, vp, vp,
                                     c_st, vp],
        "qift_w2a4_linear_ex": [vp, vp, i64, i64, vp, vp, c_st, c_st, ctypes.c_uint32, i64, vp,
                                c_st, vp],
        "qift_rotate_quant_act": [vp, c_st, i64, i64, i32, vp, vp, vp, vp],
        "qift_w2a4_linear": [vp, vp, i64, i64, vp, vp, c_st, c_st, i64, vp, c_st, vp],
        "qift_kv4_quant": [vp, c_st, i64, i64, i64, i32, vp, vp, vp],
        "qift_kv4_quant_kv": [vp, vp, c_st, i64, i64, i64, i32, vp, vp, vp, vp, vp],
        "qift_rotate_w2a4_linear": [vp, c_st, i64, i64, i32, vp, vp, vp, vp, c_st, c_st,
                                    ctypes.c_uint32, i64, vp, c_st, vp],
        "qift_linear_group_workspace_bytes": [vp, i32, ctypes.POINTER(ctypes.c_size_t)],
        "qift_linear_group_prepare": [vp, i32, c_st, c_st, vp, ctypes.c_size_t,
                                      ctypes.POINTER(ctypes.c_int64), vp],
        "qift_w2a4_linear_grouped": [vp, i64, vp],
        "qift_rotate_quant_act_batched": [vp, i32, vp],
        "qift_kv4_attention_workspace_bytes": [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)],
        "qift_kv4_attention_decode": [vp, c_st, i64, i64, i64, i64, i32, vp, vp, vp, vp,
                                      ctypes.c_float, vp, c_st, vp, ctypes.c_size_t, vp],
        "qift_kv4_attention_decode_noalloc": [vp, c_st, i64, i64, i64, i64, i32, vp, vp, vp, vp,
                                              ctypes.c_float, vp, c_st, vp],
        "qift_gptq_hessian_workspace_bytes": [i64, i64, ctypes.POINTER(ctypes.c_size_t)],
        "qift_gptq_hessian": [vp, c_st, i64, i64, i32, i32, vp, vp, ctypes.c_size_t, vp],
        "qift_gptq_workspace_bytes": [i64, i64, ctypes.POINTER(ctypes.c_size_t)],
        "qift_gptq_quantize_weights": [vp, c_st, i64, i64, vp, i32, c_st, ctypes.c_uint32, c_st,
                                       ctypes.c_double, vp, vp, c_st, vp, ctypes.c_size_t, vp],
        "qift_measure_stream": [vp, vp, i64, i32, vp, vp],
        "qift_measure_mfma_i8": [i64, i64, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = c_st
    lib.qift_status_string.argtypes = [c_st]
    lib.qift_status_string.restype = ctypes.c_char_p
    lib.qift_last_error.argtypes = []
    lib.qift_last_error.restype = ctypes.c_char_p
    lib.qift_abi_version.argtypes = []
    lib.qift_abi_version.restype = ctypes.c_int32
    return lib


class _Lib:
    """libqift.so, loaded on first use; raises QiftUnavailable if missing."""

    def __init__(self):
        self._lib = None

    def __getattr__(self, name):
        if self._lib is None:
            self._lib = _load()
        return getattr(self._lib, name)

    def handle(self):
        if self._lib is None:
            self._lib = _load()
        return self._lib


_C = _Lib()


def load_library():
    """Load libqift.so now (raises QiftUnavailable if it is not built)."""
    return _C.handle()


def status_string(status: int) -> str:
    return _C.qift_status_string(status).decode()


def last_error() -> str:
    return _C.qift_last_error().decode()


def abi_version() -> int:
    return int(_C.qift_abi_version())


def _check(status: int, where: str):
    if status != QIFT_OK:
        raise QiftError(status, where, last_error())


def _stream(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t, name, dtypes=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def _levels(levels) -> int:
    if isinstance(levels, str):
        return LEVELS[levels]
    return int(levels)


def level_table_word(table) -> int:
    """Four integer levels (one per 2-bit code, each in [-15, 15]) -> the
    uint32 level table of the C ABI (byte c = level of code c)."""
    t = [int(v) for v in table]
    if len(t) != 4:
        raise ValueError("a level table has four entries")
    return sum((v & 0xFF) << (8 * c) for c, v in enumerate(t))


def _table_arg(levels, table) -> int:
    if _levels(levels) == LEVELS["lut"]:
        if table is None:
            raise ValueError("levels='lut' needs a level table")
        return level_table_word(table)
    if table is not None:
        raise ValueError("a level table is only used with levels='lut'")
    return 0


def scale_entries(N: int, levels) -> int:
    """Entries of a linear's scales buffer: N, or 2N for levels='asym' (the
    steps, then the zero points)."""
    return 2 * N if _levels(levels) == LEVELS["asym"] else N


def default_channels(scales, levels) -> int:
    """N of a linear whose N is not given: from its scales ([N], or the
    [2, N] / [2N] steps and zero points of levels='asym')."""
    return scales.numel() // 2 if _levels(levels) == LEVELS["asym"] else scales.shape[0]


def code_words_per_row(K: int, levels) -> int:
    return K // 8 if _levels(levels) == LEVELS["int4"] else K // 16


def padded_channels(N: int) -> int:
    """Channels of a weight buffer: N rounded up to whole 16-channel tiles."""
    return (N + 15) // 16 * 16


# ---------------------------------------------------------------------------
# the four calls
# ---------------------------------------------------------------------------

def qift_quantize_weights(W, had_block: int, levels="mnz", scale_dtype=torch.float16,
                          codes=None, scales=None, stream=None, table=None, scale_rule="absmax"):
    """W [N, K] float32/bfloat16 -> (codes int32 [Np, K/16 or K/8] holding the
    uint32 words in the tiled layout (Np = N rounded up to 16), scales [N] in
    scale_dtype). levels='lut' takes a level table (four integers);
    levels='asym' (the min-max grid with a zero point) returns scales [2, N]:
    the steps, then the zero points; scale_rule 'absmax' or 'mse'
    (qift_quantize_weights_ex)."""
    _dev_tensor(W, "W", (torch.float32, torch.bfloat16))
    N, K = W.shape
    lv = _levels(levels)
    if codes is None:
        codes = torch.empty((padded_channels(N), code_words_per_row(K, lv)), dtype=torch.int32,
                            device=W.device)
    if scales is None:
        shape = (2, N) if lv == LEVELS["asym"] else (N,)
        scales = torch.empty(shape, dtype=scale_dtype, device=W.device)
    _dev_tensor(codes, "codes", (torch.int32,))
    _dev_tensor(scales, "scales", (torch.float32, torch.float16))
    if codes.numel() < padded_channels(N) * code_words_per_row(K, lv) or \
            scales.numel() < scale_entries(N, lv):
        raise ValueError("codes or scales buffer too small")
    st = _C.qift_quantize_weights_ex(_ptr(W), _TORCH_TO_QIFT[W.dtype], N, K, had_block, lv,
                                     _table_arg(lv, table), SCALE_RULES[scale_rule], _ptr(codes),
                                     _ptr(scales), _TORCH_TO_QIFT[scales.dtype],
                                     _stream(stream, W.device))
    _check(st, "qift_quantize_weights_ex")
    return codes, scales


def qift_gptq_hessian_workspace_bytes(S: int, K: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_C.qift_gptq_hessian_workspace_bytes(S, K, ctypes.byref(n)),
           "qift_gptq_hessian_workspace_bytes")
    return int(n.value)


def qift_gptq_hessian(X, had_block: int, H=None, accumulate=False, workspace=None, stream=None):
    """Calibration activations X [S, K] float32/bfloat16 -> H = X'^T X'
    (float64 [K, K], X' rotated along K in blocks of had_block); with
    accumulate, X'^T X' is added to the given H. workspace (uint8, device) is
    allocated if not given."""
    _dev_tensor(X, "X", (torch.float32, torch.bfloat16))
    S, K = X.shape
    if H is None:
        if accumulate:
            raise ValueError("accumulate needs H")
        H = torch.empty((K, K), dtype=torch.float64, device=X.device)
    _dev_tensor(H, "H", (torch.float64,))
    if H.numel() < K * K:
        raise ValueError("H too small")
    need = qift_gptq_hessian_workspace_bytes(S, K)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=X.device)
    _dev_tensor(workspace, "workspace", (torch.uint8,))
    st = _C.qift_gptq_hessian(_ptr(X), _TORCH_TO_QIFT[X.dtype], S, K, had_block,
                              1 if accumulate else 0, _ptr(H), _ptr(workspace), workspace.numel(),
                              _stream(stream, X.device))
    _check(st, "qift_gptq_hessian")
    return H


def qift_gptq_workspace_bytes(N: int, K: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_C.qift_gptq_workspace_bytes(N, K, ctypes.byref(n)), "qift_gptq_workspace_bytes")
    return int(n.value)


def qift_gptq_quantize_weights(W, H, had_block: int, levels="mnz", scale_dtype=torch.float16,
                               table=None, scale_rule="absmax", damp=0.01, codes=None,
                               scales=None, workspace=None, stream=None):
    """Error-compensated quantization of W [N, K] float32/bfloat16 with the
    Hessian H [K, K] float64 (qift_gptq_hessian): codes and scales in the
    layout of qift_quantize_weights. workspace (uint8, device) is allocated if
    not given."""
    _dev_tensor(W, "W", (torch.float32, torch.bfloat16))
    _dev_tensor(H, "H", (torch.float64,))
    N, K = W.shape
    if H.numel() < K * K:
        raise ValueError("H too small")
    lv = _levels(levels)
    if codes is None:
        codes = torch.empty((padded_channels(N), code_words_per_row(K, lv)), dtype=torch.int32,
                            device=W.device)
    if scales is None:
        shape = (2, N) if lv == LEVELS["asym"] else (N,)
        scales = torch.empty(shape, dtype=scale_dtype, device=W.device)
    _dev_tensor(codes, "codes", (torch.int32,))
    _dev_tensor(scales, "scales", (torch.float32, torch.float16))
    if codes.numel() < padded_channels(N) * code_words_per_row(K, lv) or \
            scales.numel() < scale_entries(N, lv):
        raise ValueError("codes or scales buffer too small")
    need = qift_gptq_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=W.device)
    _dev_tensor(workspace, "workspace", (torch.uint8,))
    st = _C.qift_gptq_quantize_weights(_ptr(W), _TORCH_TO_QIFT[W.dtype], N, K, _ptr(H), had_block,
                                       lv, _table_arg(lv, table), SCALE_RULES[scale_rule],
                                       float(damp), _ptr(codes), _ptr(scales),
                                       _TORCH_TO_QIFT[scales.dtype], _ptr(workspace),
                                       workspace.numel(), _stream(stream, W.device))
    _check(st, "qift_gptq_quantize_weights")
    return codes, scales


def qift_rotate_quant_act(X, had_block: int, xq=None, s_a=None, x_rot=None, want_x_rot=False,
                          stream=None):
    """X [M, K] float32/bfloat16 -> (xq uint8 [M, K/2], s_a float32 [M],
    x_rot float32 [M, K] or None)."""
    _dev_tensor(X, "X", (torch.float32, torch.bfloat16))
    M, K = X.shape
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if s_a is None:
        s_a = torch.empty((M,), dtype=torch.float32, device=X.device)
    if x_rot is None and want_x_rot:
        x_rot = torch.empty((M, K), dtype=torch.float32, device=X.device)
    _check_rotate_buffers(M, K, xq, s_a, x_rot)
    st = _C.qift_rotate_quant_act(_ptr(X), _TORCH_TO_QIFT[X.dtype], M, K, had_block, _ptr(xq),
                                  _ptr(s_a), _ptr(x_rot), _stream(stream, X.device))
    _check(st, "qift_rotate_quant_act")
    return xq, s_a, x_rot


def _check_rotate_buffers(M, K, xq, s_a, x_rot):
    _dev_tensor(xq, "xq", (torch.uint8,))
    _dev_tensor(s_a, "s_a", (torch.float32,))
    if x_rot is not None:
        _dev_tensor(x_rot, "x_rot", (torch.float32,))
    if xq.numel() < M * (K // 2) or s_a.numel() < M or (x_rot is not None and x_rot.numel() < M * K):
        raise ValueError("xq, s_a or x_rot too small for [M, K]")


class RotateBatch:
    """A fixed set of qift_rotate_quant_act_batched descriptors (inputs and
    output buffers given once); run() enqueues the one call."""

    def __init__(self, items):
        items = list(items)
        if not 0 < len(items) <= QIFT_MAX_ROTATE_BATCH:
            raise ValueError(f"1..{QIFT_MAX_ROTATE_BATCH} matrices per batch")
        self._descs = (qift_rotate_desc * len(items))()
        self._keep = []
        for j, it in enumerate(items):
            X, had_block, xq, s_a = it[0], it[1], it[2], it[3]
            x_rot = it[4] if len(it) > 4 else None
            _dev_tensor(X, "X", (torch.float32, torch.bfloat16))
            M, K = X.shape
            _check_rotate_buffers(M, K, xq, s_a, x_rot)
            self._descs[j] = qift_rotate_desc(_ptr(X), _TORCH_TO_QIFT[X.dtype], had_block, M, K,
                                              _ptr(xq), _ptr(s_a), _ptr(x_rot))
            self._keep.append((X, xq, s_a, x_rot))
        self.device = items[0][0].device
        self.count = len(items)

    def run(self, stream=None):
        st = _C.qift_rotate_quant_act_batched(ctypes.cast(self._descs, ctypes.c_void_p), self.count,
                                              _stream(stream, self.device))
        _check(st, "qift_rotate_quant_act_batched")


def qift_rotate_quant_act_batched(items, stream=None):
    """Several activation matrices in one call. items: sequence of
    (X, had_block) or (X, had_block, xq, s_a, x_rot) with X [M, K]
    float32/bfloat16 (None outputs are allocated; x_rot None means not
    wanted). Returns [(xq, s_a, x_rot), ...] in the same order."""
    items = list(items)
    if len(items) > QIFT_MAX_ROTATE_BATCH:
        raise ValueError(f"at most {QIFT_MAX_ROTATE_BATCH} matrices per call")
    descs = (qift_rotate_desc * max(1, len(items)))()
    outs = []
    dev = None
    for j, it in enumerate(items):
        X, had_block = it[0], it[1]
        xq, s_a, x_rot = (tuple(it[2:5]) + (None, None, None))[:3]
        _dev_tensor(X, "X", (torch.float32, torch.bfloat16))
        dev = X.device
        M, K = X.shape
        if xq is None:
            xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
        if s_a is None:
            s_a = torch.empty((M,), dtype=torch.float32, device=X.device)
        _check_rotate_buffers(M, K, xq, s_a, x_rot)
        descs[j] = qift_rotate_desc(_ptr(X), _TORCH_TO_QIFT[X.dtype], had_block, M, K, _ptr(xq),
                                    _ptr(s_a), _ptr(x_rot))
        outs.append((xq, s_a, x_rot))
    if not items:
        return outs
    st = _C.qift_rotate_quant_act_batched(ctypes.cast(descs, ctypes.c_void_p), len(items),
                                          _stream(stream, dev))
    _check(st, "qift_rotate_quant_act_batched")
    return outs


_LINEAR_DTYPES = (("xq", (torch.uint8,)), ("s_a", (torch.float32,)), ("codes", (torch.int32,)),
                  ("scales", (torch.float32, torch.float16)),
                  ("Y", (torch.float32, torch.bfloat16, torch.int32)))


def _check_linear_buffers(bufs, N, levels, scale_dtype=None, y_dtype=None, placement=True):
    """The buffers of one linear (dict with xq, s_a, codes, scales, Y):
    dtypes, and sizes against M, K (from xq [M, K/2]) and N, checked before
    their placement; then (placement=True) each must be a contiguous GPU
    tensor. scale_dtype and y_dtype, if given, are the dtypes the call was
    set up for (a grouped plan fixes them for every linear). Returns (M, K)."""
    for name, dts in _LINEAR_DTYPES:
        t = bufs[name]
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in dts:
            raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dts}")
    xq, s_a, codes, scales, Y = (bufs[k] for k, _ in _LINEAR_DTYPES)
    if scale_dtype is not None and scales.dtype != scale_dtype:
        raise TypeError(f"scales has dtype {scales.dtype}, the call is set up for {scale_dtype}")
    if y_dtype is not None and Y.dtype != y_dtype:
        raise TypeError(f"Y has dtype {Y.dtype}, the call is set up for {y_dtype}")
    if xq.dim() != 2:
        raise ValueError("xq must be [M, K/2]")
    M, K = xq.shape[0], xq.shape[1] * 2
    if N < 0:
        raise ValueError("negative N")
    if s_a.numel() < M:
        raise ValueError(f"s_a has {s_a.numel()} elements, M = {M} needed")
    if scales.numel() < scale_entries(N, levels):
        raise ValueError(f"scales has {scales.numel()} elements, {scale_entries(N, levels)} "
                         f"needed for N = {N}")
    need = padded_channels(N) * code_words_per_row(K, levels)
    if codes.numel() < need:
        raise ValueError(f"codes has {codes.numel()} words, {need} needed for N = {N}, K = {K}")
    if Y.numel() < M * N:
        raise ValueError(f"Y has {Y.numel()} elements, M * N = {M * N} needed")
    if placement:
        for name, _ in _LINEAR_DTYPES:
            _dev_tensor(bufs[name], name)
    return M, K


def qift_w2a4_linear(xq, s_a, codes, scales, levels="mnz", out_dtype=torch.float32, Y=None,
                     N=None, stream=None, table=None):
    """(xq [M, K/2], s_a [M], codes [N, ...], scales [N]) -> Y [M, N] in
    out_dtype (float32, bfloat16, or int32 for the raw accumulator).
    levels='lut' takes a level table, levels='asym' the 2N steps and zero
    points as scales (qift_w2a4_linear_ex)."""
    if N is None:
        N = default_channels(scales, levels)
    if Y is None:
        _dev_tensor(xq, "xq", (torch.uint8,))
        Y = torch.empty((xq.shape[0], N), dtype=out_dtype, device=xq.device)
    M, K = _check_linear_buffers(dict(xq=xq, s_a=s_a, codes=codes, scales=scales, Y=Y), N, levels)
    st = _C.qift_w2a4_linear_ex(_ptr(xq), _ptr(s_a), M, K, _ptr(codes), _ptr(scales),
                                _TORCH_TO_QIFT[scales.dtype], _levels(levels),
                                _table_arg(levels, table), N, _ptr(Y), _TORCH_TO_QIFT[Y.dtype],
                                _stream(stream, xq.device))
    _check(st, "qift_w2a4_linear_ex")
    return Y


def qift_rotate_w2a4_linear(X, had_block: int, codes, scales, levels="mnz",
                            out_dtype=torch.float32, Y=None, N=None, xq=None, s_a=None,
                            stream=None, table=None):
    """X [M, K] float32/bfloat16 -> (Y [M, N], xq [M, K/2], s_a [M]): the
    rotation + int4 quantization of X and the linear in one call (one launch
    for a single token row), with the results of qift_rotate_quant_act
    followed by qift_w2a4_linear."""
    _dev_tensor(X, "X", (torch.float32, torch.bfloat16))
    M, K = X.shape
    if N is None:
        N = default_channels(scales, levels)
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if s_a is None:
        s_a = torch.empty((M,), dtype=torch.float32, device=X.device)
    if Y is None:
        Y = torch.empty((M, N), dtype=out_dtype, device=X.device)
    _check_rotate_buffers(M, K, xq, s_a, None)
    if xq.numel() != M * (K // 2):
        raise ValueError("xq must hold exactly [M, K/2] (it is also the linear's input)")
    _check_linear_buffers(dict(xq=xq.view(M, K // 2), s_a=s_a, codes=codes, scales=scales, Y=Y),
                          N, levels)
    st = _C.qift_rotate_w2a4_linear(_ptr(X), _TORCH_TO_QIFT[X.dtype], M, K, had_block, _ptr(xq),
                                    _ptr(s_a), _ptr(codes), _ptr(scales),
                                    _TORCH_TO_QIFT[scales.dtype], _levels(levels),
                                    _table_arg(levels, table), N, _ptr(Y), _TORCH_TO_QIFT[Y.dtype],
                                    _stream(stream, X.device))
    _check(st, "qift_rotate_w2a4_linear")
    return Y, xq, s_a


def qift_kv4_quant(KV, had_block: int, kvq=None, scales=None, stream=None):
    """KV [T, H, D] bfloat16/float32 -> (kvq uint8 [T, H, D/2], scales float32 [T, H])."""
    _dev_tensor(KV, "KV", (torch.float32, torch.bfloat16))
    T, H, D = KV.shape
    if kvq is None:
        kvq = torch.empty((T, H, D // 2), dtype=torch.uint8, device=KV.device)
    if scales is None:
        scales = torch.empty((T, H), dtype=torch.float32, device=KV.device)
    _dev_tensor(kvq, "kvq", (torch.uint8,))
    _dev_tensor(scales, "scales", (torch.float32,))
    st = _C.qift_kv4_quant(_ptr(KV), _TORCH_TO_QIFT[KV.dtype], T, H, D, had_block, _ptr(kvq),
                           _ptr(scales), _stream(stream, KV.device))
    _check(st, "qift_kv4_quant")
    return kvq, scales


def qift_kv4_quant_kv(K, V, had_block: int, kq=None, ks=None, vq=None, vs=None, stream=None):
    """K and V [T, H, D] (same shape and dtype, bfloat16/float32) of one layer
    in one call -> (kq, ks, vq, vs): the results of qift_kv4_quant on each."""
    _dev_tensor(K, "K", (torch.float32, torch.bfloat16))
    _dev_tensor(V, "V", (K.dtype,))
    if K.shape != V.shape or K.device != V.device:
        raise ValueError("K and V must have the same shape and device")
    T, H, D = K.shape
    outs = []
    for name, t, shape, dt in (("kq", kq, (T, H, D // 2), torch.uint8), ("ks", ks, (T, H), torch.float32),
                               ("vq", vq, (T, H, D // 2), torch.uint8), ("vs", vs, (T, H), torch.float32)):
        if t is None:
            t = torch.empty(shape, dtype=dt, device=K.device)
        _dev_tensor(t, name, (dt,))
        outs.append(t)
    kq, ks, vq, vs = outs
    st = _C.qift_kv4_quant_kv(_ptr(K), _ptr(V), _TORCH_TO_QIFT[K.dtype], T, H, D, had_block,
                              _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), _stream(stream, K.device))
    _check(st, "qift_kv4_quant_kv")
    return kq, ks, vq, vs


def qift_kv4_attention_workspace_bytes(S: int, T: int, H: int, D: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_C.qift_kv4_attention_workspace_bytes(S, T, H, D, ctypes.byref(n)),
           "qift_kv4_attention_workspace_bytes")
    return int(n.value)


def qift_kv4_attention_decode(q, kq, ks, vq, vs, had_block: int, softmax_scale=None, out=None,
                              out_dtype=torch.float32, workspace=None, stream=None):
    """Decode attention over a KV4 cache. q [S, H, D] (or [H, D]) float32 /
    bfloat16; kq, vq [S, T, H, D/2] (or [T, H, D/2]) uint8; ks, vs [S, T, H]
    (or [T, H]) float32 -> out [S, H, D] (or [H, D]). softmax_scale defaults
    to 1/sqrt(D); workspace (uint8, device) is allocated if not given."""
    _dev_tensor(q, "q", (torch.float32, torch.bfloat16))
    single = q.dim() == 2
    S = 1 if single else q.shape[0]
    H, D = q.shape[-2], q.shape[-1]
    T = kq.shape[-3]
    for name, t_, dt in (("kq", kq, torch.uint8), ("vq", vq, torch.uint8), ("ks", ks, torch.float32),
                         ("vs", vs, torch.float32)):
        _dev_tensor(t_, name, (dt,))
    if kq.numel() < S * T * H * (D // 2) or vq.numel() < S * T * H * (D // 2) or \
            ks.numel() < S * T * H or vs.numel() < S * T * H:
        raise ValueError("cache buffers too small for [S, T, H, D]")
    if softmax_scale is None:
        softmax_scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _dev_tensor(out, "out", (torch.float32, torch.bfloat16))
    if out.numel() < S * H * D:
        raise ValueError("out too small")
    need = qift_kv4_attention_workspace_bytes(S, T, H, D)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    _dev_tensor(workspace, "workspace", (torch.uint8,))
    st = _C.qift_kv4_attention_decode(_ptr(q), _TORCH_TO_QIFT[q.dtype], S, T, H, D, had_block,
                                      _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), float(softmax_scale),
                                      _ptr(out), _TORCH_TO_QIFT[out.dtype], _ptr(workspace),
                                      workspace.numel(), _stream(stream, q.device))
    _check(st, "qift_kv4_attention_decode")
    return out


def qift_kv4_attention_decode_noalloc(q, kq, ks, vq, vs, had_block: int, out,
                                      softmax_scale=None, stream=None):
    """qift_kv4_attention_decode without a workspace: the partial results go
    to the library's fixed per-GPU array (QIFT_ATTENTION_SCRATCH_BYTES), and
    nothing is allocated, here either: ``out`` [S, H, D] (or [H, D]) float32 /
    bfloat16 must be given. Calls that overlap on one GPU race."""
    _dev_tensor(q, "q", (torch.float32, torch.bfloat16))
    single = q.dim() == 2
    S = 1 if single else q.shape[0]
    H, D = q.shape[-2], q.shape[-1]
    T = kq.shape[-3]
    for name, t_, dt in (("kq", kq, torch.uint8), ("vq", vq, torch.uint8), ("ks", ks, torch.float32),
                         ("vs", vs, torch.float32)):
        _dev_tensor(t_, name, (dt,))
    if kq.numel() < S * T * H * (D // 2) or vq.numel() < S * T * H * (D // 2) or \
            ks.numel() < S * T * H or vs.numel() < S * T * H:
        raise ValueError("cache buffers too small for [S, T, H, D]")
    _dev_tensor(out, "out", (torch.float32, torch.bfloat16))
    if out.numel() < S * H * D:
        raise ValueError("out too small")
    if softmax_scale is None:
        softmax_scale = 1.0 / float(D) ** 0.5
    st = _C.qift_kv4_attention_decode_noalloc(_ptr(q), _TORCH_TO_QIFT[q.dtype], S, T, H, D,
                                              had_block, _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs),
                                              float(softmax_scale), _ptr(out),
                                              _TORCH_TO_QIFT[out.dtype], _stream(stream, q.device))
    _check(st, "qift_kv4_attention_decode_noalloc")
    return out


# ---------------------------------------------------------------------------
# measurement calls (include/qift_measure.h): no step of the method
# ---------------------------------------------------------------------------

def _sink(device):
    return torch.empty((QIFT_MEASURE_SINK_WORDS,), dtype=torch.int32, device=device)


def qift_measure_stream(src, dst=None, sink=None, stream=None):
    """Stream the bytes of ``src`` through the GPU: read only if ``dst`` is
    None, else copy them into ``dst`` (same byte size, no overlap). For
    timing the HBM rate; returns nothing useful."""
    _dev_tensor(src, "src")
    nbytes = src.numel() * src.element_size()
    if dst is not None:
        _dev_tensor(dst, "dst")
        if dst.numel() * dst.element_size() != nbytes:
            raise ValueError("dst must have the byte size of src")
    sink = _sink(src.device) if sink is None else sink
    st = _C.qift_measure_stream(_ptr(src), _ptr(dst), nbytes, 0 if dst is None else 1, _ptr(sink),
                                _stream(stream, src.device))
    _check(st, "qift_measure_stream")


def qift_measure_mfma_i8(iters: int, workgroups: int, clk, sink=None, stream=None):
    """Run iters x 8 int8 16x16x64 matrix-core instructions on each of
    4 * workgroups waves (32768 operations each); ``clk`` (int64 [4] on the
    GPU) receives the shader clock and the 100 MHz counter at the start and
    end of the first wave."""
    _dev_tensor(clk, "clk", (torch.int64,))
    if clk.numel() < 4:
        raise ValueError("clk must hold 4 int64")
    sink = _sink(clk.device) if sink is None else sink
    st = _C.qift_measure_mfma_i8(int(iters), int(workgroups), _ptr(sink), _ptr(clk),
                                 _stream(stream, clk.device))
    _check(st, "qift_measure_mfma_i8")


# ---------------------------------------------------------------------------
# grouped linear
# ---------------------------------------------------------------------------

class LinearGroup:
    """Many decode linears (M <= 16 each) run by one launch.

    ``items`` is a sequence of dicts with keys xq, s_a, codes, scales, Y and
    levels, plus table for levels='lut' (tensors already allocated on one
    device). The plan lives in a
    device workspace owned by this object; the tensors must stay alive.
    """

    def __init__(self, items, scale_dtype=torch.float16, y_dtype=torch.float32, stream=None):
        n = len(items)
        descs = (qift_linear_desc * max(n, 1))()
        self._keep = []
        device = None
        # dtypes and sizes of every item first, then their placement
        for placement in (False, True):
            for i, it in enumerate(items):
                try:
                    _check_linear_buffers(it, it.get("N", default_channels(it["scales"], it["levels"])),
                                          it["levels"],
                                          scale_dtype, y_dtype, placement)
                except (TypeError, ValueError) as e:
                    raise type(e)(f"item {i}: {e}") from None
                if placement:
                    device = device or it["xq"].device
                    for key, _ in _LINEAR_DTYPES:
                        if it[key].device != device:
                            raise ValueError(f"item {i}: {key} is on {it[key].device}, "
                                             f"the group on {device}")
        for i, it in enumerate(items):
            N = it.get("N", default_channels(it["scales"], it["levels"]))
            M, K = it["xq"].shape[0], it["xq"].shape[1] * 2
            tw = _table_arg(it["levels"], it.get("table"))  # the descriptor's int32 table word
            descs[i] = qift_linear_desc(it["xq"].data_ptr(), it["s_a"].data_ptr(),
                                        it["codes"].data_ptr(), it["scales"].data_ptr(),
                                        it["Y"].data_ptr(), M, K, N, _levels(it["levels"]),
                                        tw - (1 << 32) if tw >= 1 << 31 else tw)
            self._keep.append(it)
        nbytes = ctypes.c_size_t(0)
        _check(_C.qift_linear_group_workspace_bytes(descs, n, ctypes.byref(nbytes)),
               "qift_linear_group_workspace_bytes")
        self.workspace = torch.empty((max(int(nbytes.value), 256),), dtype=torch.uint8, device=device)
        tiles = ctypes.c_int64(0)
        _check(_C.qift_linear_group_prepare(descs, n, _TORCH_TO_QIFT[scale_dtype],
                                            _TORCH_TO_QIFT[y_dtype], _ptr(self.workspace),
                                            self.workspace.numel(), ctypes.byref(tiles),
                                            _stream(stream, device)),
               "qift_linear_group_prepare")
        self.launch_tiles = int(tiles.value)
        self.device = device

    def run(self, stream=None):
        _check(_C.qift_w2a4_linear_grouped(_ptr(self.workspace), self.launch_tiles,
                                           _stream(stream, self.device)),
               "qift_w2a4_linear_grouped")


__all__ = ["load_library", "QiftUnavailable", "qift_quantize_weights", "qift_rotate_quant_act",
           "qift_rotate_quant_act_batched", "RotateBatch", "qift_w2a4_linear", "qift_kv4_quant",
           "qift_kv4_quant_kv",
           "LinearGroup", "QiftError", "qift_linear_desc", "LEVELS", "status_string", "last_error",
           "abi_version", "code_words_per_row", "padded_channels", "LIB_PATH", "SCALE_RULES",
           "level_table_word", "scale_entries", "qift_kv4_attention_decode", "qift_kv4_attention_workspace_bytes",
           "qift_kv4_attention_decode_noalloc", "QIFT_ATTENTION_SCRATCH_BYTES",
           "qift_rotate_w2a4_linear",
           "qift_gptq_hessian", "qift_gptq_hessian_workspace_bytes", "qift_gptq_quantize_weights",
           "qift_gptq_workspace_bytes"]
