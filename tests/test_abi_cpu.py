"""Host-side checks of libqift.so that need no GPU: the library loads, it
exports every function declared in include/qift.h, and invalid arguments are
rejected with the documented status before anything is launched (these calls
never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import bit_quantized_fwht_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qift.h")
MEASURE_HEADER = os.path.join(ROOT, "include", "qift_measure.h")

V = ctypes.c_void_p
A16 = V(0x10000)   # fake, 16-byte aligned device addresses (never dereferenced)
A16b = V(0x20000)
A16c = V(0x30000)
A16d = V(0x40000)
A16e = V(0x50000)


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(qift_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = q.load_library()
    names = declared_functions()
    assert "qift_w2a4_linear" in names and "qift_kv4_quant" in names
    assert len(names) == 22, names
    for n in names:
        assert hasattr(lib, n), n
    assert q.abi_version() == 8
    for s in range(5):
        assert q.status_string(s).startswith("QIFT_")


def test_measurement_calls_exported_and_validated():
    """The two measurement calls of include/qift_measure.h are exported and
    reject bad arguments before any launch."""
    lib = q.load_library()
    names = declared_functions(MEASURE_HEADER)
    assert names == ["qift_measure_mfma_i8", "qift_measure_stream"], names
    for n in names:
        assert hasattr(lib, n), n
    ms, mm = q._C.qift_measure_stream, q._C.qift_measure_mfma_i8
    assert ms(A16, A16b, 1024, 2, A16c, None) == q.QIFT_ERR_INVALID_ARG     # mode
    assert ms(A16, A16b, 1000, 1, A16c, None) == q.QIFT_ERR_INVALID_ARG     # not a multiple of 16
    assert ms(A16, A16b, 0, 0, A16c, None) == q.QIFT_ERR_INVALID_ARG
    assert ms(A16, A16b, (1 << 40) + 16, 0, A16c, None) == q.QIFT_ERR_INVALID_ARG
    assert ms(None, A16b, 1024, 0, A16c, None) == q.QIFT_ERR_INVALID_ARG
    assert ms(A16, None, 1024, 1, A16c, None) == q.QIFT_ERR_INVALID_ARG     # copy needs dst
    assert ms(A16, A16b, 1024, 0, None, None) == q.QIFT_ERR_INVALID_ARG     # sink
    assert ms(V(0x10008), A16b, 1024, 0, A16c, None) == q.QIFT_ERR_ALIGNMENT
    assert ms(A16, V(0x10200), 1024, 1, A16c, None) == q.QIFT_ERR_INVALID_ARG  # overlap
    assert mm(0, 16, A16, A16b, None) == q.QIFT_ERR_INVALID_ARG
    assert mm(1 << 25, 16, A16, A16b, None) == q.QIFT_ERR_INVALID_ARG
    assert mm(16, 0, A16, A16b, None) == q.QIFT_ERR_INVALID_ARG
    assert mm(16, (1 << 20) + 1, A16, A16b, None) == q.QIFT_ERR_INVALID_ARG
    assert mm(16, 16, None, A16b, None) == q.QIFT_ERR_INVALID_ARG
    assert mm(16, 16, A16, V(0x20008), None) == q.QIFT_ERR_ALIGNMENT


def lin(**kw):
    args = dict(xq=A16, s_a=A16b, M=4, K=256, codes=A16c, scales=A16d, sd=q.QIFT_F16, lv=0,
                N=64, Y=A16e, yd=q.QIFT_F32)
    args.update(kw)
    return q._C.qift_w2a4_linear(args["xq"], args["s_a"], args["M"], args["K"], args["codes"],
                                 args["scales"], args["sd"], args["lv"], args["N"], args["Y"],
                                 args["yd"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(xq=None), q.QIFT_ERR_INVALID_ARG),
    (dict(codes=None), q.QIFT_ERR_INVALID_ARG),
    (dict(K=100), q.QIFT_ERR_INVALID_ARG),
    (dict(K=0), q.QIFT_ERR_INVALID_ARG),
    (dict(K=65536 + 64), q.QIFT_ERR_UNSUPPORTED),
    (dict(M=-1), q.QIFT_ERR_INVALID_ARG),
    (dict(lv=7), q.QIFT_ERR_INVALID_ARG),
    (dict(sd=q.QIFT_BF16), q.QIFT_ERR_INVALID_ARG),
    (dict(yd=q.QIFT_F16), q.QIFT_ERR_INVALID_ARG),
    (dict(xq=V(0x10008)), q.QIFT_ERR_ALIGNMENT),
    (dict(codes=V(0x30004)), q.QIFT_ERR_ALIGNMENT),
    (dict(Y=V(0x50001)), q.QIFT_ERR_ALIGNMENT),
])
def test_linear_rejects(kw, status):
    assert lin(**kw) == status
    assert q.last_error() != ""


def test_linear_empty_is_noop():
    # M = 0 or N = 0: valid, nothing to do, no launch
    assert lin(M=0, xq=None, s_a=None, codes=None, scales=None, Y=None) == q.QIFT_OK
    assert lin(N=0) == q.QIFT_OK


def rot(**kw):
    args = dict(X=A16, xd=q.QIFT_BF16, M=2, K=256, B=256, xq=A16b, s_a=A16c, x_rot=None)
    args.update(kw)
    return q._C.qift_rotate_quant_act(args["X"], args["xd"], args["M"], args["K"], args["B"],
                                      args["xq"], args["s_a"], args["x_rot"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=3), q.QIFT_ERR_INVALID_ARG),
    (dict(B=0), q.QIFT_ERR_INVALID_ARG),
    (dict(B=512), q.QIFT_ERR_INVALID_ARG),         # does not divide K=256
    (dict(K=8192 * 2, B=8192), q.QIFT_ERR_UNSUPPORTED),
    (dict(K=16384 + 2), q.QIFT_ERR_UNSUPPORTED),
    (dict(K=255, B=1), q.QIFT_ERR_INVALID_ARG),
    (dict(xd=q.QIFT_F16), q.QIFT_ERR_INVALID_ARG),
    (dict(X=None), q.QIFT_ERR_INVALID_ARG),
    (dict(xq=V(0x20004)), q.QIFT_ERR_ALIGNMENT),
    (dict(x_rot=V(0x20002)), q.QIFT_ERR_ALIGNMENT),
])
def test_rotate_rejects(kw, status):
    assert rot(**kw) == status


def test_rotate_empty_is_noop():
    assert rot(M=0, X=None, xq=None, s_a=None) == q.QIFT_OK


def rot_batch(descs, count=None):
    arr = (q.qift_rotate_desc * max(1, len(descs)))(*descs)
    n = len(descs) if count is None else count
    return q._C.qift_rotate_quant_act_batched(ctypes.cast(arr, ctypes.c_void_p), n, None)


def rdesc(**kw):
    args = dict(X=A16.value, x_dtype=q.QIFT_BF16, had_block=256, M=2, K=256, xq=A16b.value,
                s_a=A16c.value, x_rot=None)
    args.update(kw)
    return q.qift_rotate_desc(**args)


def test_rotate_batched_struct_matches_header():
    # X, x_dtype, had_block, M, K, xq, s_a, x_rot with natural alignment
    assert ctypes.sizeof(q.qift_rotate_desc) == 56
    assert q.qift_rotate_desc.M.offset == 16 and q.qift_rotate_desc.xq.offset == 32


@pytest.mark.parametrize("descs,count,status", [
    ([rdesc()] * 9, None, q.QIFT_ERR_INVALID_ARG),                      # more than 8
    ([rdesc()], -1, q.QIFT_ERR_INVALID_ARG),
    ([rdesc(), rdesc(had_block=3)], None, q.QIFT_ERR_INVALID_ARG),      # second one invalid
    ([rdesc(M=0), rdesc(K=16384 + 2)], None, q.QIFT_ERR_UNSUPPORTED),
    ([rdesc(xq=0x20004)], None, q.QIFT_ERR_ALIGNMENT),
    ([rdesc(X=None)], None, q.QIFT_ERR_INVALID_ARG),
])
def test_rotate_batched_rejects(descs, count, status):
    assert rot_batch(descs, count) == status
    assert q.last_error() != ""


def test_rotate_batched_empty_is_noop():
    assert rot_batch([], 0) == q.QIFT_OK
    assert q._C.qift_rotate_quant_act_batched(None, 0, None) == q.QIFT_OK
    # all descriptors with M = 0: validated, nothing launched
    assert rot_batch([rdesc(M=0, X=None, xq=None, s_a=None)] * 3) == q.QIFT_OK


def qw(**kw):
    args = dict(W=A16, wd=q.QIFT_F32, N=8, K=256, B=256, lv=0, codes=A16b, scales=A16c,
                sd=q.QIFT_F16)
    args.update(kw)
    return q._C.qift_quantize_weights(args["W"], args["wd"], args["N"], args["K"], args["B"],
                                      args["lv"], args["codes"], args["scales"], args["sd"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), q.QIFT_ERR_INVALID_ARG),
    (dict(lv=3), q.QIFT_ERR_INVALID_ARG),
    (dict(sd=q.QIFT_I32), q.QIFT_ERR_INVALID_ARG),
    (dict(wd=q.QIFT_I32), q.QIFT_ERR_INVALID_ARG),
    (dict(codes=V(0x20008)), q.QIFT_ERR_ALIGNMENT),
    (dict(B=6), q.QIFT_ERR_INVALID_ARG),
    (dict(scales=None), q.QIFT_ERR_INVALID_ARG),
])
def test_quantize_weights_rejects(kw, status):
    assert qw(**kw) == status


def kv(**kw):
    args = dict(KV=A16, d=q.QIFT_BF16, T=4, H=2, D=128, B=128, kvq=A16b, scales=A16c)
    args.update(kw)
    return q._C.qift_kv4_quant(args["KV"], args["d"], args["T"], args["H"], args["D"], args["B"],
                               args["kvq"], args["scales"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96, B=32), q.QIFT_ERR_UNSUPPORTED),
    (dict(D=512, B=512), q.QIFT_ERR_UNSUPPORTED),
    (dict(B=256), q.QIFT_ERR_UNSUPPORTED),
    (dict(B=12), q.QIFT_ERR_INVALID_ARG),
    (dict(KV=V(0x10002)), q.QIFT_ERR_ALIGNMENT),
    (dict(kvq=None), q.QIFT_ERR_INVALID_ARG),
    (dict(T=-1), q.QIFT_ERR_INVALID_ARG),
])
def test_kv4_rejects(kw, status):
    assert kv(**kw) == status


def test_kv4_empty_is_noop():
    assert kv(T=0, KV=None, kvq=None, scales=None) == q.QIFT_OK


def kv_pair(**kw):
    args = dict(K=A16, Vt=A16b, d=q.QIFT_BF16, T=4, H=2, D=128, B=128, kq=A16c, ks=A16d,
                vq=A16e, vs=V(0x60000))
    args.update(kw)
    return q._C.qift_kv4_quant_kv(args["K"], args["Vt"], args["d"], args["T"], args["H"],
                                  args["D"], args["B"], args["kq"], args["ks"], args["vq"],
                                  args["vs"], None)


# T * H = 8 vectors of D = 128: 512 bytes of codes and 32 bytes of scales each
@pytest.mark.parametrize("kw,status", [
    (dict(D=96, B=32), q.QIFT_ERR_UNSUPPORTED),
    (dict(B=256), q.QIFT_ERR_UNSUPPORTED),
    (dict(B=12), q.QIFT_ERR_INVALID_ARG),
    (dict(d=q.QIFT_I32), q.QIFT_ERR_INVALID_ARG),
    (dict(Vt=V(0x20002)), q.QIFT_ERR_ALIGNMENT),
    (dict(vq=V(0x50008)), q.QIFT_ERR_ALIGNMENT),
    (dict(K=None), q.QIFT_ERR_INVALID_ARG),
    (dict(vs=None), q.QIFT_ERR_INVALID_ARG),
    (dict(H=-1), q.QIFT_ERR_INVALID_ARG),
    (dict(vq=V(0x30000 + 496)), q.QIFT_ERR_INVALID_ARG),   # V's codes overlap K's by 16 bytes
    (dict(vs=V(0x40000 + 28)), q.QIFT_ERR_INVALID_ARG),    # V's scales overlap K's by 4 bytes
])
def test_kv4_pair_rejects(kw, status):
    assert kv_pair(**kw) == status


def test_kv4_pair_empty_is_noop():
    assert kv_pair(T=0, K=None, Vt=None, kq=None, ks=None, vq=None, vs=None) == q.QIFT_OK


def make_desc(**kw):
    d = dict(xq=0x10000, s_a=0x20000, codes=0x30000, scales=0x40000, Y=0x50000, M=1, K=4096,
             N=4096, levels=0, reserved=0)
    d.update(kw)
    return q.qift_linear_desc(d["xq"], d["s_a"], d["codes"], d["scales"], d["Y"], d["M"], d["K"],
                              d["N"], d["levels"], d["reserved"])


def lin_ex(table, **kw):
    args = dict(xq=A16, s_a=A16b, M=4, K=256, codes=A16c, scales=A16d, sd=q.QIFT_F16, lv=3,
                N=64, Y=A16e, yd=q.QIFT_F32)
    args.update(kw)
    return q._C.qift_w2a4_linear_ex(args["xq"], args["s_a"], args["M"], args["K"], args["codes"],
                                    args["scales"], args["sd"], args["lv"], table, args["N"],
                                    args["Y"], args["yd"], None)


@pytest.mark.parametrize("table,lv,status", [
    (q.level_table_word((-2, -1, 0, 1)), 3, q.QIFT_OK),
    (q.level_table_word((3, 10, -3, -10)), 3, q.QIFT_OK),
    (q.level_table_word((15, -15, 0, 0)), 3, q.QIFT_OK),
    (0, 3, q.QIFT_ERR_INVALID_ARG),                                # all zero
    (q.level_table_word((16, 1, 1, 1)), 3, q.QIFT_ERR_INVALID_ARG),  # |L| > 15
    (q.level_table_word((1, -16, 1, 1)), 3, q.QIFT_ERR_INVALID_ARG),
    (q.level_table_word((1, 3, -3, -1)), 0, q.QIFT_ERR_INVALID_ARG),  # table with MNZ
])
def test_linear_ex_table_rules(table, lv, status):
    # M = 0: a valid call is a no-op; invalid tables are rejected first
    assert lin_ex(table, lv=lv, M=0) == status


def test_linear_accepts_asym_and_rejects_a_table_with_it():
    assert lin(lv=4, M=0) == q.QIFT_OK
    assert q._C.qift_w2a4_linear_ex(A16, A16b, 0, 256, A16c, A16d, q.QIFT_F16, 4,
                                    q.level_table_word((0, 1, 2, 3)), 64, A16e, q.QIFT_F32,
                                    None) == q.QIFT_ERR_INVALID_ARG


def test_asym_buffer_sizes_in_the_binding():
    import torch
    assert q.scale_entries(40, "asym") == 80 and q.scale_entries(40, "mnz") == 40
    assert q.default_channels(torch.empty((2, 40)), "asym") == 40
    assert q.default_channels(torch.empty((80,)), "asym") == 40
    bufs = dict(xq=torch.empty((1, 128), dtype=torch.uint8), s_a=torch.empty((1,)),
                codes=torch.empty((48, 16), dtype=torch.int32),
                scales=torch.empty((40,), dtype=torch.float16),
                Y=torch.empty((1, 40)))
    with pytest.raises(ValueError, match="80"):
        q._check_linear_buffers(bufs, 40, "asym", placement=False)
    bufs["scales"] = torch.empty((2, 40), dtype=torch.float16)
    assert q._check_linear_buffers(bufs, 40, "asym", placement=False) == (1, 256)


def test_linear_without_table_rejects_lut():
    assert lin(lv=3, M=0) == q.QIFT_ERR_INVALID_ARG
    assert "table" in q.last_error()


def qw_ex(table, lv, rule, **kw):
    args = dict(W=A16, wd=q.QIFT_F32, N=0, K=256, B=256, codes=A16c, scales=A16d, sd=q.QIFT_F16)
    args.update(kw)
    return q._C.qift_quantize_weights_ex(args["W"], args["wd"], args["N"], args["K"], args["B"],
                                         lv, table, rule, args["codes"], args["scales"], args["sd"],
                                         None)


@pytest.mark.parametrize("table,lv,rule,status", [
    (q.level_table_word((-2, -1, 0, 1)), 3, 0, q.QIFT_OK),
    (q.level_table_word((-2, -1, 0, 1)), 3, 1, q.QIFT_OK),
    (0, 0, 1, q.QIFT_OK),
    (0, 2, 1, q.QIFT_OK),
    (0, 3, 0, q.QIFT_ERR_INVALID_ARG),
    (q.level_table_word((1, 4, -1, -4)), 1, 0, q.QIFT_ERR_INVALID_ARG),
    (0, 0, 2, q.QIFT_ERR_INVALID_ARG),
    (0, 4, 0, q.QIFT_OK),                                  # asymmetric min-max grid
    (0, 4, 1, q.QIFT_ERR_INVALID_ARG),                     # ... takes no searched scale
    (q.level_table_word((0, 1, 2, 3)), 4, 0, q.QIFT_ERR_INVALID_ARG),  # ... nor a table
    (0, 5, 0, q.QIFT_ERR_INVALID_ARG),
])
def test_quantize_weights_ex_rules(table, lv, rule, status):
    assert qw_ex(table, lv, rule) == status


def test_group_accepts_level_tables():
    nbytes = ctypes.c_size_t(0)
    tw = q.level_table_word((3, 10, -3, -10))
    ok = (q.qift_linear_desc * 2)(make_desc(), make_desc(levels=3, reserved=tw))
    assert q._C.qift_linear_group_workspace_bytes(ok, 2, ctypes.byref(nbytes)) == q.QIFT_OK
    bad = (q.qift_linear_desc * 1)(make_desc(levels=3, reserved=0))
    assert q._C.qift_linear_group_workspace_bytes(bad, 1, ctypes.byref(nbytes)) == q.QIFT_ERR_INVALID_ARG


def attn(**kw):
    args = dict(q=A16, qd=q.QIFT_BF16, S=1, T=4096, H=32, D=128, B=128, kq=A16b, ks=A16c,
                vq=A16d, vs=A16e, scale=0.088, out=V(0x60000), od=q.QIFT_F32, ws=V(0x70000),
                wsb=1 << 30)
    args.update(kw)
    return q._C.qift_kv4_attention_decode(args["q"], args["qd"], args["S"], args["T"], args["H"],
                                          args["D"], args["B"], args["kq"], args["ks"], args["vq"],
                                          args["vs"], args["scale"], args["out"], args["od"],
                                          args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), q.QIFT_ERR_UNSUPPORTED),
    (dict(H=65), q.QIFT_ERR_UNSUPPORTED),
    (dict(T=0), q.QIFT_ERR_UNSUPPORTED),
    (dict(S=-1), q.QIFT_ERR_INVALID_ARG),
    (dict(B=96), q.QIFT_ERR_INVALID_ARG),
    (dict(B=256), q.QIFT_ERR_UNSUPPORTED),
    (dict(qd=q.QIFT_I32), q.QIFT_ERR_INVALID_ARG),
    (dict(od=q.QIFT_F16), q.QIFT_ERR_INVALID_ARG),
    (dict(kq=None), q.QIFT_ERR_INVALID_ARG),
    (dict(ws=None), q.QIFT_ERR_INVALID_ARG),
    (dict(kq=V(0x20008)), q.QIFT_ERR_ALIGNMENT),
    (dict(ws=V(0x70010)), q.QIFT_ERR_ALIGNMENT),
    (dict(wsb=64), q.QIFT_ERR_INVALID_ARG),
    (dict(scale=float("nan")), q.QIFT_ERR_INVALID_ARG),
    (dict(S=0, q=None, kq=None), q.QIFT_OK),
])
def test_kv4_attention_rejects(kw, status):
    assert attn(**kw) == status


def test_kv4_attention_workspace_bytes():
    n = ctypes.c_size_t(0)
    assert q._C.qift_kv4_attention_workspace_bytes(1, 4096, 32, 128, ctypes.byref(n)) == q.QIFT_OK
    # about 512 workgroups of two heads: 32 runs of 128 tokens x 32 heads x (2 + 128) floats
    assert n.value == 32 * 32 * 130 * 4
    assert q._C.qift_kv4_attention_workspace_bytes(8, 4096, 32, 128, ctypes.byref(n)) == q.QIFT_OK
    assert n.value == 8 * 4 * 32 * 130 * 4  # 4 runs of 1024 tokens per sequence
    assert q._C.qift_kv4_attention_workspace_bytes(1, 1 << 20, 32, 128, ctypes.byref(n)) == q.QIFT_OK
    assert n.value == 32 * 32 * 130 * 4  # longer runs, not more of them
    assert q._C.qift_kv4_attention_workspace_bytes(1, 1, 64, 128, ctypes.byref(n)) == q.QIFT_OK
    assert n.value == 64 * 130 * 4


def test_group_workspace_and_rejects():
    arr = (q.qift_linear_desc * 3)(make_desc(), make_desc(K=11008, N=4096), make_desc(N=11008))
    nbytes = ctypes.c_size_t(0)
    assert q._C.qift_linear_group_workspace_bytes(arr, 3, ctypes.byref(nbytes)) == q.QIFT_OK
    tiles = 16 + 16 + 43
    assert nbytes.value >= 64 + 3 * 88 + 4 * tiles and nbytes.value % 256 == 0
    bad = (q.qift_linear_desc * 2)(make_desc(), make_desc(M=17))
    assert q._C.qift_linear_group_workspace_bytes(bad, 2, ctypes.byref(nbytes)) == q.QIFT_ERR_UNSUPPORTED
    assert "descriptor 1" in q.last_error()
    bad = (q.qift_linear_desc * 1)(make_desc(reserved=1))
    assert q._C.qift_linear_group_workspace_bytes(bad, 1, ctypes.byref(nbytes)) == q.QIFT_ERR_INVALID_ARG
    # a 2-byte-aligned output suits a bfloat16 plan: sizing accepts it,
    # prepare checks it against the plan's dtype
    odd = (q.qift_linear_desc * 1)(make_desc(Y=0x50002))
    assert q._C.qift_linear_group_workspace_bytes(odd, 1, ctypes.byref(nbytes)) == q.QIFT_OK
    assert q._C.qift_linear_group_prepare(odd, 1, q.QIFT_F16, q.QIFT_F32, V(0x100000), 1 << 20,
                                          ctypes.byref(ctypes.c_int64(0)), None) == q.QIFT_ERR_ALIGNMENT
    bad = (q.qift_linear_desc * 1)(make_desc(codes=0x30008))
    assert q._C.qift_linear_group_workspace_bytes(bad, 1, ctypes.byref(nbytes)) == q.QIFT_ERR_ALIGNMENT
    tiles_out = ctypes.c_int64(0)
    # too small a workspace, or misaligned: rejected before any copy
    assert q._C.qift_linear_group_prepare(arr, 3, q.QIFT_F16, q.QIFT_F32, V(0x100000), 64,
                                          ctypes.byref(tiles_out), None) == q.QIFT_ERR_INVALID_ARG
    assert q._C.qift_linear_group_prepare(arr, 3, q.QIFT_F16, q.QIFT_F32, V(0x100010), 1 << 20,
                                          ctypes.byref(tiles_out), None) == q.QIFT_ERR_ALIGNMENT
    assert q._C.qift_w2a4_linear_grouped(None, 1, None) == q.QIFT_ERR_INVALID_ARG
    assert q._C.qift_w2a4_linear_grouped(V(0x100000), -1, None) == q.QIFT_ERR_INVALID_ARG
    assert q._C.qift_w2a4_linear_grouped(V(0x100000), 0, None) == q.QIFT_OK


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        q.qift_rotate_quant_act(torch.zeros(2, 256), 256)


# --- error-compensated quantization ---------------------------------------------

def hess(**kw):
    args = dict(X=A16, xd=q.QIFT_BF16, S=64, K=256, B=256, acc=0, H=A16b, ws=A16c,
                wsb=1 << 30)
    args.update(kw)
    return q._C.qift_gptq_hessian(args["X"], args["xd"], args["S"], args["K"], args["B"],
                                  args["acc"], args["H"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), q.QIFT_ERR_INVALID_ARG),
    (dict(H=None), q.QIFT_ERR_INVALID_ARG),
    (dict(ws=None), q.QIFT_ERR_INVALID_ARG),
    (dict(xd=q.QIFT_F16), q.QIFT_ERR_INVALID_ARG),
    (dict(S=-1), q.QIFT_ERR_INVALID_ARG),
    (dict(K=100), q.QIFT_ERR_INVALID_ARG),
    (dict(K=16384 + 64), q.QIFT_ERR_UNSUPPORTED),
    (dict(B=3), q.QIFT_ERR_INVALID_ARG),
    (dict(acc=2), q.QIFT_ERR_INVALID_ARG),
    (dict(wsb=100), q.QIFT_ERR_INVALID_ARG),
    (dict(H=V(0x20004)), q.QIFT_ERR_ALIGNMENT),
    (dict(ws=V(0x30080)), q.QIFT_ERR_ALIGNMENT),
])
def test_gptq_hessian_rejects(kw, status):
    assert hess(**kw) == status
    assert q.last_error() != ""


def test_gptq_hessian_accumulate_nothing_is_noop():
    assert hess(S=0, acc=1, X=None, H=None, ws=None) == q.QIFT_OK


def gq(**kw):
    args = dict(W=A16, wd=q.QIFT_F32, N=32, K=256, H=A16b, B=256, lv=0, table=0, rule=0,
                damp=0.01, codes=A16c, scales=A16d, sd=q.QIFT_F16, ws=A16e, wsb=1 << 40)
    args.update(kw)
    return q._C.qift_gptq_quantize_weights(args["W"], args["wd"], args["N"], args["K"],
                                           args["H"], args["B"], args["lv"], args["table"],
                                           args["rule"], args["damp"], args["codes"],
                                           args["scales"], args["sd"], args["ws"], args["wsb"],
                                           None)


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), q.QIFT_ERR_INVALID_ARG),
    (dict(H=None), q.QIFT_ERR_INVALID_ARG),
    (dict(codes=None), q.QIFT_ERR_INVALID_ARG),
    (dict(ws=None), q.QIFT_ERR_INVALID_ARG),
    (dict(damp=0.0), q.QIFT_ERR_INVALID_ARG),
    (dict(damp=-1.0), q.QIFT_ERR_INVALID_ARG),
    (dict(damp=float("nan")), q.QIFT_ERR_INVALID_ARG),
    (dict(damp=float("inf")), q.QIFT_ERR_INVALID_ARG),
    (dict(lv=9), q.QIFT_ERR_INVALID_ARG),
    (dict(lv=3, table=0), q.QIFT_ERR_INVALID_ARG),
    (dict(lv=4), q.QIFT_ERR_INVALID_ARG),      # the asymmetric grid: plain quantizer only
    (dict(table=5), q.QIFT_ERR_INVALID_ARG),
    (dict(rule=7), q.QIFT_ERR_INVALID_ARG),
    (dict(sd=q.QIFT_BF16), q.QIFT_ERR_INVALID_ARG),
    (dict(K=80), q.QIFT_ERR_INVALID_ARG),
    (dict(N=-1), q.QIFT_ERR_INVALID_ARG),
    (dict(wsb=1000), q.QIFT_ERR_INVALID_ARG),
    (dict(N=1 << 30, K=4096), q.QIFT_ERR_UNSUPPORTED),
    (dict(codes=V(0x30008)), q.QIFT_ERR_ALIGNMENT),
    (dict(ws=V(0x50010)), q.QIFT_ERR_ALIGNMENT),
])
def test_gptq_quantize_rejects(kw, status):
    assert gq(**kw) == status
    assert q.last_error() != ""


def test_gptq_empty_is_noop_and_workspace_sizes():
    assert gq(N=0, W=None, codes=None, scales=None, ws=None) == q.QIFT_OK
    assert q.qift_gptq_workspace_bytes(0, 256) == 0
    # two K x K float64 matrices, float64 weights, the errors of a column
    # block, codes and flags
    N, K = 11008, 4096
    b = q.qift_gptq_workspace_bytes(N, K)
    assert 8 * (2 * K * K + N * K) < b <= 8 * (2 * K * K + N * K) + N * K + 8 * 64 * N + K + 8 * 256
    assert q.qift_gptq_hessian_workspace_bytes(100, 256) == 100 * 256 * 8
    assert q.qift_gptq_hessian_workspace_bytes(10000, 256) == 4096 * 256 * 8


def _group_item(**over):
    """Buffers of one grouped linear (M = 2, K = 256, N = 40, MNZ) as CPU
    tensors: the binding checks dtypes and sizes before the device, so each
    mismatch below is reported without a GPU."""
    import torch
    it = dict(xq=torch.zeros((2, 128), dtype=torch.uint8), s_a=torch.ones(2),
              codes=torch.zeros((48, 16), dtype=torch.int32),
              scales=torch.ones(40, dtype=torch.float16),
              Y=torch.zeros((2, 40), dtype=torch.bfloat16), levels="mnz", N=40)
    it.update(over)
    return it


@pytest.mark.parametrize("over,exc,match", [
    (dict(Y="float32"), TypeError, "Y has dtype torch.float32, the call is set up for torch.bfloat16"),
    (dict(scales="float32"), TypeError, "scales has dtype torch.float32"),
    (dict(Y=(2, 39)), ValueError, "Y has 78 elements"),
    (dict(scales=(39,)), ValueError, "scales has 39 elements"),
    (dict(codes=(32, 16)), ValueError, "codes has 512 words, 768 needed"),
    (dict(s_a=(1,)), ValueError, "s_a has 1 elements"),
    (dict(xq="int8"), TypeError, "xq has dtype torch.int8"),
    (dict(levels="int4"), ValueError, "codes has 768 words, 1536 needed"),
    (dict(), ValueError, "must be on a GPU device"),
])
def test_linear_group_rejects_mismatched_items(over, exc, match):
    import torch
    fixed = {}
    base = _group_item()
    for k, v in over.items():
        if k == "levels":
            fixed[k] = v
        elif isinstance(v, str):
            fixed[k] = torch.zeros(base[k].shape, dtype=getattr(torch, v))
        else:
            fixed[k] = torch.zeros(v, dtype=base[k].dtype)
    items = [_group_item(), _group_item(**fixed)]
    with pytest.raises(exc, match=match):
        q.LinearGroup(items, scale_dtype=torch.float16, y_dtype=torch.bfloat16)
    if over:  # the first item is valid: the error names the second
        with pytest.raises(exc, match="item 1"):
            q.LinearGroup(items, scale_dtype=torch.float16, y_dtype=torch.bfloat16)


def test_single_linear_rejects_small_buffers():
    import torch
    it = _group_item(Y=torch.zeros((2, 39), dtype=torch.float32))
    with pytest.raises(ValueError, match="Y has 78 elements"):
        q.qift_w2a4_linear(it["xq"], it["s_a"], it["codes"], it["scales"], Y=it["Y"], N=40)


def attn_noalloc(**kw):
    a = dict(q=A16, qd=q.QIFT_F32, S=1, T=64, H=4, D=128, B=128, kq=A16b, ks=A16c, vq=A16d,
             vs=A16e, scale=0.1, out=V(0x60000), od=q.QIFT_F32)
    a.update(kw)
    return q._C.qift_kv4_attention_decode_noalloc(a["q"], a["qd"], a["S"], a["T"], a["H"], a["D"],
                                                  a["B"], a["kq"], a["ks"], a["vq"], a["vs"],
                                                  a["scale"], a["out"], a["od"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(S=4096, T=4096, H=64), q.QIFT_ERR_UNSUPPORTED),  # partials above the fixed array
    (dict(D=64), q.QIFT_ERR_UNSUPPORTED),
    (dict(kq=None), q.QIFT_ERR_INVALID_ARG),
    (dict(out=None), q.QIFT_ERR_INVALID_ARG),
    (dict(vq=V(0x40008)), q.QIFT_ERR_ALIGNMENT),
    (dict(B=3), q.QIFT_ERR_INVALID_ARG),
    (dict(scale=float("inf")), q.QIFT_ERR_INVALID_ARG),
])
def test_kv4_attention_noalloc_rejects(kw, status):
    """Rejected before any device call (the size limit included)."""
    assert attn_noalloc(**kw) == status
    assert q.last_error() != ""


def test_kv4_attention_noalloc_limit_matches_workspace_rule():
    """The largest partial-result size the fixed array takes is the one the
    workspace entry point would ask for; S = 0 is a no-op."""
    import ctypes as ct
    n = ct.c_size_t(0)
    limit = q.QIFT_ATTENTION_SCRATCH_BYTES
    for S, T, H in ((1, 4096, 32), (8, 4096, 32), (64, 4096, 64), (500, 128, 64), (600, 128, 64)):
        assert q._C.qift_kv4_attention_workspace_bytes(S, T, H, 128, ct.byref(n)) == q.QIFT_OK
        st = attn_noalloc(S=S, T=T, H=H)
        if n.value > limit:
            assert st == q.QIFT_ERR_UNSUPPORTED and "exceed" in q.last_error()
        else:
            assert st != q.QIFT_ERR_UNSUPPORTED  # fits (the launch itself needs a GPU)
    assert attn_noalloc(S=0, q=None, kq=None, out=None) == q.QIFT_OK


def rot_lin(**kw):
    a = dict(X=A16, xd=q.QIFT_BF16, M=1, K=4096, B=4096, xq=A16b, s_a=A16c, codes=A16d,
             scales=A16e, sd=q.QIFT_F16, lv=0, table=0, N=4096, Y=V(0x60000), yd=q.QIFT_BF16)
    a.update(kw)
    return q._C.qift_rotate_w2a4_linear(a["X"], a["xd"], a["M"], a["K"], a["B"], a["xq"], a["s_a"],
                                        a["codes"], a["scales"], a["sd"], a["lv"], a["table"],
                                        a["N"], a["Y"], a["yd"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), q.QIFT_ERR_INVALID_ARG),
    (dict(xq=None), q.QIFT_ERR_INVALID_ARG),
    (dict(codes=None), q.QIFT_ERR_INVALID_ARG),
    (dict(K=4000, B=16), q.QIFT_ERR_INVALID_ARG),          # not a multiple of 64 (linear rule)
    (dict(K=32768, B=4096), q.QIFT_ERR_UNSUPPORTED),       # above the rotation's row limit
    (dict(B=3), q.QIFT_ERR_INVALID_ARG),
    (dict(xd=q.QIFT_F16), q.QIFT_ERR_INVALID_ARG),
    (dict(lv=3), q.QIFT_ERR_INVALID_ARG),                  # level table missing
    (dict(yd=q.QIFT_F16), q.QIFT_ERR_INVALID_ARG),
    (dict(xq=V(0x20008)), q.QIFT_ERR_ALIGNMENT),
])
def test_rotate_linear_rejects(kw, status):
    assert rot_lin(**kw) == status
    assert q.last_error() != ""


def test_rotate_linear_empty_is_noop():
    assert rot_lin(M=0, X=None, xq=None, s_a=None, codes=None, scales=None, Y=None) == q.QIFT_OK
