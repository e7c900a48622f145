"""Benchmark of the rotated W2A4 linear on one MI355X.

Headline (``value``): decode weight-stream GB/s of a LLaMA-7B-shaped stack:
32 decoder layers x 7 linears (q, k, v, o: 4096 -> 4096; gate, up:
4096 -> 11008; down: 11008 -> 4096 with a 256-block Hadamard), 2-bit MNZ codes
with float16 per-channel scales (1.6217 GB of codes + scales), synthetic
N(0, 0.02^2) weights and bf16 N(0, 1) activations with 1% outlier channels
x20. One step = one pass over the whole stack:
  1. rotate + int4-quantize the 96 K=4096 layer inputs and the 32 K=11008
     down_proj inputs (one batched launch),
  2. all 224 W2A4 linears (one grouped decode launch).
value = algorithmic weight-stream bytes of one pass / step time.

Also measured and reported under "extra": the same stack at M = 4, 8, 16;
prefill int8-MFMA TOPS at M = 2048 (up_proj, down_proj; bfloat16 output,
and float32 output under the "_f32_out" keys) and for a 512-token up_proj
chunk; the
LLaMA-3.1-8B-shaped power-of-two layer (decode over 32 layer copies, prefill
at M = 4096); the mixed W2/W4 stack (layers 0-15 MNZ, 16-31 int4) at M = 16;
KV4 of K and V [4096, 32, 128]; the level sets of the abstract (MNZ, PoT, the
standard {-2, -1, 0, 1} set, {+-1, +-2}, a Lloyd-like {+-3, +-10} table,
int4) under the absmax and the searched scale, by the output error of a
LLaMA-7B-shaped q_proj.

``roofline`` describes the dominant kernel of the step (the grouped decode
launch): algorithmic bytes per launch / its mean duration from HIP events on
the launch stream. ``traffic`` comes from the committed rocprofv3 counter
summary when it was taken on the current kernel source, else null.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same stack.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
FP64_PEAK_TFLOPS = 78.6        # MI355X float64 (matrix cores and vector ALUs), TFLOP/s
METRIC = "W2A4 linear: decode weight-stream GB/s + prefill int8 TOPS, % of roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "linear_grouped_decode_llama7b_counters.json")
# the sources the grouped decode kernel is compiled from: the counter summary
# is valid only for the code it was taken on
KERNEL_SRCS = [os.path.join(ROOT, "bit_quantized_fwht_amd", "csrc", f)
               for f in ("linear_decode.hip", "linear_common.h", "qift_internal.h")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # ~25 ms of untimed steps: the clocks settle after the weight quantization
    # that builds the stack (fewer warm-up steps measure 3-5% low)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--m", type=int, default=1, help="tokens per decode step for the headline")
    p.add_argument("--only-headline", action="store_true",
                   help="skip the extra measurements and the CPU baseline (profiling runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run the measurement copy kernel on 1 GiB three times (the "
                        "reference reading for counter runs)")
    p.add_argument("--unit", choices=sorted(UNITS),
                   help="run only this unit --steps times (for profiling runs) and exit")
    return p.parse_args()


def unit_prefill_up_proj(q, torch, dev, steps):
    """LLaMA-7B up_proj prefill: M = 2048, K = 4096, N = 11008, MNZ, bf16 out."""
    import synth_inputs as si
    W = si.device_weights(11008, 4096, seed=5, sigma=0.02, device=dev)
    cw, sw = q.qift_quantize_weights(W, 4096, "mnz", torch.float16)
    X = si.device_activations(2048, 4096, seed=6, device=dev)
    xq, sa, _ = q.qift_rotate_quant_act(X, 4096)
    Y = torch.empty((2048, 11008), dtype=torch.bfloat16, device=dev)
    for _ in range(steps):
        q.qift_w2a4_linear(xq, sa, cw, sw, "mnz", Y=Y)


def unit_prefill_down_proj(q, torch, dev, steps):
    """LLaMA-7B down_proj prefill: M = 2048, K = 11008 (block 256), N = 4096,
    MNZ, bf16 out."""
    import synth_inputs as si
    W = si.device_weights(4096, 11008, seed=5, sigma=0.02, device=dev)
    cw, sw = q.qift_quantize_weights(W, 256, "mnz", torch.float16)
    X = si.device_activations(2048, 11008, seed=6, device=dev)
    xq, sa, _ = q.qift_rotate_quant_act(X, 256)
    Y = torch.empty((2048, 4096), dtype=torch.bfloat16, device=dev)
    for _ in range(steps):
        q.qift_w2a4_linear(xq, sa, cw, sw, "mnz", Y=Y)


def unit_kv4(q, torch, dev, steps):
    """KV4 of K and V [4096, 32, 128] bf16 of one layer (one launch per step)."""
    import synth_inputs as si
    K = si.device_kv(4096, 32, 128, seed=60, device=dev)
    V = si.device_kv(4096, 32, 128, seed=61, device=dev)
    for _ in range(steps):
        q.qift_kv4_quant_kv(K, V, 128)


def unit_attention(q, torch, dev, steps):
    """Decode attention over a KV4 cache: 8 sequences x 4096 tokens, H = 32, D = 128."""
    S, T, H, D = 8, 4096, 32, 128
    g = torch.Generator(device=dev)
    g.manual_seed(109)
    kq = torch.randint(0, 256, (S, T, H, D // 2), dtype=torch.uint8, device=dev, generator=g)
    vq = torch.randint(0, 256, (S, T, H, D // 2), dtype=torch.uint8, device=dev, generator=g)
    ks = torch.rand((S, T, H), device=dev, generator=g) * 0.1
    vs = torch.rand((S, T, H), device=dev, generator=g)
    qv = torch.randn((S, H, D), device=dev, generator=g).to(torch.bfloat16)
    for _ in range(steps):
        q.qift_kv4_attention_decode(qv, kq, ks, vq, vs, D)


def gptq_inputs(torch, dev, N=11008, K=4096, S=2048, extra_tokens=0):
    """LLaMA-7B up_proj weights (11008 x 4096, N(0, 0.02^2)), S correlated
    calibration tokens (bf16) and extra_tokens more from the same draw
    (float32, for evaluation), on the device."""
    import synth_inputs as si
    W = si.device_weights(N, K, seed=5, sigma=0.02, device=dev)
    Xall = si.calibration_activations(S + extra_tokens, K, seed=41)
    X = si.to_bf16(Xall[:S]).to(dev)
    Xe = torch.from_numpy(Xall[S:]).to(dev)
    return W, X, Xe


def unit_gptq(q, torch, dev, steps):
    """Error-compensated quantization of the LLaMA-7B up_proj (11008 x 4096,
    block 4096, MNZ, fp16 scales) with 2048 calibration tokens: H, then the
    codes, per step."""
    W, X, _ = gptq_inputs(torch, dev)
    ws = torch.empty((q.qift_gptq_workspace_bytes(*W.shape),), dtype=torch.uint8, device=dev)
    for _ in range(steps):
        H = q.qift_gptq_hessian(X, 4096)
        q.qift_gptq_quantize_weights(W, H, 4096, "mnz", torch.float16, workspace=ws)


def unit_decode_layer_by_layer(q, torch, dev, steps):
    """The 32-layer dependent decode at M = 1 (per layer: qkv, o, gate+up,
    down, each a rotation call then a linear call) replayed from one HIP
    graph, steps times."""
    items, _ = layer_by_layer_items(q, torch, dev, 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for it in items:
            q.qift_rotate_quant_act(it["X"], it["B"], xq=it["xq"], s_a=it["sa"])
            q.qift_w2a4_linear(it["xq"], it["sa"], it["cw"], it["sw"], "mnz", Y=it["Y"])
    for _ in range(steps):
        g.replay()


def unit_decode_layer_by_layer_fused(q, torch, dev, steps):
    """The same 32-layer dependent decode with each input's rotation and
    linear in one call (qift_rotate_w2a4_linear), replayed steps times."""
    items, _ = layer_by_layer_items(q, torch, dev, 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for it in items:
            q.qift_rotate_w2a4_linear(it["X"], it["B"], it["cw"], it["sw"], "mnz", Y=it["Y"],
                                      xq=it["xq"], s_a=it["sa"])
    for _ in range(steps):
        g.replay()


def unit_decode_single_4096(q, torch, dev, steps):
    """One 4096 x 4096 MNZ linear at M = 1 (bf16 output), steps eager calls,
    each on one of 64 weight copies (268 MB, past the last-level cache)."""
    import synth_inputs as si
    ws = []
    for i in range(64):
        W = si.device_weights(4096, 4096, seed=900 + i, sigma=0.02, device=dev)
        ws.append(q.qift_quantize_weights(W, 4096, "mnz", torch.float16))
        del W
    X = si.device_activations(1, 4096, seed=901, device=dev)
    xq, sa, _ = q.qift_rotate_quant_act(X, 4096)
    Y = torch.empty((1, 4096), dtype=torch.bfloat16, device=dev)
    for i in range(steps):
        cw, sw = ws[i % 64]
        q.qift_w2a4_linear(xq, sa, cw, sw, "mnz", Y=Y)


def unit_rotate_up_proj_input(q, torch, dev, steps):
    """Rotate + int4-quantize the up_proj input of a 2048-token prefill:
    X [2048, 4096] bf16, one 4096-point Hadamard block per row."""
    import synth_inputs as si
    X = si.device_activations(2048, 4096, seed=6, device=dev)
    xq = torch.empty((2048, 2048), dtype=torch.uint8, device=dev)
    sa = torch.empty((2048,), dtype=torch.float32, device=dev)
    for _ in range(steps):
        q.qift_rotate_quant_act(X, 4096, xq=xq, s_a=sa)


def unit_rotate_down_proj_input(q, torch, dev, steps):
    """Rotate + int4-quantize the down_proj input of a 2048-token prefill:
    X [2048, 11008] bf16, blocks of 256 (the matrix-core group kernel)."""
    import synth_inputs as si
    X = si.device_activations(2048, 11008, seed=6, device=dev)
    xq = torch.empty((2048, 5504), dtype=torch.uint8, device=dev)
    sa = torch.empty((2048,), dtype=torch.float32, device=dev)
    for _ in range(steps):
        q.qift_rotate_quant_act(X, 256, xq=xq, s_a=sa)


COPY_BYTES = 1 << 30


def unit_copy(q, torch, dev, steps):
    """The measurement copy kernel on 1 GiB (1 GiB read + 1 GiB written per
    launch): the reference reading for the HBM byte counters."""
    src = torch.empty((COPY_BYTES,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        q.qift_measure_stream(src, dst)


def unit_mfma_i8(q, torch, dev, steps):
    """The int8 matrix-core loop (2048 workgroups x 4096 rounds), steps launches."""
    clk = torch.zeros((4,), dtype=torch.int64, device=dev)
    for _ in range(steps):
        q.qift_measure_mfma_i8(MFMA_ITERS, MFMA_WORKGROUPS, clk)


UNITS = {"prefill_up_proj": unit_prefill_up_proj, "prefill_down_proj": unit_prefill_down_proj,
         "rotate_down_proj_input": unit_rotate_down_proj_input,
         "rotate_up_proj_input": unit_rotate_up_proj_input,
         "copy": unit_copy, "mfma_i8": unit_mfma_i8, "kv4": unit_kv4, "attention": unit_attention,
         "gptq": unit_gptq, "decode_layer_by_layer": unit_decode_layer_by_layer,
         "decode_layer_by_layer_fused": unit_decode_layer_by_layer_fused,
         "decode_single_4096": unit_decode_single_4096}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workload construction
# ---------------------------------------------------------------------------

class DecodeStack:
    """A stack of layers, each a list of (name, K, N, had_block, levels)."""

    def __init__(self, q, torch, layers, M, sigma, dev, seed0=0, scale_dtype=None, y_dtype=None):
        import synth_inputs as si
        self.q, self.torch = q, torch
        self.M = M
        scale_dtype = scale_dtype or torch.float16
        y_dtype = y_dtype or torch.bfloat16
        self.codes, self.scales = [], []
        self.items = []
        self.bytes = 0
        # distinct inputs per layer: the q/k/v input, the o input, the gate/up
        # input, the down input (as in a decoder layer)
        groups = {}
        for li, layer in enumerate(layers):
            for name, K, N, B, lv in layer:
                key = ("attn" if name in ("q_proj", "k_proj", "v_proj") else
                       "o" if name == "o_proj" else "mlp" if name in ("gate_proj", "up_proj") else "down")
                groups.setdefault((K, B), []).append((li, key))
        # one stacked activation buffer per (K, block)
        self.act = {}
        for (K, B), users in groups.items():
            slots = sorted(set(users))
            n_rows = len(slots) * M
            X = si.device_activations(n_rows, K, seed=seed0 + 31 * K + B, device=dev)
            xq = torch.empty((n_rows, K // 2), dtype=torch.uint8, device=dev)
            sa = torch.empty((n_rows,), dtype=torch.float32, device=dev)
            self.act[(K, B)] = dict(X=X, xq=xq, sa=sa, slot={s: i for i, s in enumerate(slots)})
        ytot = sum(M * N for layer in layers for (_, K, N, B, lv) in layer)
        # bfloat16 outputs, the dtype of the model's activations (as for the
        # prefill shapes); set y_dtype=torch.float32 for float32 outputs
        self.y_dtype = y_dtype
        self.Y = torch.empty((ytot,), dtype=y_dtype, device=dev)
        yoff = 0
        for li, layer in enumerate(layers):
            for idx, (name, K, N, B, lv) in enumerate(layer):
                W = si.device_weights(N, K, seed=1000 * li + idx + seed0, sigma=sigma, device=dev)
                c, s = q.qift_quantize_weights(W, B, lv, scale_dtype)
                del W
                key = ("attn" if name in ("q_proj", "k_proj", "v_proj") else
                       "o" if name == "o_proj" else "mlp" if name in ("gate_proj", "up_proj") else "down")
                a = self.act[(K, B)]
                r0 = a["slot"][(li, key)] * M
                Y = self.Y[yoff:yoff + M * N].view(M, N)
                yoff += M * N
                self.items.append(dict(xq=a["xq"][r0:r0 + M], s_a=a["sa"][r0:r0 + M], codes=c,
                                       scales=s, Y=Y, levels=lv))
                self.codes.append(c)
                self.scales.append(s)
                self.bytes += c.numel() * 4 + s.numel() * s.element_size()
        torch.cuda.synchronize()
        self.group = q.LinearGroup(self.items, scale_dtype=scale_dtype, y_dtype=y_dtype)
        # all stacked inputs (one matrix per (K, block)) in one batched launch
        self.rot = q.RotateBatch([(a["X"], B, a["xq"], a["sa"]) for (K, B), a in self.act.items()])

    def rotate_all(self):
        self.rot.run()

    def step(self):
        self.rotate_all()
        self.group.run()


def llama7b_layers(levels="mnz"):
    import synth_inputs as si
    return [[(n, K, N, B, levels) for (n, K, N, B) in si.LLAMA7B_LAYER] for _ in range(si.N_LAYERS)]


def llama31_8b_layers(levels="pot"):
    import synth_inputs as si
    return [[(n, K, N, B, levels) for (n, K, N, B) in si.LLAMA31_8B_LAYER] for _ in range(si.N_LAYERS)]


def mixed_layers():
    import synth_inputs as si
    return [[(n, K, N, B, "mnz" if li < 16 else "int4") for (n, K, N, B) in si.LLAMA7B_LAYER]
            for li in range(si.N_LAYERS)]


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

# untimed calls before each prefill shape is timed: the matrix cores run at a
# lower clock for the first few milliseconds of a burst of GEMMs (as the
# headline's settle phase handles for the decode stream)
PREFILL_WARMUP = 30


def time_fn(torch, fn, reps, warmup=3):
    """Median, min and mean of per-call durations (ms) from HIP events on
    the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(t)), float(t.min()), float(t.mean())


def time_graph(torch, calls, reps=20, warmup=3):
    """Per-call duration (ms: median, min) of the calls in `calls` (a list of
    thunks, each one library call) captured back to back into one HIP graph
    and replayed `reps` times: the GPU time of short launches without the
    host time an eager call leaves between two launches."""
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    med, mn, _ = time_fn(torch, g.replay, reps, warmup=warmup)
    del g
    return med / len(calls), mn / len(calls)


def fused_prefill_shapes(q, torch, dev, levels, M, sigma, shapes):
    """Prefill GEMMs of linears that read the same input, with their weights
    concatenated along N (one launch; per-channel scales make the codes those
    of the separate linears): bfloat16 output, M tokens."""
    import synth_inputs as si
    out = {}
    for name, K, N, B in shapes:
        W = si.device_weights(N, K, seed=5, sigma=sigma, device=dev)
        cw, sw = q.qift_quantize_weights(W, B, levels, torch.float16)
        del W
        X = si.device_activations(M, K, seed=6, device=dev)
        xq, sa, _ = q.qift_rotate_quant_act(X, B)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        med, _, _ = time_fn(torch, lambda: q.qift_w2a4_linear(xq, sa, cw, sw, levels, Y=Y), 20,
                            warmup=PREFILL_WARMUP)
        ops = 2.0 * M * N * K
        out[name] = {"M": M, "K": K, "N": N, "gemm_ms": round(med, 4),
                     "TOPS": round(ops / med / 1e9, 1),
                     "frac_of_int8_peak": round(ops / med / 1e9 / INT8_PEAK_TOPS, 4)}
        del cw, sw, X, xq, sa, Y
        torch.cuda.empty_cache()
    return out


def vendor_int8_gemm(torch, M, K, N, dev):
    """Context only, not this library's path: the vendor int8 GEMM
    (torch._int_mm, int8 [M, K] x int8 [K, N] -> int32, i.e. 8-bit weights
    already expanded in memory, no unpack) on the same shape, best of the
    N-major and K-major weight layouts."""
    try:
        a = torch.randint(-7, 8, (M, K), dtype=torch.int8, device=dev)
        b = torch.randint(-3, 4, (K, N), dtype=torch.int8, device=dev)
        best = None
        for bb in (b, b.t().contiguous().t()):
            torch._int_mm(a, bb)
            med, _, _ = time_fn(torch, lambda: torch._int_mm(a, bb), 20, warmup=PREFILL_WARMUP)
            best = med if best is None else min(best, med)
        ops = 2.0 * M * N * K
        return {"ms": round(best, 4), "TOPS": round(ops / best / 1e9, 1),
                "frac_of_int8_peak": round(ops / best / 1e9 / INT8_PEAK_TOPS, 4)}
    except Exception as e:  # not available in this torch build
        return {"error": repr(e)[:120]}


MFMA_ITERS = 4096
MFMA_WORKGROUPS = 2048   # 8 waves per compute unit, 2 per SIMD


def measured_peaks(q, torch, dev):
    """Measured ceilings of this GPU beside the published ones: the read-only and copy
    rates of the measurement stream kernel (2 GiB read; 1 GiB copied), the
    int8 matrix-core rate of a register-only MFMA loop, and the shader clock
    read during that loop. Median of 20 timed launches each."""
    out = {}
    buf = torch.empty((2 << 30,), dtype=torch.uint8, device=dev)
    med, mn, _ = time_fn(torch, lambda: q.qift_measure_stream(buf), 20, warmup=5)
    out["hbm_read_GBps"] = round(buf.numel() / (med * 1e-3) / 1e9, 1)
    out["hbm_read_GBps_best"] = round(buf.numel() / (mn * 1e-3) / 1e9, 1)
    src, dst = buf[:COPY_BYTES], buf[COPY_BYTES:]
    med, mn, _ = time_fn(torch, lambda: q.qift_measure_stream(src, dst), 20, warmup=5)
    out["hbm_copy_GBps"] = round(2 * COPY_BYTES / (med * 1e-3) / 1e9, 1)
    out["hbm_copy_GBps_best"] = round(2 * COPY_BYTES / (mn * 1e-3) / 1e9, 1)
    del buf, src, dst
    clk = torch.zeros((4,), dtype=torch.int64, device=dev)
    med, mn, _ = time_fn(torch, lambda: q.qift_measure_mfma_i8(MFMA_ITERS, MFMA_WORKGROUPS, clk),
                         20, warmup=5)
    ops = 32.0 * 32768 * MFMA_ITERS * MFMA_WORKGROUPS
    c = clk.cpu().tolist()
    mhz = 100.0 * (c[2] - c[0]) / max(c[3] - c[1], 1)
    out["int8_mfma_TOPS"] = round(ops / (med * 1e-3) / 1e12, 1)
    out["int8_mfma_TOPS_best"] = round(ops / (mn * 1e-3) / 1e12, 1)
    out["shader_clock_MHz_under_mfma"] = round(mhz, 0)
    out["int8_TOPS_per_GHz"] = round(out["int8_mfma_TOPS"] / (mhz / 1e3), 1) if mhz > 0 else None
    out["method"] = (f"qift_measure_stream (64 KB per workgroup, non-temporal 16-byte loads and "
                     f"stores) and "
                     f"qift_measure_mfma_i8 ({MFMA_WORKGROUPS} workgroups x 4 waves x "
                     f"{MFMA_ITERS} x 8 v_mfma_i32_16x16x64_i8); HIP events, median of 20")
    return out


def settle_clocks(fn, torch, min_s=0.3, max_s=3.0, window=20, tol=0.01):
    """Untimed steps until the GPU clocks have settled: at least min_s of
    steps, then until the mean of the last `window` steps is within `tol` of
    the window before (at most max_s). Returns what it did."""
    t0 = time.perf_counter()
    times = []
    reason = "cap"
    while True:
        a = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - a)
        el = time.perf_counter() - t0
        if el >= min_s and len(times) >= 2 * window:
            prev = float(np.mean(times[-2 * window:-window]))
            last = float(np.mean(times[-window:]))
            if abs(last - prev) <= tol * prev:
                reason = "stable"
                break
        if el >= max_s:
            break
    return {"s": round(time.perf_counter() - t0, 3), "steps": len(times), "until": reason,
            "first_step_ms": round(times[0] * 1e3, 4), "last_step_ms": round(times[-1] * 1e3, 4),
            "why": "the clocks ramp after the weight quantization that builds the stack; "
                   "synchronized untimed steps run until the step time is flat, before the "
                   "--warmup steps and the timed steps"}


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(achieved_unit_bytes):
    """HBM bytes per grouped launch from the committed counter summary, if
    it was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    if prof.get("kernel_source_hash") != kernel_source_hash():
        return None
    return prof.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the decode stack
# ---------------------------------------------------------------------------

def cpu_baseline(budget_s=15.0):
    """The oracle on the host cores this process may run on (its affinity
    set), with the BLAS pool limited to that many threads."""
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        out = _cpu_baseline(budget_s)
    out["cores"] = cores
    out["cores_source"] = "len(os.sched_getaffinity(0)); BLAS threads limited to it"
    return out


def _cpu_baseline(budget_s):
    from oracle import qift_oracle as O
    import synth_inputs as si
    done_bytes = 0
    n_lin = 0
    t_total = 0.0
    layer = si.LLAMA7B_LAYER
    # setup (not timed): the timed work does not depend on the code values,
    # so uniform codes of the layer's shapes are packed by the oracle's packer
    prepared = []
    for i, (name, K, N, B) in enumerate(layer):
        codes = si.uniform_codes((N, K), 4, seed=200 + i)
        words = O.pack_weights(codes, "mnz")
        s_w = si.positive_scales(N, 300 + i).astype(np.float16)
        X = si.activations(1, K, seed=400 + i)
        prepared.append((K, N, B, words, s_w, X))
        del codes
    while t_total < budget_s:
        for (K, N, B, words, s_w, X) in prepared:
            t0 = time.perf_counter()
            qa, s_a, _, _ = O.rotate_quant_act(X.astype(np.float64), B)
            codes = O.unpack_weights(words, N, "mnz")
            O.linear(qa, s_a, codes, s_w.astype(np.float64), "mnz")
            t_total += time.perf_counter() - t0
            done_bytes += words.nbytes + s_w.nbytes
            n_lin += 1
            if t_total >= budget_s:
                break
    return {"value": done_bytes / t_total / 1e9, "unit": "GB/s", "kind": "oracle",
            "sample": f"{n_lin} linears of one LLaMA-7B-shaped layer at M=1 (rotate+quantize the "
                      f"input, unpack the oracle-packed 2-bit codes, exact integer matmul), "
                      f"{t_total:.1f} s of CPU time; GB/s of packed codes+scales consumed"}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family/model/stepping
    numbers (a virtualised host may give only a generic name) and the number
    of CPUs online."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if info:
                        break
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in info:
                    info[k] = v
    except OSError:
        return None
    name = info.get("model name", "unknown")
    return (f"{name} (family {info.get('cpu family', '?')}, model {info.get('model', '?')}, "
            f"stepping {info.get('stepping', '?')}; {os.cpu_count()} CPUs online)")


def cpu_oracle_units():
    """The oracle on bounded samples of the other measured units (rotate +
    quantize, the prefill GEMM, KV4), each timed once; a few seconds each."""
    from oracle import qift_oracle as O
    import synth_inputs as si
    out = {"cpu_model": cpu_model()}
    # rotate + quantize: 512 of the 2048 up_proj input rows (K = 4096, block 4096)
    M, K, B = 512, 4096, 4096
    X = si.activations(M, K, seed=6)
    t0 = time.perf_counter()
    O.rotate_quant_act(X.astype(np.float64), B)
    dt = time.perf_counter() - t0
    out["rotate_quant_up_proj_input"] = {"rows": M, "K": K, "block": B, "s": round(dt, 3),
                                         "GBps": round(M * (2.5 * K + 4) / dt / 1e9, 4)}
    # prefill GEMM: 1024 of the 2048 up_proj rows against all 11008 channels
    M, K, N = 1024, 4096, 11008
    qa = si.uniform_int4((M, K), seed=7).astype(np.int8)
    codes = si.uniform_codes((N, K), 4, seed=8)
    s_a = si.positive_scales(M, 9).astype(np.float32)
    s_w = si.positive_scales(N, 10).astype(np.float64)
    t0 = time.perf_counter()
    O.linear(qa, s_a, codes, s_w, "mnz")
    dt = time.perf_counter() - t0
    out["gemm_up_proj"] = {"rows": M, "K": K, "N": N, "s": round(dt, 3),
                           "TOPS": round(2.0 * M * N * K / dt / 1e12, 5)}
    # KV4: 2048 of the 4096 tokens, 32 heads x 128
    T, H, D = 2048, 32, 128
    KV = si.kv(T, H, D, seed=11)
    t0 = time.perf_counter()
    O.kv4_quant(KV, D)
    dt = time.perf_counter() - t0
    out["kv4"] = {"T": T, "H": H, "D": D, "s": round(dt, 3),
                  "GBps": round(T * H * (2.5 * D + 4) / dt / 1e9, 4)}
    # decode attention over a KV4 cache: one sequence of 1024 tokens, 32 heads
    T, H, D = 1024, 32, 128
    kc = si.uniform_int4((T * H, D), seed=12).reshape(1, T, H, D)
    vc = si.uniform_int4((T * H, D), seed=13).reshape(1, T, H, D)
    ksc = si.positive_scales(T * H, 14, 0.01, 0.1).reshape(1, T, H)
    vsc = si.positive_scales(T * H, 15).reshape(1, T, H)
    qv = si.activations(H, D, seed=16, n_outliers=0).reshape(1, H, D)
    t0 = time.perf_counter()
    O.kv4_attention_decode(qv, kc, ksc, vc, vsc, D, 1 / np.sqrt(D))
    dt = time.perf_counter() - t0
    out["kv4_attention"] = {"S": 1, "T": T, "H": H, "D": D, "s": round(dt, 3),
                            "GBps": round(T * H * (D + 8) / dt / 1e9, 4)}
    # the searched (least-squares) weight scale: 16 rows of K = 4096, MNZ
    W = si.weights(16, 4096, seed=17)
    t0 = time.perf_counter()
    O.quantize_weights(W.astype(np.float64), 4096, "mnz", "f16", rule="mse")
    dt = time.perf_counter() - t0
    out["weight_quantizer_searched_scale"] = {"rows": 16, "K": 4096, "s": round(dt, 3),
                                              "rows_per_s": round(16 / dt, 2)}
    # error-compensated quantization of the up_proj: H and its factor from 2048
    # calibration tokens (once per layer input), then 8 of the 11008 channels
    K, S = 4096, 2048
    X = si.calibration_activations(S, K, seed=41)
    t0 = time.perf_counter()
    Hm, dead = O.gptq_hessian(X, K, 0.01)
    factor = (O.gptq_factor(Hm), dead)
    dt_f = time.perf_counter() - t0
    W = si.weights(8, K, seed=18)
    t0 = time.perf_counter()
    O.gptq_quantize_weights(W, X, K, "mnz", "f16", factor=factor)
    dt_r = time.perf_counter() - t0
    out["gptq_up_proj"] = {"K": K, "calibration_tokens": S, "hessian_and_factor_s": round(dt_f, 3),
                           "rows": 8, "rows_s": round(dt_r, 3),
                           "rows_per_s": round(8 / dt_r, 2)}
    return out


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the linear "
              f"would shard by output channel with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_quantized_fwht_amd as q
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q.load_library()

    if args.copy_calibration:
        unit_copy(q, torch, dev, 3)
        torch.cuda.synchronize()

    if args.unit:
        UNITS[args.unit](q, torch, dev, args.steps)
        torch.cuda.synchronize()
        log(f"unit {args.unit}: {args.steps} steps")
        return

    log(f"building LLaMA-7B-shaped W2 stack, M={args.m}")
    t0 = time.time()
    stack = DecodeStack(q, torch, llama7b_layers("mnz"), args.m, 0.02, dev)
    log(f"  built in {time.time() - t0:.1f}s: {len(stack.items)} linears, {stack.bytes / 1e9:.4f} GB")

    settle = settle_clocks(stack.step, torch)
    log(f"  clocks settled: {settle['steps']} steps in {settle['s']} s ({settle['until']})")
    for _ in range(args.warmup):
        stack.step()
    torch.cuda.synchronize()
    # timed region: K steps; events around each grouped launch give the
    # dominant kernel's mean duration
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        stack.rotate_all()
        ev[i][0].record()
        stack.group.run()
        ev[i][1].record()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = t_total * 1e3 / args.steps
    k_ms = np.array([a.elapsed_time(b) for a, b in ev])
    k_mean = float(k_ms.mean())
    value = stack.bytes / (ms_step * 1e-3) / 1e9
    achieved = stack.bytes / (k_mean * 1e-3) / 1e9
    log(f"decode M={args.m}: step {ms_step:.4f} ms ({value:.0f} GB/s); grouped kernel mean "
        f"{k_mean:.4f} ms ({achieved:.0f} GB/s), median {np.median(k_ms):.4f} ms")

    extra = {}
    peaks = None
    if not args.only_headline:
        extra = measure_extras(q, torch, dev, stack, args)
        log("measuring the GPU's own ceilings")
        peaks = measured_peaks(q, torch, dev)
        extra["measured_peaks"] = peaks
        log(f"  read {peaks['hbm_read_GBps']} GB/s, copy {peaks['hbm_copy_GBps']} GB/s, "
            f"int8 {peaks['int8_mfma_TOPS']} TOPS at {peaks['shader_clock_MHz_under_mfma']} MHz")

    traffic = traffic_from_profile(stack.bytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "linear_grouped_kernel (decode, 224 linears)",
                "algorithmic_bytes_per_launch": stack.bytes,
                "mean_launch_ms": round(k_mean, 5)}
    if peaks:
        roofline["measured_read_peak"] = peaks["hbm_read_GBps"]
        roofline["frac_of_measured_read_peak"] = round(achieved / peaks["hbm_read_GBps"], 4)
    cpu = None
    if not args.only_headline and not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        cpu = cpu_baseline()
        cpu["cpu_model"] = cpu_model()
        log(f"  oracle: {cpu['value']:.4f} GB/s on {cpu['cores']} threads")
        if extra:
            extra["cpu_oracle_other_units"] = cpu_oracle_units()
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"llama7b-shaped decode stack, 32 layers x 7 linears, W2 MNZ + fp16 "
                               f"scales, A4, M={args.m} (rotate+quantize 1 batched launch + grouped linear)",
                   "global_batch": args.m, "seq_len": 1, "parallelism": "single-gpu",
                   "weight_stream_bytes": stack.bytes},
        "settle": settle, "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(out), flush=True)


def single_call_graphs(q, torch, st):
    """The stack's linears as single qift_w2a4_linear calls in layer order,
    captured into HIP graphs (all 224, and per distinct shape the calls of
    that shape). Every replay is checked against the eager calls' output
    before timing."""
    def call(it):
        q.qift_w2a4_linear(it["xq"], it["s_a"], it["codes"], it["scales"], it["levels"], Y=it["Y"])

    st.rotate_all()
    for it in st.items:
        call(it)
    torch.cuda.synchronize()
    ref = st.Y.clone()

    def capture(items):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for it in items:
                call(it)
        torch.cuda.synchronize()
        return g

    g_all = capture(st.items)
    for _ in range(3):
        st.Y.zero_()
        torch.cuda.synchronize()
        g_all.replay()
        torch.cuda.synchronize()
        if not torch.equal(st.Y, ref):
            raise RuntimeError("graph replay of the single calls differs from the eager calls")
    med, _, _ = time_fn(torch, g_all.replay, 30, warmup=10)
    out = {"calls": len(st.items), "graph_ms": round(med, 4),
           "GBps": round(st.bytes / med / 1e6, 1),
           "frac_of_hbm_peak": round(st.bytes / med / 1e6 / HBM_PEAK_GBS, 4)}
    del g_all
    shapes = {}
    for it in st.items:
        K, N = it["xq"].shape[1] * 2, it["scales"].shape[0]
        shapes.setdefault((K, N), []).append(it)
    per = {}
    for (K, N), items in shapes.items():
        g = capture(items)
        st.Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for it in items:
            n0 = it["Y"].numel()
            off = it["Y"].data_ptr() - st.Y.data_ptr()
            el = st.Y.element_size()
            if not torch.equal(st.Y[off // el:off // el + n0], ref[off // el:off // el + n0]):
                raise RuntimeError(f"graph replay for shape {K}x{N} differs from the eager calls")
        nbytes = sum(it["codes"].numel() * 4 + it["scales"].numel() * it["scales"].element_size()
                     for it in items)
        med, _, _ = time_fn(torch, g.replay, 30, warmup=10)
        per[f"K={K},N={N}"] = {"calls": len(items), "us_per_call": round(med * 1e3 / len(items), 2),
                               "GBps": round(nbytes / med / 1e6, 1),
                               "frac_of_hbm_peak": round(nbytes / med / 1e6 / HBM_PEAK_GBS, 4)}
        del g
    out["per_shape"] = per
    return out


def kv4_attention_bench(q, torch, dev):
    """Decode attention over a KV4 cache of LLaMA-7B shape (H = 32, D = 128,
    T = 4096 cached tokens) for S = 1 and 8 sequences: bytes read = the K and
    V codes and scales; cycled over enough cache copies to exceed the 256 MB
    last-level cache."""
    T, H, D = 4096, 32, 128
    out = {}
    for S in (1, 8):
        per_set = S * T * H * (D + 8)  # K and V codes (D/2 bytes each) + two float32 scales
        n_sets = max(2, -(-600_000_000 // per_set))
        g = torch.Generator(device=dev)
        g.manual_seed(101 + S)
        sets = []
        for _ in range(n_sets):
            kq = torch.randint(0, 256, (S, T, H, D // 2), dtype=torch.uint8, device=dev, generator=g)
            vq = torch.randint(0, 256, (S, T, H, D // 2), dtype=torch.uint8, device=dev, generator=g)
            ks = torch.rand((S, T, H), device=dev, generator=g) * 0.1
            vs = torch.rand((S, T, H), device=dev, generator=g)
            sets.append((kq, ks, vq, vs))
        qv = torch.randn((S, H, D), device=dev, generator=g).to(torch.bfloat16)
        o = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((q.qift_kv4_attention_workspace_bytes(S, T, H, D),), dtype=torch.uint8,
                         device=dev)
        # one call per cache copy, replayed from a HIP graph (no host time
        # between calls)
        for kq, ks, vq, vs in sets:
            q.qift_kv4_attention_decode(qv, kq, ks, vq, vs, D, out=o, workspace=ws)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for kq, ks, vq, vs in sets:
                q.qift_kv4_attention_decode(qv, kq, ks, vq, vs, D, out=o, workspace=ws)
        torch.cuda.synchronize()
        med, _, _ = time_fn(torch, gr.replay, 20, warmup=3)
        med /= n_sets
        out[f"S={S}"] = {"T": T, "H": H, "D": D, "us_per_call": round(med * 1e3, 2),
                         "GBps": round(per_set / med / 1e6, 1),
                         "frac_of_hbm_peak": round(per_set / med / 1e6 / HBM_PEAK_GBS, 4),
                         "cache_copies_cycled": n_sets}
        del sets, ws, gr
        torch.cuda.empty_cache()
    return out


LEVEL_SETS = [("mnz", "mnz", None), ("pot", "pot", None), ("standard_w2", "lut", (-2, -1, 0, 1)),
              ("pm1_pm2", "lut", (-2, -1, 1, 2)), ("lloyd_like_pm3_pm10", "lut", (3, 10, -3, -10)),
              ("int4", "int4", None)]


def level_set_comparison(q, torch, dev):
    """The level sets of the Qift abstract on one LLaMA-7B-shaped q_proj
    (4096 x 4096, N(0, 0.02^2) weights, block 4096) through the whole W2A4
    path: relative L2 error of the quantized linear's float32 output against
    the float32 product x W^T over 64 tokens (int4 activations in every case),
    with the absmax and the searched (mse) scale, and of the asymmetric
    min-max grid with a zero point; the weight quantizer's time with each rule;
    and the decode / prefill speed of a level table and of the asymmetric
    grid."""
    import synth_inputs as si
    N, K, B, M = 4096, 4096, 4096, 64
    W = si.device_weights(N, K, seed=91, sigma=0.02, device=dev)
    X = si.device_activations(M, K, seed=92, device=dev)
    Yref = X.float() @ W.t()
    xq, sa, _ = q.qift_rotate_quant_act(X, B)
    err, qt = {}, {}
    for name, kind, table in LEVEL_SETS:
        for rule in ("absmax", "mse"):
            cw, sw = q.qift_quantize_weights(W, B, kind, torch.float16, table=table, scale_rule=rule)
            Y = q.qift_w2a4_linear(xq, sa, cw, sw, kind, torch.float32, table=table)
            err[f"{name}_{rule}"] = round(((Y - Yref).norm() / Yref.norm()).item(), 5)
            if name in ("mnz", "standard_w2"):
                med, _, _ = time_fn(torch, lambda: q.qift_quantize_weights(
                    W, B, kind, torch.float16, codes=cw, scales=sw, table=table, scale_rule=rule), 5,
                    warmup=1)
                qt[f"{name}_{rule}_ms"] = round(med, 3)
    # the conventional asymmetric grid with a zero point (min-max step; it has
    # no searched-scale form)
    cw, sw = q.qift_quantize_weights(W, B, "asym", torch.float16)
    Y = q.qift_w2a4_linear(xq, sa, cw, sw, "asym", torch.float32)
    err["asym_minmax"] = round(((Y - Yref).norm() / Yref.norm()).item(), 5)
    med, _, _ = time_fn(torch, lambda: q.qift_quantize_weights(
        W, B, "asym", torch.float16, codes=cw, scales=sw), 5, warmup=1)
    qt["asym_minmax_ms"] = round(med, 3)
    out = {"rel_l2_output_error": err, "weight_quantizer": qt,
           "mnz_beats_standard_at_searched_scale": err["mnz_mse"] < err["standard_w2_mse"],
           "asym_minmax_beats_standard_absmax": err["asym_minmax"] < err["standard_w2_absmax"]}
    # speed: the level-table decode (single call, M = 1) and prefill (M = 2048)
    # against MNZ on the up_proj shape
    Wu = si.device_weights(11008, 4096, seed=93, sigma=0.02, device=dev)
    table = (3, 10, -3, -10)
    spd = {}
    for M in (1, 2048):
        Xu = si.device_activations(M, 4096, seed=94, device=dev)
        xu, su, _ = q.qift_rotate_quant_act(Xu, 4096)
        Yu = torch.empty((M, 11008), dtype=torch.bfloat16, device=dev)
        for name, kind, tb in (("mnz", "mnz", None), ("lut", "lut", table), ("asym", "asym", None)):
            cw, sw = q.qift_quantize_weights(Wu, 4096, kind, torch.float16, table=tb)

            def call():
                q.qift_w2a4_linear(xu, su, cw, sw, kind, Y=Yu, table=tb)

            if M == 1:  # 16 calls replayed from a HIP graph (no host time per call)
                call()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(16):
                        call()
                med, _, _ = time_fn(torch, g.replay, 20, warmup=5)
                spd[f"decode_M1_{name}_us_per_call"] = round(med * 1e3 / 16, 2)
                del g
            else:
                med, _, _ = time_fn(torch, call, 30, warmup=5)
                spd[f"prefill_M2048_{name}_TOPS"] = round(2.0 * M * 11008 * 4096 / med / 1e9, 1)
    out["up_proj_speed"] = spd
    return out


def gptq_bench(q, torch, dev):
    """Error-compensated quantization of the LLaMA-7B up_proj with 2048
    calibration tokens: the time of the Hessian and of the quantizer, their
    float64 work (the symmetric product S K (K + 1); Cholesky and triangular
    inverse 2 K^3 / 3; the column updates N K (K - 1)) as TFLOP/s against the
    float64 peak, and the W2A4 output error of plain and compensated codes on
    64 further tokens of the calibration distribution."""
    N, K, S, B = 11008, 4096, 2048, 4096
    W, X, Xe = gptq_inputs(torch, dev, N, K, S, extra_tokens=64)
    hws = torch.empty((q.qift_gptq_hessian_workspace_bytes(S, K),), dtype=torch.uint8, device=dev)
    ws = torch.empty((q.qift_gptq_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
    H = torch.empty((K, K), dtype=torch.float64, device=dev)
    h_ms, h_min, _ = time_fn(torch, lambda: q.qift_gptq_hessian(X, B, H=H, workspace=hws), 5, 1)
    codes = torch.empty((N, K // 16), dtype=torch.int32, device=dev)
    scales = torch.empty((N,), dtype=torch.float16, device=dev)
    g_ms, g_min, _ = time_fn(torch, lambda: q.qift_gptq_quantize_weights(
        W, H, B, "mnz", torch.float16, codes=codes, scales=scales, workspace=ws), 3, 1)
    h_flop = S * K * (K + 1)
    f_flop = 2 * K ** 3 / 3
    u_flop = N * K * (K - 1)
    # output error against the unquantized product, plain and compensated codes
    ref = (Xe.double() @ W.double().T)
    xq, s_a, _ = q.qift_rotate_quant_act(Xe, B)
    errs = {}
    for name, cs in (("plain", q.qift_quantize_weights(W, B, "mnz", torch.float16)),
                     ("compensated", (codes, scales))):
        Y = q.qift_w2a4_linear(xq, s_a, cs[0], cs[1], "mnz", N=N)
        errs[name] = round(float(torch.linalg.norm(Y.double() - ref) / torch.linalg.norm(ref)), 4)
    torch.cuda.synchronize()
    del ws, hws
    return {"N": N, "K": K, "calibration_tokens": S, "block": B, "levels": "mnz",
            "hessian_ms": round(h_ms, 3), "hessian_TFLOPs": round(h_flop / h_ms / 1e9, 2),
            "quantize_ms": round(g_ms, 3),
            "quantize_TFLOPs": round((f_flop + u_flop) / g_ms / 1e9, 2),
            "quantize_frac_of_fp64_peak": round((f_flop + u_flop) / g_ms / 1e9 / FP64_PEAK_TFLOPS, 4),
            "w2a4_rel_l2_output_error": errs}


LAYER_BY_LAYER_SHAPES = [("qkv", 4096, 12288, 4096), ("o", 4096, 4096, 4096),
                         ("gate_up", 4096, 22016, 4096), ("down", 11008, 4096, 256)]


def layer_by_layer_items(q, torch, dev, M):
    """Weights, inputs and outputs of the 32-layer dependent decode (see
    layer_by_layer_decode). Returns (items, weight bytes)."""
    import synth_inputs as si
    items, nbytes = [], 0
    for li in range(si.N_LAYERS):
        for j, (name, K, N, B) in enumerate(LAYER_BY_LAYER_SHAPES):
            W = si.device_weights(N, K, seed=5000 + 10 * li + j, sigma=0.02, device=dev)
            cw, sw = q.qift_quantize_weights(W, B, "mnz", torch.float16)
            del W
            X = si.device_activations(M, K, seed=7000 + 10 * li + j, device=dev)
            items.append(dict(K=K, N=N, B=B, cw=cw, sw=sw, X=X,
                              xq=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                              sa=torch.empty((M,), dtype=torch.float32, device=dev),
                              Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
            nbytes += cw.numel() * 4 + sw.numel() * 2
    torch.cuda.synchronize()
    return items, nbytes


def layer_by_layer_decode(q, torch, dev, M=1):
    """A dependent, layer-by-layer decode of the LLaMA-7B-shaped stack: per
    layer four linears with the q/k/v and the gate/up weights concatenated
    along N (qkv 4096 -> 12288, o 4096 -> 4096, gate+up 4096 -> 22016, down
    11008 -> 4096), each input rotated and quantized first; 32 layers with
    their own weights and inputs, replayed from one HIP graph: a rotation
    call and a linear call per input."""
    import synth_inputs as si
    items, nbytes = layer_by_layer_items(q, torch, dev, M)

    def separate():
        for it in items:
            q.qift_rotate_quant_act(it["X"], it["B"], xq=it["xq"], s_a=it["sa"])
            q.qift_w2a4_linear(it["xq"], it["sa"], it["cw"], it["sw"], "mnz", Y=it["Y"])

    def fused():
        for it in items:
            q.qift_rotate_w2a4_linear(it["X"], it["B"], it["cw"], it["sw"], "mnz", Y=it["Y"],
                                      xq=it["xq"], s_a=it["sa"])

    out = {"M": M, "layers": si.N_LAYERS, "weight_bytes": nbytes}
    ref = None
    for name, fn in (("rotate_then_linear", separate), ("rotate_linear_one_call", fused)):
        fn()
        torch.cuda.synchronize()
        if ref is None:
            ref = torch.cat([it["Y"].reshape(-1) for it in items])
        elif not torch.equal(torch.cat([it["Y"].reshape(-1) for it in items]), ref):
            raise RuntimeError("the one-call path differs from the two calls")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        for it in items:
            it["Y"].zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(torch.cat([it["Y"].reshape(-1) for it in items]), ref):
            raise RuntimeError("graph replay differs from the eager calls")
        med, _, _ = time_fn(torch, g.replay, 20, warmup=3)
        out[name] = {"ms_per_pass": round(med, 4), "us_per_layer": round(med * 1e3 / si.N_LAYERS, 2),
                     "GBps": round(nbytes / med / 1e6, 1),
                     "frac_of_hbm_peak": round(nbytes / med / 1e6 / HBM_PEAK_GBS, 4)}
        del g
    return out


def measure_extras(q, torch, dev, stack, args):
    import synth_inputs as si
    extra = {}
    # headline stack at other batch sizes (same weights are rebuilt per M)
    dec = {}
    for M in (1, 4, 8, 16):
        if M == args.m:
            s = stack
        else:
            log(f"decode stack M={M}")
            s = DecodeStack(q, torch, llama7b_layers("mnz"), M, 0.02, dev)
        med, mn, _ = time_fn(torch, s.group.run, 30, warmup=30)
        smed, _, _ = time_fn(torch, s.step, 30, warmup=10)
        dec[f"M={M}"] = {"grouped_kernel_ms": round(med, 4), "kernel_GBps": round(s.bytes / med / 1e6, 1),
                         "step_ms": round(smed, 4), "step_GBps": round(s.bytes / smed / 1e6, 1),
                         "frac_of_hbm_peak": round(s.bytes / med / 1e6 / HBM_PEAK_GBS, 4)}
        if s is not stack:
            del s
            torch.cuda.empty_cache()
    extra["decode_llama7b_w2_mnz"] = dec
    log("layer-by-layer decode (concatenated qkv and gate+up)")
    extra["decode_llama7b_layer_by_layer"] = {f"M={M}": layer_by_layer_decode(q, torch, dev, M)
                                              for M in (1, 8)}
    torch.cuda.empty_cache()
    if args.m == 1:
        extra["decode_llama7b_w2_mnz"]["M=1_single_calls_hipgraph"] = single_call_graphs(q, torch, stack)

    # prefill int8 MFMA GEMM, M = 2048; and a 512-token chunk of up_proj (the
    # 64-row tile path: 128-row tiles would leave workgroup slots empty)
    pre = {}
    for name, K, N, B, M in (("up_proj", 4096, 11008, 4096, 2048),
                             ("down_proj", 11008, 4096, 256, 2048),
                             ("up_proj_M512", 4096, 11008, 4096, 512)):
        W = si.device_weights(N, K, seed=5, sigma=0.02, device=dev)
        cw, sw = q.qift_quantize_weights(W, B, "mnz", torch.float16)
        del W
        X = si.device_activations(M, K, seed=6, device=dev)
        xq, sa, _ = q.qift_rotate_quant_act(X, B)
        ops = 2.0 * M * N * K
        pre[name] = {"M": M, "K": K, "N": N}
        # bfloat16 output (the dtype of the layer's input activations) first,
        # then float32 output for comparison
        for tag, ydt in (("", torch.bfloat16), ("_f32_out", torch.float32)):
            Y = torch.empty((M, N), dtype=ydt, device=dev)
            med, _, _ = time_fn(torch, lambda: q.qift_w2a4_linear(xq, sa, cw, sw, "mnz", Y=Y), 30,
                                warmup=PREFILL_WARMUP)
            pre[name].update({"gemm_ms" + tag: round(med, 4), "TOPS" + tag: round(ops / med / 1e9, 1),
                              "frac_of_int8_peak" + tag: round(ops / med / 1e9 / INT8_PEAK_TOPS, 4)})
            del Y
        rmed, _ = time_graph(torch, [lambda: q.qift_rotate_quant_act(X, B, xq=xq, s_a=sa)] * 20)
        rbytes = M * K * 2 + M * K / 2 + 4 * M
        # the same call cycled over copies of X larger than the last-level cache
        ncp = max(2, -(-400_000_000 // (M * K * 2)))
        Xs = [si.device_activations(M, K, seed=600 + i, device=dev) for i in range(ncp)]
        cmed, _ = time_graph(torch, [lambda x=x: q.qift_rotate_quant_act(x, B, xq=xq, s_a=sa)
                                     for x in Xs], reps=10)
        del Xs
        pre[name].update({"rotate_quant_ms": round(rmed, 4),
                          "rotate_quant_GBps": round(rbytes / rmed / 1e6, 1),
                          "rotate_quant_input_cache_resident": True,
                          "rotate_quant_timing": "per call, 20 calls replayed from a HIP graph",
                          "rotate_quant_ms_cycled": round(cmed, 4),
                          "rotate_quant_GBps_cycled": round(rbytes / cmed / 1e6, 1),
                          "TOPS_incl_rotate": round(ops / (pre[name]["gemm_ms"] + rmed) / 1e9, 1)})
        pre[name]["vendor_int8_gemm"] = vendor_int8_gemm(torch, M, K, N, dev)
        del cw, sw, X, xq, sa
    # the linears of a layer that read the same input, as one GEMM over their
    # concatenated weights (as a prefill step runs them): q/k/v and gate/up
    pre["fused"] = fused_prefill_shapes(q, torch, dev, "mnz", 2048, 0.02,
                                        (("qkv_proj", 4096, 3 * 4096, 4096),
                                         ("gate_up_proj", 4096, 2 * 11008, 4096)))
    extra["prefill_llama7b_mnz"] = pre

    # LLaMA-3.1-8B-shaped PoT layer: decode over 32 copies; prefill M = 4096
    log("decode stack LLaMA-3.1-8B PoT")
    s8 = DecodeStack(q, torch, llama31_8b_layers("pot"), 1, 0.015, dev, seed0=77)
    med, _, _ = time_fn(torch, s8.group.run, 30)
    pot = {"decode_M1_32_layers": {"bytes": s8.bytes, "grouped_kernel_ms": round(med, 4),
                                   "kernel_GBps": round(s8.bytes / med / 1e6, 1),
                                   "frac_of_hbm_peak": round(s8.bytes / med / 1e6 / HBM_PEAK_GBS, 4)}}
    del s8
    torch.cuda.empty_cache()
    pf = {}
    for name, K, N, B in si.LLAMA31_8B_LAYER:
        if name in ("k_proj", "o_proj", "up_proj"):
            continue  # same shapes as v_proj, q_proj, gate_proj
        M = 4096
        W = si.device_weights(N, K, seed=8, sigma=0.015, device=dev)
        cw, sw = q.qift_quantize_weights(W, B, "pot", torch.float16)
        del W
        X = si.device_activations(M, K, seed=9, device=dev)
        xq, sa, _ = q.qift_rotate_quant_act(X, B)
        ops = 2.0 * M * N * K
        pf[name] = {"M": M, "K": K, "N": N}
        for tag, ydt in (("", torch.bfloat16), ("_f32_out", torch.float32)):
            Y = torch.empty((M, N), dtype=ydt, device=dev)
            med, _, _ = time_fn(torch, lambda: q.qift_w2a4_linear(xq, sa, cw, sw, "pot", Y=Y), 20,
                                warmup=PREFILL_WARMUP)
            pf[name].update({"gemm_ms" + tag: round(med, 4), "TOPS" + tag: round(ops / med / 1e9, 1),
                             "frac_of_int8_peak" + tag: round(ops / med / 1e9 / INT8_PEAK_TOPS, 4)})
            del Y
        pf[name]["vendor_int8_gemm"] = vendor_int8_gemm(torch, M, K, N, dev)
        if name == "down_proj":
            # the rotation of this GEMM's input (K = 14336, blocks of 1024)
            rmed, _ = time_graph(torch, [lambda: q.qift_rotate_quant_act(X, B, xq=xq, s_a=sa)] * 20)
            rbytes = M * K * 2 + M * K / 2 + 4 * M
            pf[name].update({"rotate_quant_ms": round(rmed, 4),
                             "rotate_quant_GBps": round(rbytes / rmed / 1e6, 1),
                             "rotate_quant_frac_of_hbm_peak": round(rbytes / rmed / 1e6 / HBM_PEAK_GBS, 4),
                             "rotate_quant_timing": "per call, 20 calls replayed from a HIP graph",
                             "TOPS_incl_rotate": round(ops / (pf[name]["gemm_ms"] + rmed) / 1e9, 1)})
        del cw, sw, X, xq, sa
    # k/v (1024 channels each: 256 tiles of 128 x 128, half a round of
    # workgroup slots) and q/k/v as one GEMM each, as a prefill step runs them
    pf["fused"] = fused_prefill_shapes(q, torch, dev, "pot", 4096, 0.015,
                                       (("kv_proj", 4096, 2 * 1024, 4096),
                                        ("qkv_proj", 4096, 4096 + 2 * 1024, 4096)))
    pot["prefill_M4096"] = pf
    extra["llama31_8b_pot"] = pot

    # mixed W2/W4 stack at M = 16
    log("mixed W2/W4 stack M=16")
    sm = DecodeStack(q, torch, mixed_layers(), 16, 0.02, dev, seed0=55)
    med, _, _ = time_fn(torch, sm.group.run, 30)
    smed, _, _ = time_fn(torch, sm.step, 30)
    extra["mixed_w2_w4_llama7b_M16"] = {"bytes": sm.bytes, "grouped_kernel_ms": round(med, 4),
                                        "kernel_GBps": round(sm.bytes / med / 1e6, 1),
                                        "step_ms": round(smed, 4),
                                        "frac_of_hbm_peak": round(sm.bytes / med / 1e6 / HBM_PEAK_GBS, 4)}
    del sm
    torch.cuda.empty_cache()

    # KV4: K and V [4096, 32, 128] bf16 of one layer, cycled over 4 layers'
    # K and V (8 buffer sets, 1.3 GB: more than the caches hold)
    T, H, D = 4096, 32, 128
    sets = [(si.device_kv(T, H, D, seed=60 + i, device=dev),
             torch.empty((T, H, D // 2), dtype=torch.uint8, device=dev),
             torch.empty((T, H), dtype=torch.float32, device=dev)) for i in range(8)]
    layers = [(sets[2 * i], sets[2 * i + 1]) for i in range(4)]
    pair = lambda a, b: q.qift_kv4_quant_kv(a[0], b[0], D, kq=a[1], ks=a[2], vq=b[1], vs=b[2])
    # one call per layer (K and V in one launch), the 4 calls replayed from one HIP graph
    med, _ = time_graph(torch, [lambda a=a, b=b: pair(a, b) for a, b in layers], reps=20)
    # the same tensors with one qift_kv4_quant call each (two launches per layer)
    med2, _ = time_graph(torch, [lambda a=a: q.qift_kv4_quant(a[0], D, kvq=a[1], scales=a[2])
                                 for a in sets], reps=20)
    med2 *= 2
    kv_bytes = 2 * (T * H * D * 2 + T * H * D // 2 + T * H * 4)
    # the pair call on one layer with a 512 MB write between repetitions (the
    # caches hold none of the inputs); only the calls are timed
    flush = torch.empty((1 << 29,), dtype=torch.uint8, device=dev)
    a, b = layers[0]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(20)]
    for i, (e0, e1) in enumerate(evs):
        flush.fill_(i & 0xFF)
        e0.record()
        pair(a, b)
        e1.record()
    torch.cuda.synchronize()
    fmed = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    extra["kv4_llama7b_K_and_V"] = {"T": T, "H": H, "D": D, "ms_K_and_V": round(med, 4),
                                    "GBps": round(kv_bytes / med / 1e6, 1),
                                    "frac_of_hbm_peak": round(kv_bytes / med / 1e6 / HBM_PEAK_GBS, 4),
                                    "note": "qift_kv4_quant_kv (K and V of a layer in one launch), cycled over 4 layers' K and V (1.3 GB), the 4 calls replayed from one HIP graph",
                                    "ms_K_and_V_two_calls": round(med2, 4),
                                    "frac_of_hbm_peak_two_calls": round(kv_bytes / med2 / 1e6 / HBM_PEAK_GBS, 4),
                                    "ms_K_and_V_after_flush": round(fmed, 4),
                                    "GBps_after_flush": round(kv_bytes / fmed / 1e6, 1)}
    del sets, layers, flush
    extra["kv4_attention_decode_llama7b"] = kv4_attention_bench(q, torch, dev)
    extra["level_sets_llama7b_q_proj"] = level_set_comparison(q, torch, dev)
    extra["gptq_llama7b_up_proj"] = gptq_bench(q, torch, dev)
    extra["context"] = {"qtea_lut_kernel_per_token_speedup_vs_fp16": 7.2,
                        "note": "speedup printed for a different (ternary) method; hardware not stated"}
    return extra


if __name__ == "__main__":
    main()
