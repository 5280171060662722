"""Benchmark of the gated delta rule forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--no-extras] [--no-cpu]

One step is one forward of a GatedDeltaNet layer's core over the packed
workload (8192 tokens in 8 samples of seeded random lengths, H_qk = 16,
H_v = 32, K = V = 128, bf16): gates, causal conv1d + SiLU + q/k L2 norm over
the 8192 q|k|v channels, and the chunked delta rule reading q, k, v straight
out of the conv output.  Inputs are resident in HBM before the timed region;
the K timed steps cycle through four copies of the conv input, so no step
finds its input in the caches the previous step filled.  `value` is tokens
per second of the whole step (wall clock over the K steps, the device
synchronised on both sides).

Kernel lines time one library call at a time with HIP events recorded on the
stream it runs on, R times, each after a 1 GiB read of an unrelated buffer
outside the events (so neither L2 nor the 256 MB MALL holds the inputs, and no
foreign dirty lines are left to write back), and report mean, median, p10 and
p90.  Each chunk-call line
carries a roofline block: its algorithmic bytes and flops per call over the
mean duration, against 8 TB/s HBM and against the bf16 matrix-core peak, both
the published 2.5 PFLOP/s and the rate a probe kernel measures in the same
run.  Lines: the packed workload's chunk call with fp32 and bf16 o and its
conv; the long sequence in 8 segments through the segmented entry point and
through the packed call's own split; the batched prefill (whole step, chunk
call, conv); the wide-state workload; the recurrent decode step on 256
sequences; the gated output norm; the chunk call with the norm fused.  The
fp64 CPU oracle is timed on the packed workload on the host.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import gdn_inputs  # noqa: E402

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "GDN fwd tokens/s at H_v=32,K=V=128 bf16; % bf16 MFMA peak"
MAIN = "packed_varlen_bf16_T8192_N8_Hv32_K128"
LONG = "long_segmented_bf16_T32768_P8_Hv32_K128"
BATCHED = "batched_prefill_bf16_B8_T4096_Hv32_K128"
WIDE = "wide_state_bf16_T32768_N4_H64_K128_V256"
FLUSH_BYTES = 1 << 30


def chunk_alg_flops(T, Hqk, Hv, K, V, C=64):
    """Algorithmic flops of the chunked rule per forward (triangles count half, Gram once per qk head)."""
    per_tok = 2 * (Hqk * C * K + Hv * (C * K / 2 + C * V + 3 * K * V + C * C / 6))
    return per_tok * T


def chunk_alg_bytes(T, N, Hqk, Hv, K, V, o_bytes, in_bytes=2, s0=False):
    """HBM bytes the chunk kernel must move at least: q, k, v in, g and beta in, o out, states."""
    per_tok = in_bytes * (2 * Hqk * K + Hv * V) + 8 * Hv + o_bytes * Hv * V
    states = N * Hv * K * V * 4 * (2 if s0 else 1)
    return per_tok * T + states


def conv_alg_bytes(T, C, in_bytes=2):
    return 2 * in_bytes * T * C


def conv_alg_flops(T, C, width):
    """conv taps, SiLU (exp, add, divide) and the L2 norm (square, sum, scale) per channel and token."""
    return (2 * width + 6) * T * C


def conv_chunk_alg_bytes(T, N, Hqk, Hv, K, V, o_bytes, in_bytes=2, s0=False):
    """The fused conv + chunk call: raw q | k | v channels in, gates in, o out, states (weights negligible)."""
    return chunk_alg_bytes(T, N, Hqk, Hv, K, V, o_bytes, in_bytes, s0)


CHUNK_SOURCES = ("chunk_prep.hip", "chunk_bf16.hip", "compose.hip", "split_plan.cpp", "api.cpp", "device_common.h",
                 "kernels.h")


def sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_deltanet_linear_chunk_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload, key="traffic_bytes_per_launch"):
    """HBM bytes per chunk call (FETCH_SIZE + WRITE_SIZE of its kernels, scaled by a copy
    calibration) from the committed rocprofv3 summary of that workload (`key` names the call when
    the summary covers several); None when the kernel sources have changed since the counters were
    taken, or when there is no summary."""
    path = os.path.join(ROOT, "profiles", "chunk_fwd_%s.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|", "`")):
                name, _, val = line.partition(":")
                fields[name.strip()] = val.strip()
    if fields.get("chunk_sources_sha256_16") != sources_digest(CHUNK_SOURCES):
        return None
    try:
        return int(fields[key])
    except (KeyError, ValueError):
        return None


def _torch():
    import torch

    return torch


class Flush:
    """A 1 GiB buffer read between timed reps (outside the events): it evicts L2 and the MALL and,
    being a read, leaves no dirty lines whose write-back the next timed call would pay for (the
    previous call's own outputs are written back during the flush)."""

    def __init__(self):
        torch = _torch()
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
        self.out = torch.zeros(1, dtype=torch.float32, device="cuda:0")

    def __call__(self):
        torch = _torch()
        torch.sum(self.buf, dim=0, keepdim=True, out=self.out)


def time_call(call, reps, flush):
    """Durations (ms) of `call` over reps, each after a flush, from HIP events on the current stream.
    One untimed call first: a kernel's first launch in a process also loads its code."""
    torch = _torch()
    call()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(reps):
        flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def summary(ms):
    ms = np.asarray(ms, dtype=np.float64)
    return {"mean_ms": float(ms.mean()), "median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
            "p90_ms": float(np.percentile(ms, 90)), "reps": int(ms.size)}


def roofline(alg_bytes, alg_flops, st, kernel, mfma_peak_tflops, traffic=None):
    """Roofline block of one call: algorithmic bytes and flops over its mean duration."""
    sec = st["mean_ms"] * 1e-3
    achieved = alg_bytes / sec / 1e9
    tflops = alg_flops / sec / 1e12
    out = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "kernel": kernel,
           "alg_bytes_per_launch": int(alg_bytes), "alg_flops_per_launch": float(alg_flops),
           "avg_launch_ms": st["mean_ms"], "median_ms": st["median_ms"], "p10_ms": st["p10_ms"],
           "p90_ms": st["p90_ms"], "reps": st["reps"], "mfma_tflops": tflops,
           "mfma_frac_published_peak": tflops / PEAK_BF16_TFLOPS}
    if mfma_peak_tflops:
        out["mfma_frac_measured_peak"] = tflops / mfma_peak_tflops
    if traffic:
        out["traffic_over_alg"] = traffic / alg_bytes
    return out


def measure_mfma_peak():
    """Dense bf16 matrix-core rate (TFLOP/s) of this device from the probe kernel; None without it."""
    torch = _torch()
    path = os.path.join(ROOT, "gated_deltanet_linear_chunk_amd", "libgdn_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.gdn_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.gdn_probe_mfma_bf16.restype = ctypes.c_int
    lib.gdn_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.gdn_probe_mfma_bf16_flops.restype = ctypes.c_double
    props = torch.cuda.get_device_properties(0)
    blocks = 8 * props.multi_processor_count  # 32 waves per compute unit
    iters = 4096
    out = torch.empty(blocks, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        rc = lib.gdn_probe_mfma_bf16(blocks, iters, out.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError("probe launch failed (%d)" % rc)

    call()
    torch.cuda.synchronize()
    ms = time_call(call, 10, lambda: None)
    flops = lib.gdn_probe_mfma_bf16_flops(blocks, iters)
    return flops / (float(np.median(ms)) * 1e-3) / 1e12


def rotated_inputs(x, copies):
    """`copies` separate buffers holding x (the first is x itself)."""
    return [x] + [x.clone() for _ in range(copies - 1)]


def build_pipeline(w, d, o_dtype, rotate=4):
    """Device inputs and the calls of a conv + gates + chunk workload."""
    torch = _torch()
    import gated_deltanet_linear_chunk_amd as gdn

    dev = torch.device("cuda:0")
    T = w.total_tokens
    Hqk, Hv, K, V = w.Hqk, w.Hv, w.K, w.V
    C = 2 * Hqk * K + Hv * V
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)  # noqa: E731
    B = w.batch_rows
    L = T // B
    x0 = bf(d["x"]).reshape(B, L, C) if B > 1 else bf(d["x"])
    xs = rotated_inputs(x0, rotate)
    cw, cb = bf(d["conv_w"]), bf(d["conv_bias"])
    a, b = f32(d["a"]).reshape(B, L, Hv), f32(d["b"]).reshape(B, L, Hv)
    A_log, dt_bias = f32(d["A_log"]), f32(d["dt_bias"])
    cu = None if B > 1 else torch.from_numpy(d["cu_seqlens"]).to(dev)
    cu_host = None if B > 1 else d["cu_seqlens"]
    s0 = f32(d["s0"]) if "s0" in d else None
    state = {"i": 0}

    def conv(x=x0):
        return gdn.gdn_conv1d_fwd(x, cw, cb, cu_seqlens=cu, cu_seqlens_host=cu_host, l2norm_channels=2 * Hqk * K,
                                  head_dim=K)

    def qkv(y):
        y = y.reshape(B, L, C)
        q = y[..., : Hqk * K].unflatten(-1, (Hqk, K))
        k = y[..., Hqk * K : 2 * Hqk * K].unflatten(-1, (Hqk, K))
        v = y[..., 2 * Hqk * K :].unflatten(-1, (Hv, V))
        return q, k, v

    def chunk(q, k, v, g, beta, od=o_dtype):
        return gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu, cu_seqlens_host=cu_host,
                                 o_dtype=od)

    def step():
        x = xs[state["i"] % len(xs)]
        state["i"] += 1
        q, k, v = qkv(conv(x))
        g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
        return chunk(q, k, v, g, beta)

    def step_on(x):
        q, k, v = qkv(conv(x))
        g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
        return chunk(q, k, v, g, beta)

    def chunk_inputs():
        q, k, v = qkv(conv())
        g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
        return q, k, v, g, beta

    step_fns = [lambda x=x: step_on(x) for x in xs]
    return {"step": step, "step_fns": step_fns, "conv": conv, "chunk": chunk, "chunk_inputs": chunk_inputs, "C": C}


def build_conv_chunk(w, d):
    """The fused call of a workload (gates, conv and chunk rule in one call), on its raw inputs."""
    torch = _torch()
    import gated_deltanet_linear_chunk_amd as gdn

    dev = torch.device("cuda:0")
    T = w.total_tokens
    Hv = w.Hv
    C = 2 * w.Hqk * w.K + Hv * w.V
    B = w.batch_rows
    L = T // B
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)  # noqa: E731
    xs = rotated_inputs(bf(d["x"]).reshape(B, L, C), 4)
    cw, cb = bf(d["conv_w"]), bf(d["conv_bias"])
    a, b = f32(d["a"]).reshape(B, L, Hv), f32(d["b"]).reshape(B, L, Hv)
    A_log, dt_bias = f32(d["A_log"]), f32(d["dt_bias"])
    cu = None if B > 1 else torch.from_numpy(d["cu_seqlens"]).to(dev)
    cu_host = None if B > 1 else d["cu_seqlens"]
    s0 = f32(d["s0"]) if "s0" in d else None
    state = {"i": 0}

    def fused(x):
        return gdn.gdn_conv_chunk_fwd(x, cw, a, b, A_log, dt_bias, Hqk=w.Hqk, K=w.K, bias=cb, initial_state=s0,
                                      cu_seqlens=cu, cu_seqlens_host=cu_host, o_dtype=torch.float32)

    def step():
        x = xs[state["i"] % len(xs)]
        state["i"] += 1
        return fused(x)

    return {"step": step, "call": lambda: fused(xs[0]), "C": C}


def build_chunk_only(w, d, o_dtype, mode="plain"):
    """The chunk call of a workload with q, k, v given (mode plain, segmented or gated_norm)."""
    torch = _torch()
    import gated_deltanet_linear_chunk_amd as gdn

    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)  # noqa: E731
    q, k, v = bf(d["q"])[None], bf(d["k"])[None], bf(d["v"])[None]
    g, beta = gdn.gdn_gate_fwd(f32(d["a"])[None], f32(d["b"])[None], f32(d["A_log"]), f32(d["dt_bias"]))
    if mode == "segmented":
        off = d["seg_offsets"]
        off_dev = torch.from_numpy(off).to(dev)
        ws = torch.empty(gdn.gdn_segmented_workspace_bytes(w.total_tokens, len(off) - 1, w.Hv, w.K, w.V),
                         dtype=torch.uint8, device=dev)
        return lambda: gdn.gdn_chunk_fwd_segmented(q, k, v, g, beta, off_dev, off, o_dtype=o_dtype, workspace=ws)
    cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
    if mode == "gated_norm":
        rng = np.random.default_rng(5)
        z = bf(rng.standard_normal((w.total_tokens, w.Hv, w.V)).astype(np.float32))[None]
        nw = f32(rng.uniform(0.5, 1.5, w.V))
        return lambda: gdn.gdn_chunk_fwd_gated_norm(q, k, v, g, beta, z, norm_weight=nw, cu_seqlens=cu,
                                                    cu_seqlens_host=d["cu_seqlens"], o_dtype=o_dtype)
    return lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens"],
                                     o_dtype=o_dtype)


# Lines whose chunk call --counters runs alone: workload, build_chunk_only mode, o dtype.  The
# committed summaries divide each counter's sum over the library's chunk kernels by the calls.
COUNTER_LINES = {
    "bf16o": (MAIN, "plain", "bfloat16"),
    "segmented": (LONG, "segmented", "float32"),
    "split": (LONG, "plain", "float32"),
    "wide": (WIDE, "plain", "float32"),
}
COUNTER_CALLS = 11

DECODE_N = 256  # sequences per decode step


def decode_alg_bytes(N, Hqk, Hv, K, V, in_bytes=2, o_bytes=4):
    """HBM bytes one decode step must move: every state read and written once, plus the token's inputs and o."""
    return N * (Hv * K * V * 4 * 2 + in_bytes * (2 * Hqk * K + Hv * V) + 8 * Hv + o_bytes * Hv * V)


def build_decode(N, Hqk, Hv, K, V):
    """One decode token for each of N sequences (bf16 q/k/v, fp32 states of N(0, 0.02) updated in place)."""
    torch = _torch()
    import gated_deltanet_linear_chunk_amd as gdn

    d = gdn_inputs.small(4242, [1] * N, Hqk, Hv, K, V, "bf16", s0_std=0.02, name="decode")
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)  # noqa: E731
    q, k, v = bf(d["q"]), bf(d["k"]), bf(d["v"])
    g, beta = gdn.gdn_gate_fwd(f32(d["a"]), f32(d["b"]), f32(d["A_log"]), f32(d["dt_bias"]))
    state = f32(d["s0"])
    return lambda: gdn.gdn_decode_step(q, k, v, g, beta, state, o_dtype=torch.float32)


def build_gated_norm(rows, V):
    """The gated output norm over rows of V values: fp32 o (as the chunk rule writes it), bf16 z, bf16 y."""
    torch = _torch()
    import gated_deltanet_linear_chunk_amd as gdn

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(77)
    o = torch.randn((rows, V), generator=gen, device=dev, dtype=torch.float32)
    z = torch.randn((rows, V), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = torch.rand((V,), generator=gen, device=dev, dtype=torch.float32) + 0.5
    y = torch.empty((rows, V), dtype=torch.bfloat16, device=dev)
    return lambda: gdn.gdn_gated_rmsnorm_fwd(o, z, w, eps=1e-6, out=y)


def timed_steps(step, steps, warmup):
    """Wall-clock seconds per step over exactly `steps` steps after `warmup` untimed ones."""
    torch = _torch()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def graph_steps(fns, steps, warmup):
    """Seconds per step over `steps` replays of HIP graphs of the step, one graph per step function
    (one per input copy, replayed in turn), after `warmup` untimed replays.  Each function runs
    eagerly first (the library's one-time set-up and the planner's cache), then is captured."""
    torch = _torch()
    for f in fns:
        f()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for f in fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    del graphs
    return sec


def cpu_baseline(w, d):
    """The fp64 oracle on the same packed workload, on this host's cores."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    q, k, v = oracle.pipeline_activations(d["x"], d["conv_w"], d["conv_bias"], d["cu_seqlens"], w.Hqk, w.Hv, w.K,
                                          w.V, threads=threads)
    g, beta = oracle.gates(d["a"], d["b"], d["A_log"], d["dt_bias"])
    oracle.recurrence(q, k, v, g, beta, None, d["cu_seqlens"], threads=threads)
    dt = time.perf_counter() - t0
    return {
        "value": w.total_tokens / dt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "the whole packed workload (8192 tokens, 8 samples, 32 v-heads): fp64 conv1d + SiLU + L2 norm, "
                  "gates, token recurrence; %.1f s wall" % dt,
    }


SPLIT_KERNELS = ("chunk_prep_kernel (stores the plan) + chunk_scan_kernel<{0},8,mixed> (pass 1) + compose_kernel + "
                 "chunk_scan_kernel<{0},8> (pass 2)")


def pipeline_lines(name, w, d, o_dtype, o_bytes, reps, flush, peak, steps, warmup, main=False):
    """Whole-step rate, chunk-call roofline and conv line of a conv + gates + chunk workload."""
    torch = _torch()
    p = build_pipeline(w, d, o_dtype)
    T, N = w.total_tokens, (w.batch_rows if w.batch_rows > 1 else w.n_samples)
    s0 = "s0" in d
    sec = timed_steps(p["step"], steps, warmup)
    sec_graph = graph_steps(p["step_fns"], steps, warmup)
    q, k, v, g, beta = p["chunk_inputs"]()
    packed = w.batch_rows == 1
    kernels = SPLIT_KERNELS.format(0 if o_bytes == 4 else 1) if packed else \
        "chunk_prep_kernel + chunk_scan_kernel<%d,8>" % (0 if o_bytes == 4 else 1)
    st = summary(time_call(lambda: p["chunk"](q, k, v, g, beta), reps, flush))
    lines = {
        "step": {"tokens_per_s": T / sec, "ms_per_step": sec * 1e3, "steps": steps, "warmup": warmup,
                 "graph_tokens_per_s": T / sec_graph, "graph_ms_per_step": sec_graph * 1e3},
        "chunk": roofline(chunk_alg_bytes(T, N, w.Hqk, w.Hv, w.K, w.V, o_bytes, s0=s0),
                          chunk_alg_flops(T, w.Hqk, w.Hv, w.K, w.V),
                          st, "gdn_chunk_fwd (%s) = %s" % ("segment-split path" if packed else "batched rows", kernels),
                          peak, profiled_traffic(name) if o_bytes == 4 else None),
    }
    if main:
        other = torch.bfloat16 if o_bytes == 4 else torch.float32
        ob = 2 if o_bytes == 4 else 4
        st2 = summary(time_call(lambda: p["chunk"](q, k, v, g, beta, other), reps, flush))
        lines["chunk_%so" % ("bf16" if ob == 2 else "f32")] = roofline(
            chunk_alg_bytes(T, N, w.Hqk, w.Hv, w.K, w.V, ob, s0=s0), chunk_alg_flops(T, w.Hqk, w.Hv, w.K, w.V), st2,
            "gdn_chunk_fwd with %s o" % ("bf16" if ob == 2 else "fp32"), peak,
            profiled_traffic(name + "_bf16o") if ob == 2 else None)
    cst = summary(time_call(p["conv"], reps, flush))
    cb = conv_alg_bytes(T, p["C"])
    lines["conv1d"] = dict(cst, hbm_frac=cb / (cst["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                           achieved_gbs=cb / (cst["mean_ms"] * 1e-3) / 1e9, alg_bytes=cb,
                           kernel="conv1d_kernel (bf16, fast rounding)")
    del p, q, k, v, g, beta
    torch.cuda.empty_cache()
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=30, help="flushed reps per kernel line")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--o-dtype", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--only", default="",
                    help="comma-separated extras to run (segmented, split, batched, wide, decode, norm, fused, "
                         "conv_chunk); "
                         "default all")
    ap.add_argument("--counters", choices=list(COUNTER_LINES), default="",
                    help="only make %d chunk calls of that line (nothing else of the library runs), for "
                         "rocprofv3 counter passes" % COUNTER_CALLS)
    ap.add_argument("--copy-only", type=int, default=0,
                    help="only run N plain 256 MiB device copies (counter calibration for profiles)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the path shards by head, "
              "sequence or segment; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    torch = _torch()
    import gated_deltanet_linear_chunk_amd as gdn

    gdn.load_library()
    if args.copy_only:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.copy_only):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each": 256 << 20, "copies": args.copy_only}))
        return

    o_dtype = torch.float32 if args.o_dtype == "f32" else torch.bfloat16
    o_bytes = 4 if args.o_dtype == "f32" else 2
    if args.counters:
        name, mode, od = COUNTER_LINES[args.counters]
        wc = gdn_inputs.WORKLOADS[name]
        fn = build_chunk_only(wc, gdn_inputs.draw(wc, with_qkv=True), getattr(torch, od), mode)
        for _ in range(COUNTER_CALLS):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"counters_line": args.counters, "workload": name, "calls": COUNTER_CALLS}))
        return
    reps = max(30, args.reps)
    flush = Flush()
    peak = measure_mfma_peak()
    w = gdn_inputs.WORKLOADS[MAIN]
    d = gdn_inputs.draw(w, with_qkv=False)
    main_lines = pipeline_lines(MAIN, w, d, o_dtype, o_bytes, reps, flush, peak, args.steps, args.warmup, main=True)
    T, N = w.total_tokens, w.n_samples
    step = main_lines["step"]
    chunk = main_lines["chunk"]
    result = {
        "metric": METRIC,
        "value": step["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step["ms_per_step"],
        "ms_per_step_graph_replay": step["graph_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; packed lengths by a flat Dirichlet draw)",
        "config": {"workload": MAIN, "global_batch": N, "seq_len": T, "parallelism": "none (1 GPU)",
                   "H_qk": w.Hqk, "H_v": w.Hv, "K": w.K, "V": w.V, "chunk": 64, "conv_width": 4,
                   "o_dtype": args.o_dtype, "step": "gates + conv1d/SiLU/L2 + chunked rule",
                   "launch": "eager (HIP graph replay of the same step also reported)"},
        "mfma_frac_chunk": chunk["mfma_frac_published_peak"],
        "mfma_peak_measured_tflops": peak,
        "roofline": chunk,
        "kernels_ms": {"chunk": chunk["avg_launch_ms"], "conv1d": main_lines["conv1d"]["mean_ms"]},
        "conv1d_hbm_frac": main_lines["conv1d"]["hbm_frac"],
        "lines": {"%s[%s]" % (MAIN, k): v for k, v in main_lines.items() if k != "step"},
    }
    print("main lines done", file=sys.stderr, flush=True)

    if not args.no_extras:
        only = set(x for x in args.only.split(",") if x)
        want = lambda key: not only or key in only  # noqa: E731
        lines = result["lines"]
        wl = gdn_inputs.WORKLOADS[LONG]
        if want("segmented") or want("split"):
            dl = gdn_inputs.draw(wl, with_qkv=True)
            fl = chunk_alg_flops(wl.total_tokens, wl.Hqk, wl.Hv, wl.K, wl.V)
            by = chunk_alg_bytes(wl.total_tokens, 1, wl.Hqk, wl.Hv, wl.K, wl.V, o_bytes)
            if want("segmented"):
                st = summary(time_call(build_chunk_only(wl, dl, o_dtype, "segmented"), reps, flush))
                lines["%s[segmented entry point]" % LONG] = roofline(
                    by, fl, st, "gdn_chunk_fwd_segmented (8 segments) = " + SPLIT_KERNELS.format(0 if o_bytes == 4 else 1), peak,
                    profiled_traffic(LONG, "traffic_bytes_per_launch_segmented") if o_bytes == 4 else None)
            if want("split"):
                st = summary(time_call(build_chunk_only(wl, dl, o_dtype), reps, flush))
                lines["%s[planner-split packed call]" % LONG] = roofline(
                    by, fl, st, "gdn_chunk_fwd with host offsets (one sample; the planner splits it)", peak,
                    profiled_traffic(LONG, "traffic_bytes_per_launch_split") if o_bytes == 4 else None)
            del dl
            torch.cuda.empty_cache()
            print("long-sequence lines done", file=sys.stderr, flush=True)
        if want("batched"):
            wb = gdn_inputs.WORKLOADS[BATCHED]
            db = gdn_inputs.draw(wb, with_qkv=False)
            for k, v in pipeline_lines(BATCHED, wb, db, o_dtype, o_bytes, reps, flush, peak,
                                       max(3, args.steps // 2), 2).items():
                lines["%s[%s]" % (BATCHED, k)] = v
            del db
            print("batched lines done", file=sys.stderr, flush=True)
        if want("wide"):
            ww = gdn_inputs.WORKLOADS[WIDE]
            dw = gdn_inputs.draw(ww, with_qkv=True)
            st = summary(time_call(build_chunk_only(ww, dw, o_dtype), reps, flush))
            lines["%s[chunk]" % WIDE] = roofline(
                chunk_alg_bytes(ww.total_tokens, ww.n_samples, ww.Hqk, ww.Hv, ww.K, ww.V, o_bytes),
                chunk_alg_flops(ww.total_tokens, ww.Hqk, ww.Hv, ww.K, ww.V), st,
                "gdn_chunk_fwd (V = 256: two column tiles per head)", peak,
                profiled_traffic(WIDE) if o_bytes == 4 else None)
            del dw
            torch.cuda.empty_cache()
            print("wide line done", file=sys.stderr, flush=True)
        if want("decode"):
            st = summary(time_call(build_decode(DECODE_N, 16, 32, 128, 128), reps, flush))
            nbytes = decode_alg_bytes(DECODE_N, 16, 32, 128, 128)
            lines["decode_bf16_N%d_Hv32_K128[decode step]" % DECODE_N] = dict(
                st, tokens_per_s=DECODE_N / (st["mean_ms"] * 1e-3),
                hbm_frac=nbytes / (st["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, alg_bytes=nbytes)
            torch.cuda.empty_cache()
        if want("norm"):
            rows = w.total_tokens * w.Hv
            st = summary(time_call(build_gated_norm(rows, w.V), reps, flush))
            nbytes = rows * w.V * (4 + 2 + 2)
            lines["gated_norm_f32o_bf16z_T8192_Hv32_V128[norm]"] = dict(
                st, hbm_frac=nbytes / (st["mean_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, alg_bytes=nbytes)
            torch.cuda.empty_cache()
        if want("fused"):
            # the chunk forward with the gated norm applied as the scan writes o (bf16 z and y)
            dx = gdn_inputs.draw(w, with_qkv=True)
            st = summary(time_call(build_chunk_only(w, dx, torch.bfloat16, "gated_norm"), reps, flush))
            lines["%s[chunk + gated norm fused, bf16 z and y]" % MAIN] = dict(
                st, tokens_per_s=w.total_tokens / (st["mean_ms"] * 1e-3))
            del dx
            torch.cuda.empty_cache()

        if want("conv_chunk"):
            # conv1d + SiLU + q/k L2 norm in the chunk prep of the MFMA path (gdn_conv_chunk_fwd)
            fc = build_conv_chunk(w, d)
            sec = timed_steps(fc["step"], max(3, args.steps // 4), 1)
            st = summary(time_call(fc["call"], max(3, reps // 6), flush))
            C = fc["C"]
            fused_b = conv_chunk_alg_bytes(T, N, w.Hqk, w.Hv, w.K, w.V, o_bytes, s0="s0" in d)
            unfused_b = conv_alg_bytes(T, C) + 16 * w.Hv * T + chunk_alg_bytes(T, N, w.Hqk, w.Hv, w.K, w.V, o_bytes,
                                                                               s0="s0" in d)
            flops = chunk_alg_flops(T, w.Hqk, w.Hv, w.K, w.V) + conv_alg_flops(T, C, w.conv_width)
            kern = ("chunk_prep_conv_kernel (stores the plan and the activations) + chunk_scan_kernel<0,8,mixed> + "
                    "compose_kernel + chunk_scan_kernel<0,8>")
            lines["%s[conv + chunk fused, conv in the chunk prep]" % MAIN] = dict(
                st, step_tokens_per_s=T / sec, kernel=kern,
                bytes_per_token_fused=fused_b / T, bytes_per_token_unfused=unfused_b / T,
                achieved_gbs=fused_b / (st["median_ms"] * 1e-3) / 1e9,
                hbm_frac=fused_b / (st["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                mfma_tflops=flops / (st["median_ms"] * 1e-3) / 1e12)
            del fc
            torch.cuda.empty_cache()
            print("conv_chunk line done", file=sys.stderr, flush=True)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
