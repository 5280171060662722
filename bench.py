"""Benchmark of the gated delta rule forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--extras/--no-extras] [--no-cpu]

One step is one forward of a GatedDeltaNet layer's core over the packed
workload (8192 tokens in 8 samples of seeded random lengths, H_qk = 16,
H_v = 32, K = V = 128, bf16): gates, causal conv1d + SiLU + q/k L2 norm over
the 8192 q|k|v channels, and the chunked delta rule reading q, k, v straight
out of the conv output.  Inputs are resident in HBM before the timed region.
The line printed is one JSON object (see the fields below); `value` is tokens
per second of the whole step.  The duration of the gdn_chunk_fwd call (its
kernels: chunk prep, segment pass 1, map chains, scan) is measured with HIP
events recorded on the stream it runs on, and set against the HBM
roofline (its algorithmic bytes) and the bf16 MFMA peak (its algorithmic
flops).  The fp64 CPU oracle is timed on the same workload on the host.
Extras time the other workloads (segment-parallel long sequence, batched
prefill, wide state, the recurrent decode step on 256 sequences, and the
gated output norm on the packed workload's output) with the same method.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import gdn_inputs  # noqa: E402

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "GDN fwd tokens/s at H_v=32,K=V=128 bf16; % bf16 MFMA peak"
MAIN = "packed_varlen_bf16_T8192_N8_Hv32_K128"


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


CHUNK_SOURCES = ("chunk_prep.hip", "chunk_bf16.hip", "compose.hip", "split_plan.cpp", "api.cpp", "device_common.h",
                 "kernels.h")


def sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_deltanet_linear_chunk_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload):
    """HBM bytes per gdn_chunk_fwd call (FETCH_SIZE + WRITE_SIZE of its kernels, scaled by a copy
    calibration) from the committed rocprofv3 summary; None when the kernel sources have changed since
    the counters were taken, or when there is no summary."""
    path = os.path.join(ROOT, "profiles", "chunk_fwd_%s.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|", "`")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("chunk_sources_sha256_16") != sources_digest(CHUNK_SOURCES):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _torch():
    import torch

    return torch


class Timer:
    """HIP events on the current stream around one region; durations in ms."""

    def __init__(self):
        self.pairs = []

    def start(self):
        torch = _torch()
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        torch = _torch()
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")

    def reset(self):
        self.pairs = []


def build_pipeline(w, d, o_dtype):
    """Device inputs and a step function for a conv + gates + chunk workload."""
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
    x = bf(d["x"]).reshape(B, L, C) if B > 1 else bf(d["x"])
    cw, cb = bf(d["conv_w"]), bf(d["conv_bias"])
    a, b = f32(d["a"]).reshape(B, L, Hv), f32(d["b"]).reshape(B, L, Hv)
    A_log, dt_bias = f32(d["A_log"]), f32(d["dt_bias"])
    cu = None if B > 1 else torch.from_numpy(d["cu_seqlens"]).to(dev)
    cu_host = None if B > 1 else d["cu_seqlens"]
    s0 = f32(d["s0"]) if "s0" in d else None
    chunk_timer = Timer()
    conv_timer = Timer()

    # Only the gdn_chunk_fwd call is bracketed by timing events inside a step:
    # each recorded timing event leaves the GPU idle for a few microseconds, so
    # the conv is timed in a loop of its own (conv_step) after the timed region.
    def conv():
        return gdn.gdn_conv1d_fwd(x, cw, cb, cu_seqlens=cu, cu_seqlens_host=cu_host, l2norm_channels=2 * Hqk * K,
                                  head_dim=K)

    def conv_step():
        e = conv_timer.start()
        conv()
        conv_timer.stop(e)

    def step(time_kernels=False):
        y = conv().reshape(B, L, C)
        q = y[..., : Hqk * K].unflatten(-1, (Hqk, K))
        k = y[..., Hqk * K : 2 * Hqk * K].unflatten(-1, (Hqk, K))
        v = y[..., 2 * Hqk * K :].unflatten(-1, (Hv, V))
        g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
        e = chunk_timer.start() if time_kernels else None
        o, fin = gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu, cu_seqlens_host=cu_host,
                                   o_dtype=o_dtype)
        if time_kernels:
            chunk_timer.stop(e)
        return o, fin

    return step, chunk_timer, conv_timer, conv_step


def build_chunk_only(w, d, o_dtype, segmented=False, gated_norm=False):
    torch = _torch()
    import gated_deltanet_linear_chunk_amd as gdn

    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)  # noqa: E731
    q, k, v = bf(d["q"])[None], bf(d["k"])[None], bf(d["v"])[None]
    a, b = f32(d["a"])[None], f32(d["b"])[None]
    A_log, dt_bias = f32(d["A_log"]), f32(d["dt_bias"])
    timer = Timer()
    if segmented:
        off = d["seg_offsets"]
        off_dev = torch.from_numpy(off).to(dev)
        ws = torch.empty(gdn.gdn_segmented_workspace_bytes(w.total_tokens, len(off) - 1, w.Hv, w.K, w.V),
                         dtype=torch.uint8, device=dev)

        def step(time_kernels=False):
            g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
            e = timer.start() if time_kernels else None
            out = gdn.gdn_chunk_fwd_segmented(q, k, v, g, beta, off_dev, off, o_dtype=o_dtype, workspace=ws)
            if time_kernels:
                timer.stop(e)
            return out
    elif gated_norm:
        cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
        rng = np.random.default_rng(5)
        z = bf(rng.standard_normal((w.total_tokens, w.Hv, w.V)).astype(np.float32))[None]
        nw = f32(rng.uniform(0.5, 1.5, w.V))

        def step(time_kernels=False):
            g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
            e = timer.start() if time_kernels else None
            out = gdn.gdn_chunk_fwd_gated_norm(q, k, v, g, beta, z, norm_weight=nw, cu_seqlens=cu,
                                               cu_seqlens_host=d["cu_seqlens"], o_dtype=o_dtype)
            if time_kernels:
                timer.stop(e)
            return out
    else:
        cu = torch.from_numpy(d["cu_seqlens"]).to(dev)

        def step(time_kernels=False):
            g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
            e = timer.start() if time_kernels else None
            out = gdn.gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens"],
                                    o_dtype=o_dtype)
            if time_kernels:
                timer.stop(e)
            return out

    return step, timer


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
    timer = Timer()

    def step(time_kernels=False):
        e = timer.start() if time_kernels else None
        o = gdn.gdn_decode_step(q, k, v, g, beta, state, o_dtype=torch.float32)
        if time_kernels:
            timer.stop(e)
        return o

    return step, timer


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
    timer = Timer()

    def step(time_kernels=False):
        e = timer.start() if time_kernels else None
        out = gdn.gdn_gated_rmsnorm_fwd(o, z, w, eps=1e-6, out=y)
        if time_kernels:
            timer.stop(e)
        return out

    return step, timer


def timed(step, steps, warmup):
    torch = _torch()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(time_kernels=True)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--o-dtype", choices=["f32", "bf16"], default="f32")
    ap.add_argument("--copy-only", type=int, default=0,
                    help="only run N plain 256 MiB device copies (counter calibration for profiles)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the path shards by head, "
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
    w = gdn_inputs.WORKLOADS[MAIN]
    d = gdn_inputs.draw(w, with_qkv=False)
    step, chunk_t, conv_t, conv_step = build_pipeline(w, d, o_dtype)
    sec = timed(step, args.steps, args.warmup)
    for _ in range(args.steps):
        conv_step()
    torch.cuda.synchronize()
    T, N = w.total_tokens, w.n_samples
    chunk_ms = chunk_t.mean_ms()
    conv_ms = conv_t.mean_ms()
    bytes_chunk = chunk_alg_bytes(T, N, w.Hqk, w.Hv, w.K, w.V, o_bytes)
    flops_chunk = chunk_alg_flops(T, w.Hqk, w.Hv, w.K, w.V)
    achieved = bytes_chunk / (chunk_ms * 1e-3) / 1e9
    C = 2 * w.Hqk * w.K + w.Hv * w.V
    result = {
        "metric": METRIC,
        "value": T / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; packed lengths by a flat Dirichlet draw)",
        "config": {"workload": MAIN, "global_batch": N, "seq_len": T, "parallelism": "none (1 GPU)",
                   "H_qk": w.Hqk, "H_v": w.Hv, "K": w.K, "V": w.V, "chunk": 64, "conv_width": 4,
                   "o_dtype": args.o_dtype, "step": "gates + conv1d/SiLU/L2 + chunked rule"},
        "mfma_frac_chunk": flops_chunk / (chunk_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": profiled_traffic(MAIN),
                     "kernel": "gdn_chunk_fwd (segment-split path) = plan copy + chunk_prep_kernel + "
                               "chunk_scan_kernel<2,8> + compose_kernel + chunk_scan_kernel<0,8>",
                     "alg_bytes_per_launch": bytes_chunk, "alg_flops_per_launch": flops_chunk,
                     "avg_launch_ms": chunk_ms},
        "kernels_ms": {"chunk": chunk_ms, "conv1d": conv_ms},
        "conv1d_hbm_frac": conv_alg_bytes(T, C) / (conv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }

    if not args.no_extras:
        extras = {}
        del step
        torch.cuda.empty_cache()
        for name, kind in (("long_segmented_bf16_T32768_P8_Hv32_K128", "segmented"),
                           ("long_segmented_bf16_T32768_P8_Hv32_K128", "unsegmented"),
                           ("batched_prefill_bf16_B8_T4096_Hv32_K128", "pipeline"),
                           ("wide_state_bf16_T32768_N4_H64_K128_V256", "chunk")):
            wx = gdn_inputs.WORKLOADS[name]
            dx = gdn_inputs.draw(wx, with_qkv=(kind != "pipeline"))
            if kind == "pipeline":
                st, tm, _, _ = build_pipeline(wx, dx, o_dtype)
            else:
                st, tm = build_chunk_only(wx, dx, o_dtype, segmented=(kind == "segmented"))
            s = timed(st, max(3, args.steps // 4), 2)
            ms = tm.mean_ms()
            fl = chunk_alg_flops(wx.total_tokens, wx.Hqk, wx.Hv, wx.K, wx.V)
            extras["%s[%s]" % (name, kind)] = {
                "tokens_per_s": wx.total_tokens / s, "ms_per_step": s * 1e3, "main_kernel_ms": ms,
                "mfma_frac_useful": fl / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
            }
            del st, dx
            torch.cuda.empty_cache()
        st, tm = build_decode(DECODE_N, 16, 32, 128, 128)
        s = timed(st, max(3, args.steps // 4), 2)
        ms = tm.mean_ms()
        nbytes = decode_alg_bytes(DECODE_N, 16, 32, 128, 128)
        extras["decode_bf16_N%d_Hv32_K128[decode step]" % DECODE_N] = {
            "tokens_per_s": DECODE_N / s, "ms_per_step": s * 1e3, "main_kernel_ms": ms,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "alg_bytes": nbytes,
        }
        del st
        torch.cuda.empty_cache()
        rows = w.total_tokens * w.Hv
        st, tm = build_gated_norm(rows, w.V)
        s = timed(st, max(3, args.steps // 4), 2)
        ms = tm.mean_ms()
        nbytes = rows * w.V * (4 + 2 + 2)
        extras["gated_norm_f32o_bf16z_T8192_Hv32_V128[norm]"] = {
            "tokens_per_s": w.total_tokens / s, "ms_per_step": s * 1e3, "main_kernel_ms": ms,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "alg_bytes": nbytes,
        }
        del st
        torch.cuda.empty_cache()
        # the chunk forward with the gated norm applied as the scan writes o (bf16 z and y), against
        # the chunk call above plus the separate norm kernel
        dx = gdn_inputs.draw(w, with_qkv=True)
        st, tm = build_chunk_only(w, dx, torch.bfloat16, gated_norm=True)
        s = timed(st, max(3, args.steps // 4), 2)
        extras["%s[chunk + gated norm fused, bf16 z and y]" % MAIN] = {
            "tokens_per_s": w.total_tokens / s, "ms_per_step": s * 1e3, "main_kernel_ms": tm.mean_ms(),
        }
        del st, dx
        torch.cuda.empty_cache()
        result["extras"] = extras

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
