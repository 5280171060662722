"""Seeded synthetic inputs for the gated delta rule forward.

This module only draws random numbers and rounds them to the storage dtype.  It
holds none of the method's arithmetic (no gates, no convolution, no recurrence):
the raw gate projections a, b and the parameters A_log, dt_bias are returned as
drawn, and both the fp64 CPU oracle and the GPU path turn them into (g, beta) on
their own.  The one shaping step, normalising Gaussian q/k draws per head
vector, is the standard recipe for sampling uniformly on the unit sphere; the
workloads specify q and k as unit vectors.

Every config draws in one fixed order from ``numpy.random.default_rng(seed)``:
lengths -> A_log -> dt_bias -> q -> k -> v -> a -> b -> conv x / w / bias ->
initial_state.  Arrays of bf16 workloads are returned as float32 arrays whose
values are exactly representable in bfloat16 (rounded to nearest even), so the
oracle and the GPU consume identical numbers.

Layouts are packed and token-major: q, k [T, Hqk, K]; v [T, Hv, V];
a, b [T, Hv]; x [T, C] with C = 2 * Hqk * K + Hv * V (q | k | v channels);
w [C, W]; initial_state [N, Hv, K, V]; cu_seqlens int32 [N + 1].
A batched workload (B rows of equal length) is the packed case with
cu_seqlens = [0, L, 2L, ...].
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "bf16_round",
    "Workload",
    "WORKLOADS",
    "dirichlet_lengths",
    "draw",
    "workload",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return rounded.astype(np.uint32).view(np.float32).reshape(x.shape)


def dirichlet_lengths(rng: np.random.Generator, total: int, n: int, min_len: int) -> List[int]:
    """n lengths, each >= min_len, summing to total.

    The free tokens total - n * min_len are split by a flat Dirichlet draw,
    floored, and the remainder goes to the entries with the largest fractional
    parts (ties to the lower index).
    """
    free = total - n * min_len
    if free < 0:
        raise ValueError("total too small for n samples of min_len")
    if n == 1:
        return [total]
    share = rng.dirichlet(np.ones(n)) * free
    base = np.floor(share).astype(np.int64)
    rem = int(free - base.sum())
    order = sorted(range(n), key=lambda i: (-(share[i] - base[i]), i))
    for i in order[:rem]:
        base[i] += 1
    return [int(min_len + b) for b in base]


@dataclass
class Workload:
    """Shape and distribution recipe of one synthetic workload."""

    name: str
    seed: int
    total_tokens: int
    n_samples: int
    Hqk: int
    Hv: int
    K: int
    V: int
    dtype: str  # "f32" or "bf16": storage dtype of q, k, v (and conv x, w, bias)
    batch_rows: int = 1  # >1: B equal rows instead of cu_seqlens packing
    min_len: int = 64
    A_log_range: tuple = (0.0, math.log(16.0))
    conv_width: int = 0  # 0: no conv1d stage
    s0_std: float = 0.0  # 0: zero initial state
    segments: int = 0  # >0: equal contiguous segments of the single sequence
    lengths: Optional[List[int]] = None  # fixed lengths instead of Dirichlet draws
    gate_kind: str = "default"  # "default" | "zero_decay" (g == 0, beta ~ sigmoid(N(-3,1)))
    note: str = ""
    extra: Dict = field(default_factory=dict)


# The five workloads (sizes and distributions from the workload list).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32_T256_H2_K32", 1000, 256, 1, 2, 2, 32, 32, "f32"),
        Workload(
            "packed_varlen_bf16_T8192_N8_Hv32_K128",
            1001, 8192, 8, 16, 32, 128, 128, "bf16", conv_width=4,
        ),
        Workload(
            "long_segmented_bf16_T32768_P8_Hv32_K128",
            1002, 32768, 1, 16, 32, 128, 128, "bf16", segments=8,
        ),
        Workload(
            "batched_prefill_bf16_B8_T4096_Hv32_K128",
            1003, 32768, 8, 16, 32, 128, 128, "bf16", batch_rows=8, conv_width=4, s0_std=0.02,
        ),
        Workload(
            "wide_state_bf16_T32768_N4_H64_K128_V256",
            1004, 32768, 4, 64, 64, 128, 256, "bf16", A_log_range=(-2.0, 0.0),
        ),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _unit_rows(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Gaussian draws normalised per last-axis vector (uniform on the sphere)."""
    z = rng.standard_normal(shape, dtype=np.float64)
    z /= np.sqrt(np.sum(z * z, axis=-1, keepdims=True))
    return _store(z, dtype)


def draw(w: Workload, with_qkv: bool = True) -> Dict[str, np.ndarray]:
    """Draw every input of workload w in the fixed order.

    Returns a dict with cu_seqlens (int32), lengths, A_log, dt_bias, a, b
    (float32), q, k, v (storage-dtype values in float32) when with_qkv, conv
    inputs x, w, bias when the workload has a conv1d stage, s0 when it has a
    non-zero initial state, and seg_offsets when it is segmented.
    with_qkv=False skips materialising q/k/v but still advances the generator
    identically, so later draws do not change.
    """
    rng = np.random.default_rng(w.seed)
    T = w.total_tokens
    out: Dict[str, np.ndarray] = {}
    if w.lengths is not None:
        lengths = list(w.lengths)
    elif w.batch_rows > 1:
        lengths = [T // w.batch_rows] * w.batch_rows
    else:
        lengths = dirichlet_lengths(rng, T, w.n_samples, w.min_len)
    if sum(lengths) != T:
        raise ValueError("lengths do not sum to total_tokens")
    out["lengths"] = np.array(lengths, dtype=np.int64)
    out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H = w.Hv
    lo, hi = w.A_log_range
    A_log = rng.uniform(lo, hi, size=H)
    if w.gate_kind == "zero_decay":
        A_log = np.full(H, -np.inf)
    out["A_log"] = A_log.astype(np.float32)
    out["dt_bias"] = rng.uniform(-1.0, 1.0, size=H).astype(np.float32)
    if with_qkv:
        out["q"] = _unit_rows(rng, (T, w.Hqk, w.K), w.dtype)
        out["k"] = _unit_rows(rng, (T, w.Hqk, w.K), w.dtype)
        out["v"] = _store(rng.standard_normal((T, H, w.V), dtype=np.float32), w.dtype)
    else:
        rng.standard_normal((T, w.Hqk, w.K), dtype=np.float64)
        rng.standard_normal((T, w.Hqk, w.K), dtype=np.float64)
        rng.standard_normal((T, H, w.V), dtype=np.float32)
    out["a"] = rng.standard_normal((T, H), dtype=np.float32)
    if w.gate_kind == "zero_decay":
        out["b"] = (rng.standard_normal((T, H), dtype=np.float32) - 3.0).astype(np.float32)
    else:
        out["b"] = rng.standard_normal((T, H), dtype=np.float32)
    if w.conv_width:
        C = 2 * w.Hqk * w.K + w.Hv * w.V
        out["x"] = _store(rng.standard_normal((T, C), dtype=np.float32), w.dtype)
        out["conv_w"] = _store(0.5 * rng.standard_normal((C, w.conv_width), dtype=np.float32), w.dtype)
        out["conv_bias"] = _store(0.1 * rng.standard_normal(C, dtype=np.float32), w.dtype)
    if w.s0_std > 0:
        N = len(lengths)
        out["s0"] = (w.s0_std * rng.standard_normal((N, H, w.K, w.V), dtype=np.float32)).astype(np.float32)
    if w.segments:
        P = w.segments
        out["seg_offsets"] = (np.arange(P + 1, dtype=np.int64) * T // P).astype(np.int32)
    return out


def small(
    seed: int,
    lengths: List[int],
    Hqk: int,
    Hv: int,
    K: int,
    V: int,
    dtype: str = "f32",
    A_log_range=(0.0, math.log(16.0)),
    gate_kind: str = "default",
    conv_width: int = 0,
    s0_std: float = 0.0,
    segments: int = 0,
    name: str = "custom",
) -> Dict[str, np.ndarray]:
    """Draw a custom-shaped workload (same recipe, caller-chosen sizes)."""
    w = Workload(
        name, seed, int(sum(lengths)), len(lengths), Hqk, Hv, K, V, dtype,
        A_log_range=A_log_range, conv_width=conv_width, s0_std=s0_std,
        segments=segments, lengths=list(lengths), gate_kind=gate_kind,
    )
    return draw(w)
