"""fp64 CPU oracle for the gated delta rule forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It shares no code with the HIP library: the heavy
loops live in ``gdn_oracle.c`` (plain C, fp64, compiled here with gcc), the
rest is numpy in fp64.  Each function states the definition it follows; none
of them blocks, fuses or reorders beyond that definition, except
``chunked_form``, which is the chunk-parallel rewriting of the recurrence kept
here only so that the algebra the GPU kernels use can be checked against the
plain recurrence in exact-enough arithmetic.

Sources: the pull-request pages on GatedDeltaNet context parallelism --
prime-rl "feat: hybrid CP for Qwen3.5 MoE" (Summary: per-head state in
R^{K x V}, sequential update; Communication-cost table: state passing moves
O(H K (K+V)) numbers), sglang fork "Qwen3.5 cp - #1" (PR body: per-segment
(b, M) pairs, all-gathered and chain-reduced in fp32), LlamaFactory
"[v1] support GDN Ulysses cp" (Design: conv1d and chunk rule honour
cu_seqlens with no cross-sample leakage; the conv fallback is PyTorch's
conv1d) -- and the gated delta rule itself,
S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t,
beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.oracle_gdn_recurrence.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, f64, P, P, P, i32]
            lib.oracle_gdn_recurrence.restype = i32
            lib.oracle_transition.argtypes = [P, P, P, i64, i64, i32, i32, i32, P, i32]
            lib.oracle_transition.restype = i32
            lib.oracle_conv1d.argtypes = [P, P, P, P, i32, i32, i32, i32, P, i32]
            lib.oracle_conv1d.restype = i32
            lib.oracle_gates.argtypes = [P, P, P, P, i64, i32, P, P]
            lib.oracle_gates.restype = None
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = i32
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cu(cu, T) -> np.ndarray:
    if cu is None:
        return np.array([0, T], dtype=np.int64)
    return np.ascontiguousarray(cu, dtype=np.int64)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# --------------------------------------------------------------------------- #
# Recurrence (the definition)                                                 #
# --------------------------------------------------------------------------- #
def recurrence(
    q, k, v, g, beta, s0=None, cu=None, scale: float = 1.0,
    units: Optional[np.ndarray] = None, threads: int = 0, want_o: bool = True,
) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """Token-by-token gated delta rule in fp64.

    q, k [T, Hqk, K]; v [T, Hv, V]; g, beta [T, Hv]; s0 [N, Hv, K, V] or None;
    cu int [N+1] packed-sample offsets (None: one sequence).  Per token:
    S <- e^g S; u <- beta (v - S^T k); S <- S + k u^T; o <- scale S^T q.
    units: optional bool [N, Hv] restricting which (sequence, head) units run
    (outputs of the others are NaN).  Returns (o [T, Hv, V] or None, final
    [N, Hv, K, V]).
    """
    lib = _load()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, Hqk, K = k.shape
    Hv, V = v.shape[1], v.shape[2]
    cu = _cu(cu, T)
    N = len(cu) - 1
    s0 = None if s0 is None else _f64(s0).reshape(N, Hv, K, V)
    mask = None
    if units is not None:
        mask = np.ascontiguousarray(np.asarray(units, dtype=bool).reshape(N * Hv).astype(np.uint8))
    o = np.full((T, Hv, V), np.nan) if want_o else None
    fin = np.full((N, Hv, K, V), np.nan)
    rc = lib.oracle_gdn_recurrence(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(cu), N, Hqk, Hv, K, V,
        float(scale), _ptr(mask), _ptr(o), _ptr(fin), int(threads),
    )
    if rc != 0:
        raise ValueError("oracle_gdn_recurrence failed (%d)" % rc)
    return o, fin


def decode_step(q, k, v, g, beta, state, scale: float = 1.0, state_indices=None):
    """One token of the gated delta rule for each of N sequences, in fp64.

    The recurrent decode step that follows a prefill (the sglang fork PR
    "Qwen3.5 cp - #1" hands the final state of the prefill to the standard
    decode path): per sequence n and v-head h, with S = state[r, h] (K x V),
    S <- e^g S; u <- beta (v - S^T k); S <- S + k u^T; o <- scale S^T q.
    q, k [N, Hqk, K]; v [N, Hv, V]; g, beta [N, Hv]; state [R, Hv, K, V].
    Row r = state_indices[n] (or n when None); a negative index skips the
    sequence (o = 0, no state touched).  v-head h reads q/k head h // (Hv // Hqk).
    Returns (o [N, Hv, V], the updated state as a new array).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    S_all = _f64(state).copy()
    N, Hqk, K = k.shape
    Hv, V = v.shape[1], v.shape[2]
    grp = Hv // Hqk
    o = np.zeros((N, Hv, V))
    for n in range(N):
        r = n if state_indices is None else int(state_indices[n])
        if r < 0:
            continue
        for h in range(Hv):
            kk, qq = k[n, h // grp], q[n, h // grp]
            S = np.exp(g[n, h]) * S_all[r, h]
            u = beta[n, h] * (v[n, h] - S.T @ kk)
            S = S + np.outer(kk, u)
            o[n, h] = scale * (S.T @ qq)
            S_all[r, h] = S
    return o, S_all


def gated_rmsnorm(o, z, weight=None, eps: float = 1e-6) -> np.ndarray:
    """The output norm gated by z that follows the chunk rule, in fp64.

    The LlamaFactory PR "[v1] support GDN Ulysses cp" (Design) runs
    "chunk_gated_delta_rule + norm" with the z component; the pages give no
    formula, so this is the plain reading of a per-head RMS norm gated by SiLU(z):
    over the last axis (V), y = o / sqrt(mean(o^2) + eps) * weight * z sigmoid(z).
    o, z [..., V]; weight [V] or None (ones).
    """
    o, z = _f64(o), _f64(z)
    w = np.ones(o.shape[-1]) if weight is None else _f64(weight)
    inv = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * inv * w * (z / (1.0 + np.exp(-z)))


def transition(k, g, beta, t0: int, t1: int, Hqk: int, Hv: int, threads: int = 0) -> np.ndarray:
    """M [Hv, K, K] = A_{t1-1} ... A_{t0}, A_t = e^{g_t}(I - beta_t k_t k_t^T), by dense products."""
    lib = _load()
    k, g, beta = map(_f64, (k, g, beta))
    K = k.shape[2]
    M = np.empty((Hv, K, K))
    rc = lib.oracle_transition(_ptr(k), _ptr(g), _ptr(beta), int(t0), int(t1), Hqk, Hv, K, _ptr(M), int(threads))
    if rc != 0:
        raise ValueError("oracle_transition failed (%d)" % rc)
    return M


# --------------------------------------------------------------------------- #
# Segments: affine transitions and their chain                                #
# --------------------------------------------------------------------------- #
def segment_affine(k, v, g, beta, seg_offsets, Hqk: int, threads: int = 0):
    """Per segment i = [off_i, off_{i+1}): (M_i, b_i) with S_end = M_i S_start + b_i.

    M_i is the dense product of the per-token transitions; b_i is the
    recurrence run over the segment from a zero state.  Returns M [P, Hv, K, K],
    b [P, Hv, K, V].
    """
    v = _f64(v)
    Hv = v.shape[1]
    off = np.asarray(seg_offsets, dtype=np.int64)
    P = len(off) - 1
    Ms = np.stack([transition(k, g, beta, off[i], off[i + 1], Hqk, Hv, threads) for i in range(P)])
    _, b = recurrence(
        np.zeros_like(_f64(k)), k, v, g, beta, None, off, threads=threads, want_o=False
    )
    return Ms, b


def chain(M, b, s0=None):
    """Serial composition S_start,0 = s0 (or 0), S_start,i+1 = M_i S_start,i + b_i.

    M [P, Hv, K, K], b [P, Hv, K, V], s0 [Hv, K, V] or None.  Returns
    (S_start [P, Hv, K, V], S_final [Hv, K, V]).
    """
    M, b = _f64(M), _f64(b)
    P, Hv, K, V = b.shape
    S = np.zeros((Hv, K, V)) if s0 is None else _f64(s0).reshape(Hv, K, V).copy()
    starts = np.empty((P, Hv, K, V))
    for i in range(P):
        starts[i] = S
        S = np.matmul(M[i], S) + b[i]
    return starts, S


def compose(first, second):
    """Affine-map composition: apply `first`, then `second`.

    (M2, b2) o (M1, b1) = (M2 M1, M2 b1 + b2).  Associative.
    """
    M1, b1 = first
    M2, b2 = second
    return np.matmul(M2, M1), np.matmul(M2, b1) + b2


# --------------------------------------------------------------------------- #
# Conv1d, gates, L2 normalisation, bf16 rounding                              #
# --------------------------------------------------------------------------- #
def conv1d(x, w, bias=None, cu=None, silu: bool = True, threads: int = 0) -> np.ndarray:
    """Causal depthwise conv1d (+ SiLU) with zero history at each sample start.

    y[t,c] = act(bias[c] + sum_j w[c,j] x[t-(W-1)+j, c]); x [T, C], w [C, W].
    """
    lib = _load()
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    W = w.shape[1]
    bias = None if bias is None else _f64(bias)
    cu = _cu(cu, T)
    y = np.empty((T, C))
    rc = lib.oracle_conv1d(_ptr(x), _ptr(w), _ptr(bias), _ptr(cu), len(cu) - 1, C, W, int(bool(silu)), _ptr(y), int(threads))
    if rc != 0:
        raise ValueError("oracle_conv1d failed (%d)" % rc)
    return y


def gates(a, b, A_log, dt_bias) -> Tuple[np.ndarray, np.ndarray]:
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b), in fp64. a, b [T, H]."""
    lib = _load()
    a, b, A_log, dt_bias = map(_f64, (a, b, A_log, dt_bias))
    T, H = a.shape
    g = np.empty((T, H))
    beta = np.empty((T, H))
    lib.oracle_gates(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), T, H, _ptr(g), _ptr(beta))
    return g, beta


def l2norm(x, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis, fp64."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def round_bf16(x) -> np.ndarray:
    """Round values to the nearest bfloat16 value (ties to even), one rounding.

    fp64 input is first rounded to fp32, which keeps every bit that decides the
    bf16 result except when it lands exactly on a bf16 midpoint (the halfway
    point between two neighbouring bf16 values); there the fp64 value itself
    says on which side of the midpoint it lies.  The result is returned in fp64.
    """
    x = np.asarray(x)
    xd = x.astype(np.float64)
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) & 0xFFFF0000
    on_mid = (u & 0xFFFF) == 0x8000
    ax, af = np.abs(xd), np.abs(f.astype(np.float64))
    r = np.where(on_mid & (ax > af), (u & 0xFFFF0000) + 0x10000, r)
    r = np.where(on_mid & (ax < af), u & 0xFFFF0000, r)
    return r.astype(np.uint32).view(np.float32).astype(np.float64).reshape(f.shape)


def split_channels(y, Hqk: int, Hv: int, K: int, V: int):
    """Split conv channels [q (Hqk*K) | k (Hqk*K) | v (Hv*V)] into [T, H, D] tensors."""
    T = y.shape[0]
    nq = Hqk * K
    q = y[:, :nq].reshape(T, Hqk, K)
    k = y[:, nq : 2 * nq].reshape(T, Hqk, K)
    v = y[:, 2 * nq :].reshape(T, Hv, V)
    return q, k, v


def pipeline_activations(x, w, bias, cu, Hqk, Hv, K, V, act_round: str = "bf16", eps: float = 1e-6, threads: int = 0):
    """conv1d + SiLU -> split -> L2-normalise q, k per head -> activations.

    The layer's activations between the conv and the chunk rule are stored in
    the input dtype, so with act_round="bf16" the fp64 results are rounded to
    bf16 (nearest even) here, at the same point the GPU pipeline stores them.
    """
    y = conv1d(x, w, bias, cu, silu=True, threads=threads)
    q, k, v = split_channels(y, Hqk, Hv, K, V)
    q, k = l2norm(q, eps), l2norm(k, eps)
    if act_round == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


# --------------------------------------------------------------------------- #
# Chunk-parallel rewriting (for checking the algebra only)                    #
# --------------------------------------------------------------------------- #
def chunked_form(q, k, v, g, beta, s0=None, cu=None, C: int = 64, scale: float = 1.0):
    """The recurrence rewritten chunk by chunk (C tokens), in fp64 numpy.

    Inside a chunk with local tokens r = 1..L and G_r = sum_{s<=r} g_s:
      D_rs = exp(G_r - G_s) (r >= s), A = strictly-lower(diag(beta) K K^T * D),
      T = (I + A)^{-1}, W = T diag(beta e^G) K, U0 = T diag(beta) V,
      U = U0 - W S, O = diag(e^G) Q S + lower(Q K^T * D) U,
      S <- e^{G_L} S + (diag(e^{G_L - G}) K)^T U.
    It equals the token recurrence in exact arithmetic (induction over tokens);
    the chunk grid is anchored at each sample start.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, Hqk, K = k.shape
    Hv, V = v.shape[1], v.shape[2]
    grp = Hv // Hqk
    cu = _cu(cu, T)
    N = len(cu) - 1
    o = np.zeros((T, Hv, V))
    fin = np.zeros((N, Hv, K, V))
    for n in range(N):
        for h in range(Hv):
            hq = h // grp
            S = np.zeros((K, V)) if s0 is None else _f64(s0)[n, h].copy()
            for c0 in range(int(cu[n]), int(cu[n + 1]), C):
                c1 = min(c0 + C, int(cu[n + 1]))
                Q, Kc, Vc = q[c0:c1, hq], k[c0:c1, hq], v[c0:c1, h]
                gc, bc = g[c0:c1, h], beta[c0:c1, h]
                L = c1 - c0
                G = np.cumsum(gc)
                diff = G[:, None] - G[None, :]
                low_incl = np.tril(np.ones((L, L), dtype=bool))
                D = np.where(low_incl, np.exp(np.where(low_incl, diff, 0.0)), 0.0)
                A = np.tril(bc[:, None] * (Kc @ Kc.T) * D, -1)
                Tm = np.linalg.inv(np.eye(L) + A)
                W = Tm @ ((bc * np.exp(G))[:, None] * Kc)
                U0 = Tm @ (bc[:, None] * Vc)
                U = U0 - W @ S
                O = np.exp(G)[:, None] * (Q @ S) + ((Q @ Kc.T) * D) @ U
                o[c0:c1, h] = scale * O
                S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * Kc).T @ U
            fin[n, h] = S
    return o, fin
