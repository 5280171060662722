"""MI355X (gfx950) gated delta rule forward: thin Python binding of libgdn.so.

Each function here has the name of the C entry point it calls (include/gdn.h)
and only marshals arguments: it checks devices, dtypes and contiguity,
allocates outputs with torch, and passes raw pointers plus torch's current
HIP stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback: if the library is missing or cannot load, the calls
raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

__all__ = [
    "GdnError",
    "library_path",
    "load_library",
    "gdn_gate_fwd",
    "gdn_conv1d_fwd",
    "gdn_chunk_fwd",
    "gdn_chunk_fwd_noalloc",
    "gdn_chunk_fwd_gated_norm",
    "gdn_conv_chunk_fwd",
    "gdn_segment_state_scan",
    "gdn_chunk_fwd_segmented",
    "gdn_segmented_workspace_bytes",
    "gdn_chunk_fwd_workspace_bytes",
    "gdn_conv_chunk_fwd_workspace_bytes",
    "gdn_segment_state_scan_workspace_bytes",
    "gdn_decode_step",
    "gdn_gated_rmsnorm_fwd",
    "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgdn.so"
_lib = None

F32, BF16 = 0, 1
# size of the fixed device array behind gdn_chunk_fwd_noalloc (GDN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20

EXPORTED_SYMBOLS = (
    "gdn_status_string",
    "gdn_abi_version",
    "gdn_gate_fwd",
    "gdn_conv1d_fwd",
    "gdn_chunk_fwd_workspace_bytes",
    "gdn_chunk_fwd",
    "gdn_chunk_fwd_noalloc",
    "gdn_chunk_fwd_gated_norm",
    "gdn_conv_chunk_fwd_workspace_bytes",
    "gdn_conv_chunk_fwd",
    "gdn_segment_state_scan_workspace_bytes",
    "gdn_segment_state_scan",
    "gdn_segmented_workspace_bytes",
    "gdn_chunk_fwd_segmented",
    "gdn_decode_step",
    "gdn_gated_rmsnorm_fwd",
)


class GdnError(RuntimeError):
    """A library call returned a non-zero gdn_status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__("%s failed: status %d (%s)" % (fn, status, text))
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library():
    """Load libgdn.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            "libgdn.so is not built (%s); run `python -m gated_deltanet_linear_chunk_amd.build`" % path
        )
    lib = ctypes.CDLL(path)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = ctypes.c_int
    lib.gdn_gate_fwd.argtypes = [P, P, P, P, i64, i32, P, P, P]
    lib.gdn_conv1d_fwd.argtypes = [P, P, P, ctypes.c_int, P, P, i32, i32, i64, i32, i32, i32, i32, i32, f32,
                                   ctypes.c_int, P, P]
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [ctypes.c_int, i64, i32, i32, i32, i32]
    lib.gdn_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd.argtypes = [P, P, P, ctypes.c_int, i64, i64, i64, P, P, f32, P, P, P, i32, i32, i64, i32, i32,
                                  i32, i32, P, ctypes.c_int, P, P, sz, P]
    lib.gdn_chunk_fwd_noalloc.argtypes = [P, P, P, ctypes.c_int, i64, i64, i64, P, P, f32, P, P, P, i32, i32, i64,
                                          i32, i32, i32, i32, P, ctypes.c_int, P, P]
    lib.gdn_chunk_fwd_gated_norm.argtypes = [P, P, P, ctypes.c_int, i64, i64, i64, P, P, f32, P, P, P, i32, i32, i64,
                                             i32, i32, i32, i32, P, ctypes.c_int, P, f32, P, ctypes.c_int, P, P,
                                             sz, P]
    lib.gdn_conv_chunk_fwd_workspace_bytes.argtypes = [ctypes.c_int, i64, i32, i32, i32, i32, i32]
    lib.gdn_conv_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn_conv_chunk_fwd.argtypes = [P, P, P, ctypes.c_int, i32, f32, P, P, P, P, f32, P, P, P, i32, i32, i64, i32,
                                       i32, i32, i32, P, ctypes.c_int, P, P, sz, P]
    lib.gdn_segment_state_scan_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    lib.gdn_segment_state_scan_workspace_bytes.restype = sz
    lib.gdn_segment_state_scan.argtypes = [P, P, ctypes.c_int, i64, i64, P, P, P, P, i32, P, i64, i32, i32, i32, i32,
                                           P, P, P, P, P, sz, P]
    lib.gdn_segmented_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    lib.gdn_segmented_workspace_bytes.restype = sz
    lib.gdn_chunk_fwd_segmented.argtypes = [P, P, P, ctypes.c_int, i64, i64, i64, P, P, f32, P, P, P, i32, i64, i32,
                                            i32, i32, i32, P, ctypes.c_int, P, P, sz, P]
    lib.gdn_decode_step.argtypes = [P, P, P, ctypes.c_int, P, P, f32, P, P, i64, i32, i32, i32, i32, i32, P,
                                    ctypes.c_int, P]
    lib.gdn_gated_rmsnorm_fwd.argtypes = [P, ctypes.c_int, P, ctypes.c_int, P, f32, i64, i32, P, ctypes.c_int, P]
    for name in ("gdn_gate_fwd", "gdn_conv1d_fwd", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_gated_norm",
                 "gdn_conv_chunk_fwd", "gdn_segment_state_scan",
                 "gdn_chunk_fwd_segmented", "gdn_decode_step", "gdn_gated_rmsnorm_fwd"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        text = load_library().gdn_status_string(status).decode()
        raise GdnError(fn, status, text)


def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _require(t, name: str, device=None, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _token_stride(t, name: str) -> int:
    """Token stride of a [B, T, H, D] (or [T, H, D]) view whose (H, D) block is dense.

    Returns the element stride between consecutive tokens; batch rows must follow
    one another at that stride (B * T tokens in one strided run).
    """
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    D, H = t.shape[-1], t.shape[-2]
    st = t.stride()
    if st[-1] != 1 or (H > 1 and st[-2] != D):
        raise ValueError("%s: the head and feature dims must be dense" % name)
    ts = st[-3] if t.shape[-3] > 1 else H * D
    # (rows of no tokens have no stride to check: torch reports one anyway)
    if t.dim() == 4 and t.shape[0] > 1 and t.shape[1] > 0 and st[0] != t.shape[1] * ts:
        raise ValueError("%s: batch rows must be evenly strided" % name)
    if ts % 8 != 0 or ts < H * D or t.data_ptr() % 16 != 0:
        raise ValueError("%s: token stride must be a multiple of 8 elements and 16-byte aligned" % name)
    return int(ts)


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _host_offsets(offsets_host) -> Optional[ctypes.Array]:
    if offsets_host is None:
        return None
    vals = [int(x) for x in offsets_host]
    return (ctypes.c_int32 * len(vals))(*vals)


# --------------------------------------------------------------------------- #
def gdn_gate_fwd(a, b, A_log, dt_bias):
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); a, b fp32 [..., H]."""
    torch = _torch()
    dev = a.device
    for t, n in ((a, "a"), (b, "b"), (A_log, "A_log"), (dt_bias, "dt_bias")):
        _require(t, n, dev, torch.float32)
    H = a.shape[-1]
    if b.shape != a.shape or A_log.numel() != H or dt_bias.numel() != H:
        raise ValueError("gate shapes disagree")
    g = torch.empty_like(a)
    beta = torch.empty_like(a)
    n_tok = a.numel() // H
    st = load_library().gdn_gate_fwd(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), n_tok, H, _ptr(g), _ptr(beta),
                                     _stream(dev))
    _check("gdn_gate_fwd", st)
    return g, beta


def gdn_conv1d_fwd(x, w, bias=None, cu_seqlens=None, cu_seqlens_host=None, apply_silu: bool = True,
                   l2norm_channels: int = 0, head_dim: int = 128, l2_eps: float = 1e-6, exact_rounding: bool = False):
    """Causal depthwise conv1d (+ SiLU, + per-head L2 norm of the first l2norm_channels).

    x [B, T, C] or [T, C] (packed, with cu_seqlens); w [C, W]; bias [C] or None.
    exact_rounding: every bf16 output is the bf16 nearest to the exact value
    (GDN_ROUND_EXACT) instead of the rounded fp32 evaluation.
    """
    torch = _torch()
    dev = x.device
    _require(x, "x", dev)
    _require(w, "w", dev, x.dtype)
    _require(bias, "bias", dev, x.dtype)
    _require(cu_seqlens, "cu_seqlens", dev, torch.int32)
    if x.dim() == 2:
        B, T, C = 1, x.shape[0], x.shape[1]
    else:
        B, T, C = x.shape
    if w.dim() != 2 or w.shape[0] != C:
        raise ValueError("w must be [C, W]")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    y = torch.empty_like(x)
    host = _host_offsets(cu_seqlens_host)
    st = load_library().gdn_conv1d_fwd(
        _ptr(x), _ptr(w), _ptr(bias), _dtype_code(x), _ptr(cu_seqlens), host, n_seqs, B, T, C, w.shape[1],
        int(bool(apply_silu)), int(l2norm_channels), int(head_dim), float(l2_eps), int(bool(exact_rounding)), _ptr(y),
        _stream(dev),
    )
    _check("gdn_conv1d_fwd", st)
    return y


def gdn_chunk_fwd_workspace_bytes(in_dtype, total_tokens: int, n_seqs: int, Hv: int, K: int, V: int) -> int:
    torch = _torch()
    code = BF16 if in_dtype == torch.bfloat16 else F32
    return int(load_library().gdn_chunk_fwd_workspace_bytes(code, total_tokens, n_seqs, Hv, K, V))


def _workspace(nbytes: int, device, given=None):
    torch = _torch()
    if given is not None:
        if given.numel() * given.element_size() < nbytes:
            raise ValueError("workspace too small: %d bytes needed" % nbytes)
        return given
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gdn_chunk_fwd(q, k, v, g, beta, scale: float = 1.0, initial_state=None, cu_seqlens=None,
                  cu_seqlens_host=None, o_dtype=None, output_final_state: bool = True, workspace=None):
    """Chunked gated delta rule forward.

    q, k [B, T, Hqk, K]; v [B, T, Hv, V]; g, beta fp32 [B, T, Hv];
    initial_state fp32 [N, Hv, K, V] or None; cu_seqlens int32 [N + 1] (B == 1).
    Returns (o [B, T, Hv, V] in o_dtype (default: v's dtype), final_state fp32
    [N, Hv, K, V] or None).
    """
    torch = _torch()
    dev = q.device
    qs, ks, vs = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    if k.dtype != q.dtype or v.dtype != q.dtype or k.device != dev or v.device != dev:
        raise ValueError("q, k, v must share dtype and device")
    _require(g, "g", dev, torch.float32)
    _require(beta, "beta", dev, torch.float32)
    _require(initial_state, "initial_state", dev, torch.float32)
    _require(cu_seqlens, "cu_seqlens", dev, torch.int32)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise ValueError("q, k must be [B, T, Hqk, K] and v [B, T, Hv, V]")
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("v / g / beta shapes disagree with q")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if initial_state is not None and initial_state.shape != (N, Hv, K, V):
        raise ValueError("initial_state must be [N, Hv, K, V]")
    o_dtype = v.dtype if o_dtype is None else o_dtype
    o = torch.empty((B, T, Hv, V), dtype=o_dtype, device=dev)
    fin = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    total = T if cu_seqlens is not None else B * T
    ws = _workspace(gdn_chunk_fwd_workspace_bytes(q.dtype, total, N, Hv, K, V), dev, workspace)
    st = load_library().gdn_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), qs, ks, vs, _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
        _ptr(cu_seqlens), _host_offsets(cu_seqlens_host), 0 if cu_seqlens is None else N, B, T, Hqk, Hv, K, V,
        _ptr(o), _dtype_code(o), _ptr(fin), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev),
    )
    _check("gdn_chunk_fwd", st)
    return o, fin


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, scale: float = 1.0, initial_state=None, cu_seqlens=None,
                          cu_seqlens_host=None, o=None, final_state=None, o_dtype=None,
                          output_final_state: bool = True):
    """gdn_chunk_fwd with the per-chunk records in the library's fixed device array.

    Arguments and results as gdn_chunk_fwd; no workspace.  Pass preallocated `o`
    ([B, T, Hv, V]) and `final_state` ([N, Hv, K, V] fp32) to have nothing
    allocated at all (e.g. under graph capture).  Calls that overlap on one
    device race on the array.
    """
    torch = _torch()
    dev = q.device
    qs, ks, vs = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    if k.dtype != q.dtype or v.dtype != q.dtype or k.device != dev or v.device != dev:
        raise ValueError("q, k, v must share dtype and device")
    _require(g, "g", dev, torch.float32)
    _require(beta, "beta", dev, torch.float32)
    _require(initial_state, "initial_state", dev, torch.float32)
    _require(cu_seqlens, "cu_seqlens", dev, torch.int32)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise ValueError("q, k must be [B, T, Hqk, K] and v [B, T, Hv, V]")
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("v / g / beta shapes disagree with q")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if initial_state is not None and initial_state.shape != (N, Hv, K, V):
        raise ValueError("initial_state must be [N, Hv, K, V]")
    if o is None:
        o = torch.empty((B, T, Hv, V), dtype=v.dtype if o_dtype is None else o_dtype, device=dev)
    _require(o, "o", dev)
    if o.shape != (B, T, Hv, V):
        raise ValueError("o must be [B, T, Hv, V]")
    if final_state is None and output_final_state:
        final_state = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", dev, torch.float32)
    if final_state is not None and final_state.shape != (N, Hv, K, V):
        raise ValueError("final_state must be [N, Hv, K, V]")
    st = load_library().gdn_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), qs, ks, vs, _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
        _ptr(cu_seqlens), _host_offsets(cu_seqlens_host), 0 if cu_seqlens is None else N, B, T, Hqk, Hv, K, V,
        _ptr(o), _dtype_code(o), _ptr(final_state), _stream(dev),
    )
    _check("gdn_chunk_fwd_noalloc", st)
    return o, final_state


def gdn_chunk_fwd_gated_norm(q, k, v, g, beta, z, norm_weight=None, eps: float = 1e-6, scale: float = 1.0,
                             initial_state=None, cu_seqlens=None, cu_seqlens_host=None, o_dtype=None,
                             output_final_state: bool = True, workspace=None):
    """gdn_chunk_fwd whose output passes through the gated RMS norm:
    o = n / sqrt(mean(n^2) + eps) * norm_weight * silu(z) per (token, v-head) row.

    Arguments as gdn_chunk_fwd, plus z [B, T, Hv, V] (float32 or bfloat16, dense)
    and norm_weight fp32 [V] or None.  Returns (o, final_state).
    """
    torch = _torch()
    dev = q.device
    qs, ks, vs = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    if k.dtype != q.dtype or v.dtype != q.dtype or k.device != dev or v.device != dev:
        raise ValueError("q, k, v must share dtype and device")
    _require(g, "g", dev, torch.float32)
    _require(beta, "beta", dev, torch.float32)
    _require(z, "z", dev)
    _require(norm_weight, "norm_weight", dev, torch.float32)
    _require(initial_state, "initial_state", dev, torch.float32)
    _require(cu_seqlens, "cu_seqlens", dev, torch.int32)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4:
        raise ValueError("q, k must be [B, T, Hqk, K] and v [B, T, Hv, V]")
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("v / g / beta shapes disagree with q")
    if z.shape != (B, T, Hv, V):
        raise ValueError("z must be [B, T, Hv, V]")
    if norm_weight is not None and norm_weight.shape != (V,):
        raise ValueError("norm_weight must be [V]")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if initial_state is not None and initial_state.shape != (N, Hv, K, V):
        raise ValueError("initial_state must be [N, Hv, K, V]")
    o_dtype = v.dtype if o_dtype is None else o_dtype
    o = torch.empty((B, T, Hv, V), dtype=o_dtype, device=dev)
    fin = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    total = T if cu_seqlens is not None else B * T
    ws = _workspace(gdn_chunk_fwd_workspace_bytes(q.dtype, total, N, Hv, K, V), dev, workspace)
    st = load_library().gdn_chunk_fwd_gated_norm(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), qs, ks, vs, _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
        _ptr(cu_seqlens), _host_offsets(cu_seqlens_host), 0 if cu_seqlens is None else N, B, T, Hqk, Hv, K, V,
        _ptr(z), _dtype_code(z), _ptr(norm_weight), float(eps), _ptr(o), _dtype_code(o), _ptr(fin), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(dev),
    )
    _check("gdn_chunk_fwd_gated_norm", st)
    return o, fin


def gdn_conv_chunk_fwd_workspace_bytes(in_dtype, total_tokens: int, n_seqs: int, Hqk: int, Hv: int, K: int,
                                       V: int) -> int:
    torch = _torch()
    code = BF16 if in_dtype == torch.bfloat16 else F32
    return int(load_library().gdn_conv_chunk_fwd_workspace_bytes(code, total_tokens, n_seqs, Hqk, Hv, K, V))


def gdn_conv_chunk_fwd(x, w, a, b, A_log, dt_bias, Hqk: int, K: int, bias=None, scale: float = 1.0,
                       initial_state=None, cu_seqlens=None, cu_seqlens_host=None, l2_eps: float = 1e-6,
                       o_dtype=None, output_final_state: bool = True, workspace=None):
    """conv1d + SiLU + q/k L2 norm and the gates formed inside the chunk kernels, then the chunk rule.

    x [B, T, C] raw channels q heads | k heads | v heads, C = 2 Hqk K + Hv V;
    w [C, W] and bias [C] or None in x's dtype; a, b fp32 [B, T, Hv] gate
    inputs and A_log, dt_bias fp32 [Hv] (g and beta as gdn_gate_fwd forms
    them).  bf16 with the MFMA head sizes forms the activations in the chunk
    prep (bf16, as the separate conv stores them); other shapes keep them in
    fp32 inside the vector-ALU kernel.  Other arguments and the results as
    gdn_chunk_fwd.
    """
    torch = _torch()
    dev = x.device
    _require(x, "x", dev)
    _require(w, "w", dev, x.dtype)
    _require(bias, "bias", dev, x.dtype)
    if a is None or b is None or A_log is None or dt_bias is None:
        raise ValueError("a, b, A_log and dt_bias are required")
    for t, name in ((a, "a"), (b, "b"), (A_log, "A_log"), (dt_bias, "dt_bias")):
        _require(t, name, dev, torch.float32)
    _require(initial_state, "initial_state", dev, torch.float32)
    _require(cu_seqlens, "cu_seqlens", dev, torch.int32)
    if x.dim() != 3 or a.dim() != 3:
        raise ValueError("x must be [B, T, C] and a, b [B, T, Hv]")
    B, T, C = x.shape
    Hv = a.shape[2]
    if a.shape[:2] != (B, T) or b.shape != a.shape or A_log.shape != (Hv,) or dt_bias.shape != (Hv,):
        raise ValueError("a / b must be [B, T, Hv] and A_log / dt_bias [Hv]")
    if Hv < 1 or (C - 2 * Hqk * K) <= 0 or (C - 2 * Hqk * K) % Hv != 0:
        raise ValueError("x channels must be 2 Hqk K + Hv V")
    V = (C - 2 * Hqk * K) // Hv
    if w.dim() != 2 or w.shape[0] != C or (bias is not None and tuple(bias.shape) != (C,)):
        raise ValueError("w must be [C, W] and bias [C]")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if initial_state is not None and initial_state.shape != (N, Hv, K, V):
        raise ValueError("initial_state must be [N, Hv, K, V]")
    o = torch.empty((B, T, Hv, V), dtype=x.dtype if o_dtype is None else o_dtype, device=dev)
    fin = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    total = T if cu_seqlens is not None else B * T
    ws = _workspace(gdn_conv_chunk_fwd_workspace_bytes(x.dtype, total, N, Hqk, Hv, K, V), dev, workspace)
    st = load_library().gdn_conv_chunk_fwd(
        _ptr(x), _ptr(w), _ptr(bias), _dtype_code(x), w.shape[1], float(l2_eps), _ptr(a), _ptr(b), _ptr(A_log),
        _ptr(dt_bias), float(scale), _ptr(initial_state), _ptr(cu_seqlens), _host_offsets(cu_seqlens_host),
        0 if cu_seqlens is None else N, B, T, Hqk, Hv, K, V, _ptr(o), _dtype_code(o), _ptr(fin), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(dev),
    )
    _check("gdn_conv_chunk_fwd", st)
    return o, fin


def gdn_segment_state_scan(k, v, g, beta, seg_offsets, seg_offsets_host=None, initial_state=None, workspace=None):
    """Pass 1 + fp32 composition over P contiguous segments of one sequence.

    k [T, Hqk, K] (or [1, T, Hqk, K]); v [T, Hv, V]; g, beta fp32 [T, Hv];
    seg_offsets int32 [P + 1]; initial_state fp32 [Hv, K, V] or None.
    Returns (M [P, Hv, K, K], b [P, Hv, K, V], seg_initial_states [P, Hv, K, V],
    final_state [Hv, K, V]).
    """
    torch = _torch()
    dev = k.device
    k3 = k[0] if k.dim() == 4 else k
    v3 = v[0] if v.dim() == 4 else v
    ks, vs = _token_stride(k3, "k"), _token_stride(v3, "v")
    if v3.dtype != k3.dtype or v3.device != dev:
        raise ValueError("k, v must share dtype and device")
    _require(g, "g", dev, torch.float32)
    _require(beta, "beta", dev, torch.float32)
    _require(seg_offsets, "seg_offsets", dev, torch.int32)
    _require(initial_state, "initial_state", dev, torch.float32)
    T, Hqk, K = k3.shape
    Hv, V = v3.shape[1], v3.shape[2]
    P = seg_offsets.numel() - 1
    M = torch.empty((P, Hv, K, K), dtype=torch.float32, device=dev)
    b = torch.empty((P, Hv, K, V), dtype=torch.float32, device=dev)
    starts = torch.empty((P, Hv, K, V), dtype=torch.float32, device=dev)
    fin = torch.empty((Hv, K, V), dtype=torch.float32, device=dev)
    ws = _workspace(int(load_library().gdn_segment_state_scan_workspace_bytes(T, P, Hv, K, V)), dev, workspace)
    st = load_library().gdn_segment_state_scan(
        _ptr(k3), _ptr(v3), _dtype_code(k3), ks, vs, _ptr(g), _ptr(beta), _ptr(seg_offsets),
        _host_offsets(seg_offsets_host),
        P, _ptr(initial_state), T, Hqk, Hv, K, V, _ptr(M), _ptr(b), _ptr(starts), _ptr(fin), _ptr(ws), ws.numel(),
        _stream(dev),
    )
    _check("gdn_segment_state_scan", st)
    return M, b, starts, fin


def gdn_segment_state_scan_workspace_bytes(T: int, P: int, Hv: int, K: int, V: int) -> int:
    return int(load_library().gdn_segment_state_scan_workspace_bytes(T, P, Hv, K, V))


def gdn_segmented_workspace_bytes(T: int, P: int, Hv: int, K: int, V: int) -> int:
    return int(load_library().gdn_segmented_workspace_bytes(T, P, Hv, K, V))


def gdn_chunk_fwd_segmented(q, k, v, g, beta, seg_offsets, seg_offsets_host=None, scale: float = 1.0,
                            initial_state=None, o_dtype=None, workspace=None):
    """Segment-parallel forward of one sequence (B = 1): pass 1, fp32 chain, pass 2.

    Returns (o [1, T, Hv, V], final_state [Hv, K, V]).
    """
    torch = _torch()
    dev = q.device
    qs, ks, vs = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    if k.dtype != q.dtype or v.dtype != q.dtype or k.device != dev or v.device != dev:
        raise ValueError("q, k, v must share dtype and device")
    _require(g, "g", dev, torch.float32)
    _require(beta, "beta", dev, torch.float32)
    _require(seg_offsets, "seg_offsets", dev, torch.int32)
    _require(initial_state, "initial_state", dev, torch.float32)
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if B != 1:
        raise ValueError("segmented forward takes one sequence (B == 1)")
    P = seg_offsets.numel() - 1
    need = gdn_segmented_workspace_bytes(T, P, Hv, K, V)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _require(workspace, "workspace", dev)
    o_dtype = v.dtype if o_dtype is None else o_dtype
    o = torch.empty((1, T, Hv, V), dtype=o_dtype, device=dev)
    fin = torch.empty((Hv, K, V), dtype=torch.float32, device=dev)
    st = load_library().gdn_chunk_fwd_segmented(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), qs, ks, vs, _ptr(g), _ptr(beta), float(scale),
        _ptr(initial_state), _ptr(seg_offsets), _host_offsets(seg_offsets_host), P, T, Hqk, Hv, K, V, _ptr(o),
        _dtype_code(o), _ptr(fin),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev),
    )
    _check("gdn_chunk_fwd_segmented", st)
    return o, fin


def gdn_decode_step(q, k, v, g, beta, state, scale: float = 1.0, state_indices=None, o_dtype=None):
    """Recurrent decode step: one new token per sequence, state updated in place.

    q, k [N, Hqk, K]; v [N, Hv, V] (float32 or bfloat16); g, beta fp32 [N, Hv];
    state fp32 [R, Hv, K, V]; state_indices int32 [N] (row of state per sequence,
    negative = skip) or None (row n).  Returns o [N, Hv, V] in o_dtype (default v's dtype).
    """
    torch = _torch()
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, name, dev)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype")
    _require(g, "g", dev, torch.float32)
    _require(beta, "beta", dev, torch.float32)
    _require(state, "state", dev, torch.float32)
    _require(state_indices, "state_indices", dev, torch.int32)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or state.dim() != 4:
        raise ValueError("q, k must be [N, Hqk, K], v [N, Hv, V], state [R, Hv, K, V]")
    N, Hqk, K = q.shape
    Hv, V = v.shape[1], v.shape[2]
    if v.shape[0] != N or g.shape != (N, Hv) or beta.shape != (N, Hv) or state.shape[1:] != (Hv, K, V):
        raise ValueError("v / g / beta / state shapes disagree with q")
    if state_indices is not None and state_indices.shape != (N,):
        raise ValueError("state_indices must be [N]")
    o_dtype = v.dtype if o_dtype is None else o_dtype
    o = torch.empty((N, Hv, V), dtype=o_dtype, device=dev)
    st = load_library().gdn_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta), float(scale), _ptr(state),
        _ptr(state_indices), state.shape[0], N, Hqk, Hv, K, V, _ptr(o), _dtype_code(o), _stream(dev))
    _check("gdn_decode_step", st)
    return o


def gdn_gated_rmsnorm_fwd(o, z, weight=None, eps: float = 1e-6, y_dtype=None, out=None):
    """Output norm gated by z: y = o / sqrt(mean(o^2) + eps) * weight * silu(z) over the last axis.

    o, z [..., V] (float32 or bfloat16, same shape); weight fp32 [V] or None.
    Returns y (a new tensor in y_dtype, default o's dtype, or `out`, which may be o).
    """
    torch = _torch()
    dev = o.device
    _require(o, "o", dev)
    _require(z, "z", dev)
    _require(weight, "weight", dev, torch.float32)
    if z.shape != o.shape:
        raise ValueError("z must have o's shape")
    V = o.shape[-1]
    if weight is not None and weight.shape != (V,):
        raise ValueError("weight must be [V]")
    if out is None:
        out = torch.empty(o.shape, dtype=o.dtype if y_dtype is None else y_dtype, device=dev)
    else:
        _require(out, "out", dev)
        if out.shape != o.shape:
            raise ValueError("out must have o's shape")
    st = load_library().gdn_gated_rmsnorm_fwd(_ptr(o), _dtype_code(o), _ptr(z), _dtype_code(z), _ptr(weight),
                                              float(eps), o.numel() // V, V, _ptr(out), _dtype_code(out), _stream(dev))
    _check("gdn_gated_rmsnorm_fwd", st)
    return out

