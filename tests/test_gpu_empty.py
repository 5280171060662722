"""Calls with no tokens at all: every sample, batch row or segment is empty.

The recurrence over an empty sample applies no state update, so the final
state must equal the initial state bit for bit (zero without one), and o has
no rows (prime-rl PR "feat: hybrid CP for Qwen3.5 MoE", Summary: the per-head
state is updated once per token; LlamaFactory PR "[v1] support GDN Ulysses
cp", Design decisions 5-6: each packed sample keeps its own state).  With no
tokens the data pointers may be null: the C ABI checks them only when there
is a token to read.
"""

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402

DEV = torch.device("cuda:0")
SHAPES = [
    # dtype, Hqk, Hv, K, V: the MFMA kernels, then the vector-ALU kernel
    (torch.bfloat16, 2, 4, 128, 128),
    (torch.float32, 2, 4, 64, 64),
]


def _state(N, Hv, K, V, with_s0, seed):
    if not with_s0:
        return None
    gen = torch.Generator().manual_seed(seed)
    return torch.randn((N, Hv, K, V), generator=gen, dtype=torch.float32).mul_(0.05).to(DEV)


def _expect_state(fin, s0):
    torch.cuda.synchronize()
    got = fin.cpu().numpy()
    want = np.zeros_like(got) if s0 is None else s0.cpu().numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("packed", [True, False], ids=["packed", "batched"])
@pytest.mark.parametrize("with_s0", [True, False], ids=["s0", "no_s0"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s_K%d" % (str(s[0])[6:], s[3]))
def test_chunk_fwd_without_tokens(shape, with_s0, packed):
    dt, Hqk, Hv, K, V = shape
    N = 3 if packed else 2
    B = 1 if packed else N
    q = torch.empty((B, 0, Hqk, K), dtype=dt, device=DEV)
    k = torch.empty_like(q)
    v = torch.empty((B, 0, Hv, V), dtype=dt, device=DEV)
    g = torch.empty((B, 0, Hv), dtype=torch.float32, device=DEV)
    beta = torch.empty_like(g)
    s0 = _state(N, Hv, K, V, with_s0, 7)
    cu_np = np.zeros(N + 1, dtype=np.int32)
    cu = torch.from_numpy(cu_np).to(DEV) if packed else None
    o, fin = gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu,
                               cu_seqlens_host=cu_np if packed else None, o_dtype=torch.float32)
    assert o.shape == (B, 0, Hv, V)
    _expect_state(fin, s0)


@pytest.mark.parametrize("with_s0", [True, False], ids=["s0", "no_s0"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s_K%d" % (str(s[0])[6:], s[3]))
def test_conv_chunk_fwd_without_tokens(shape, with_s0):
    dt, Hqk, Hv, K, V = shape
    N, C, W = 3, 2 * Hqk * K + Hv * V, 4
    x = torch.empty((1, 0, C), dtype=dt, device=DEV)
    w = torch.full((C, W), 0.25, dtype=dt, device=DEV)
    a = torch.empty((1, 0, Hv), dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    A_log = torch.zeros(Hv, dtype=torch.float32, device=DEV)
    dt_bias = torch.zeros(Hv, dtype=torch.float32, device=DEV)
    s0 = _state(N, Hv, K, V, with_s0, 8)
    cu_np = np.zeros(N + 1, dtype=np.int32)
    o, fin = gdn.gdn_conv_chunk_fwd(x, w, a, b, A_log, dt_bias, Hqk=Hqk, K=K, initial_state=s0,
                                    cu_seqlens=torch.from_numpy(cu_np).to(DEV), cu_seqlens_host=cu_np)
    assert o.shape == (1, 0, Hv, V)
    _expect_state(fin, s0)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s_K%d" % (str(s[0])[6:], s[3]))
def test_chunk_fwd_c_abi_null_data_without_tokens(shape):
    """Through the C ABI with every data pointer null: only the state moves."""
    dt, Hqk, Hv, K, V = shape
    N = 2
    lib = gdn.load_library()
    in_dt = 1 if dt == torch.bfloat16 else 0
    s0 = _state(N, Hv, K, V, True, 9)
    fin = torch.full((N, Hv, K, V), float("nan"), dtype=torch.float32, device=DEV)
    cu_np = np.zeros(N + 1, dtype=np.int32)
    cu = torch.from_numpy(cu_np).to(DEV)
    nbytes = lib.gdn_chunk_fwd_workspace_bytes(in_dt, 0, N, Hv, K, V)
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=DEV)
    host_cu = (ctypes.c_int32 * (N + 1))(*[0] * (N + 1))
    st = lib.gdn_chunk_fwd(None, None, None, in_dt, 0, 0, 0, None, None, 1.0, s0.data_ptr(), cu.data_ptr(), host_cu,
                           N, 1, 0, Hqk, Hv, K, V, None, 0, fin.data_ptr(), ws.data_ptr(), int(nbytes),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.gdn_status_string(st)
    _expect_state(fin, s0)


@pytest.mark.parametrize("with_s0", [True, False], ids=["s0", "no_s0"])
@pytest.mark.parametrize("shape", [SHAPES[0], (torch.float32, 2, 4, 128, 64)],  # the segment maps need K = 128
                         ids=lambda s: "%s_K%d" % (str(s[0])[6:], s[3]))
def test_segmented_forward_without_tokens(shape, with_s0):
    """Three empty segments: each segment's map is the identity, so the chain
    hands the initial state through unchanged."""
    dt, Hqk, Hv, K, V = shape
    q = torch.empty((1, 0, Hqk, K), dtype=dt, device=DEV)
    k = torch.empty_like(q)
    v = torch.empty((1, 0, Hv, V), dtype=dt, device=DEV)
    g = torch.empty((1, 0, Hv), dtype=torch.float32, device=DEV)
    beta = torch.empty_like(g)
    s0 = _state(1, Hv, K, V, with_s0, 10)
    off = np.zeros(4, dtype=np.int32)
    o, fin = gdn.gdn_chunk_fwd_segmented(q, k, v, g, beta, torch.from_numpy(off).to(DEV), off,
                                         initial_state=None if s0 is None else s0[0], o_dtype=torch.float32)
    assert o.shape == (1, 0, Hv, V)
    _expect_state(fin[None], s0)
