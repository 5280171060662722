"""Canary test: no entry point writes a byte outside the memory it is given.

Every output (and every workspace) is placed inside a larger buffer whose guard
bands before and after, and the output itself, start filled with a sentinel
byte pattern.  The calls go straight through the C ABI with those pointers, on
packed runs with partial last chunks, zero-length and one-token samples, with
and without the segment split, and the guard bands must come back bit for bit
unchanged.  Tokens past the last offset of a device-only cu_seqlens belong to
no sample, and their o rows must stay untouched too (the no-cross-sample rule
of packed samples, LlamaFactory PR "[v1] support GDN Ulysses cp", Design
decisions 5-6).
"""

import ctypes

import numpy as np
import pytest

import gdn_inputs
from parity_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402

GUARD = 4096  # bytes of guard band on each side (a multiple of 256)
PATTERN = 0xA5


class Guarded:
    """A payload of nbytes between two guard bands, all filled with the sentinel byte."""

    def __init__(self, nbytes, dtype=torch.uint8):
        self.nbytes = int(nbytes)
        pad = (-self.nbytes) % 256
        self.buf = torch.full((GUARD + self.nbytes + pad + GUARD,), PATTERN, dtype=torch.uint8, device="cuda:0")
        self.dtype = dtype

    @property
    def ptr(self):
        return self.buf.data_ptr() + GUARD

    def payload(self, shape=None):
        t = self.buf[GUARD : GUARD + self.nbytes].view(self.dtype)
        return t if shape is None else t.reshape(shape)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.nbytes :]
        bad_h = int((head != PATTERN).sum())
        bad_t = int((tail != PATTERN).sum())
        assert bad_h == 0 and bad_t == 0, "%s: %d guard bytes before and %d after were written" % (what, bad_h, bad_t)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _host_cu(cu):
    return (ctypes.c_int32 * len(cu))(*[int(x) for x in cu])


def _inputs(lengths, Hqk, Hv, K, V, dtype="bf16", seed=91, s0=True):
    d = gdn_inputs.small(seed, lengths, Hqk, Hv, K, V, dtype, s0_std=0.05 if s0 else 0.0)
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    t = dict(q=dev(d["q"], dtype), k=dev(d["k"], dtype), v=dev(d["v"], dtype), g=g, beta=beta,
             cu=dev(d["cu_seqlens"], "i32"), cu_np=d["cu_seqlens"], s0=dev(d["s0"]) if s0 else None)
    return d, t


def _chunk_call(lib, t, T, N, Hqk, Hv, K, V, in_dt, o, o_dt, fin, ws, ws_bytes, host_cu=True, n_seqs=None):
    cu_host = _host_cu(t["cu_np"]) if host_cu else None
    st = lib.gdn_chunk_fwd(
        t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), in_dt, 0, 0, 0, t["g"].data_ptr(),
        t["beta"].data_ptr(), 0.1, None if t["s0"] is None else t["s0"].data_ptr(), t["cu"].data_ptr(), cu_host,
        N if n_seqs is None else n_seqs, 1, T, Hqk, Hv, K, V, o, o_dt, fin, ws, ws_bytes, _stream())
    assert st == 0, lib.gdn_status_string(st)


LENGTHS = [130, 0, 64, 1, 257, 0, 700]  # partial chunks, empty and one-token samples; long enough to split


@pytest.mark.parametrize("o_dt", [gdn.F32, gdn.BF16])
@pytest.mark.parametrize("split", [True, False])
def test_chunk_bf16_writes_nothing_outside(o_dt, split):
    lib = gdn.load_library()
    Hqk, Hv, K, V = 2, 4, 128, 128
    d, t = _inputs(LENGTHS, Hqk, Hv, K, V)
    T, N = sum(LENGTHS), len(LENGTHS)
    o = Guarded(T * Hv * V * (4 if o_dt == gdn.F32 else 2))
    fin = Guarded(N * Hv * K * V * 4)
    ws_bytes = lib.gdn_chunk_fwd_workspace_bytes(gdn.BF16, T, N, Hv, K, V)
    ws = Guarded(ws_bytes)
    print("canary chunk bf16: o_dt %d split %s" % (o_dt, split), flush=True)
    _chunk_call(lib, t, T, N, Hqk, Hv, K, V, gdn.BF16, o.ptr, o_dt, fin.ptr, ws.ptr, ws_bytes, host_cu=split)
    o.check("o")
    fin.check("final_state")
    ws.check("workspace")
    # every token belongs to a sample here: every o byte was written
    assert bool(torch.isfinite(o.payload().view(torch.float32 if o_dt == gdn.F32 else torch.bfloat16)).all())


def test_chunk_tokens_past_the_last_offset_stay_untouched():
    """Device-only offsets ending before T: the trailing tokens are in no sample."""
    lib = gdn.load_library()
    Hqk, Hv, K, V = 2, 4, 128, 128
    lengths = [70, 0, 129, 1, 100]
    d, t = _inputs(lengths, Hqk, Hv, K, V)
    T = sum(lengths)
    # the last sample is dropped from the offsets: its 100 tokens are in no sample
    t["cu_np"] = t["cu_np"][:-1]
    t["cu"] = t["cu"][:-1].contiguous()
    N = len(lengths) - 1
    t["s0"] = t["s0"][:N].contiguous()
    o = Guarded(T * Hv * V * 4)
    fin = Guarded(N * Hv * K * V * 4)
    ws_bytes = lib.gdn_chunk_fwd_workspace_bytes(gdn.BF16, T, N, Hv, K, V)
    ws = Guarded(ws_bytes)
    _chunk_call(lib, t, T, N, Hqk, Hv, K, V, gdn.BF16, o.ptr, gdn.F32, fin.ptr, ws.ptr, ws_bytes, host_cu=False)
    o.check("o")
    fin.check("final_state")
    ws.check("workspace")
    rows = o.payload((T, Hv * V * 4))
    last = int(t["cu_np"][-1])
    assert bool((rows[last:] == PATTERN).all()), "o rows of tokens in no sample were written"
    assert bool(torch.isfinite(rows[:last].view(torch.float32)).all())


def test_chunk_fp32_writes_nothing_outside():
    lib = gdn.load_library()
    Hqk, Hv, K, V = 2, 4, 32, 64
    d, t = _inputs(LENGTHS, Hqk, Hv, K, V, dtype="f32")
    T, N = sum(LENGTHS), len(LENGTHS)
    o = Guarded(T * Hv * V * 4)
    fin = Guarded(N * Hv * K * V * 4)
    _chunk_call(lib, t, T, N, Hqk, Hv, K, V, gdn.F32, o.ptr, gdn.F32, fin.ptr, None, 0)
    o.check("o")
    fin.check("final_state")


@pytest.mark.parametrize("exact", [0, 1])
def test_conv_writes_nothing_outside(exact):
    lib = gdn.load_library()
    lengths = [1, 63, 64, 2, 170, 0, 33]
    w = gdn_inputs.Workload("canary_conv", 17, sum(lengths), len(lengths), 2, 4, 128, 64, "bf16", conv_width=4,
                            lengths=lengths)
    d = gdn_inputs.draw(w)
    T, C = d["x"].shape
    x, cw, cb = dev(d["x"], "bf16"), dev(d["conv_w"], "bf16"), dev(d["conv_bias"], "bf16")
    cu = dev(d["cu_seqlens"], "i32")
    y = Guarded(T * C * 2)
    st = lib.gdn_conv1d_fwd(x.data_ptr(), cw.data_ptr(), cb.data_ptr(), gdn.BF16, cu.data_ptr(),
                            _host_cu(d["cu_seqlens"]), len(lengths), 1, T, C, 4, 1, 2 * 2 * 128, 128, 1e-6, exact,
                            y.ptr, _stream())
    assert st == 0
    y.check("conv y")
    assert bool(torch.isfinite(y.payload().view(torch.bfloat16)).all())


@pytest.mark.parametrize("dtype,K", [("bf16", 64), ("f32", 64), ("bf16", 128)])
def test_conv_chunk_writes_nothing_outside(dtype, K):
    """The fused conv + chunk call, with device-only offsets that leave the last
    sample's tokens in no sample: their o rows stay untouched as well.  K = 128
    in bf16 runs the MFMA path, whose workspace (activations and records) is
    guarded too."""
    lib = gdn.load_library()
    Hqk, Hv, V = 2, 4, K
    lengths = [1, 63, 0, 130, 40]
    d = gdn_inputs.small(23, lengths, Hqk, Hv, K, V, dtype, conv_width=4, s0_std=0.05)
    T, C = d["x"].shape
    N = len(lengths) - 1
    es = 2 if dtype == "bf16" else 4
    x, cw, cb = dev(d["x"], dtype), dev(d["conv_w"], dtype), dev(d["conv_bias"], dtype)
    cu = dev(d["cu_seqlens"][:-1], "i32")
    s0 = dev(d["s0"][:N])
    o = Guarded(T * Hv * V * es)
    fin = Guarded(N * Hv * K * V * 4)
    in_dt = gdn.BF16 if dtype == "bf16" else gdn.F32
    nws = lib.gdn_conv_chunk_fwd_workspace_bytes(in_dt, T, N, Hqk, Hv, K, V)
    assert (nws > 0) == (dtype == "bf16" and K == 128)
    ws = Guarded(nws) if nws else None
    ga, gb, gA, gdt = dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"])
    st = lib.gdn_conv_chunk_fwd(x.data_ptr(), cw.data_ptr(), cb.data_ptr(), in_dt, 4, 1e-6, ga.data_ptr(),
                                gb.data_ptr(), gA.data_ptr(), gdt.data_ptr(), 0.125, s0.data_ptr(), cu.data_ptr(),
                                None, N, 1, T, Hqk, Hv, K, V,
                                o.ptr, in_dt, fin.ptr, ws.ptr if ws else None, nws, _stream())
    assert st == 0
    o.check("o")
    fin.check("final_state")
    if ws:
        ws.check("workspace")
    rows = o.payload((T, Hv * V * es))
    last = int(d["cu_seqlens"][-2])
    assert bool((rows[last:] == PATTERN).all()), "o rows of tokens in no sample were written"
    vals = rows[:last].view(torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert bool(torch.isfinite(vals).all())


@pytest.mark.parametrize("dtype,V,many", [("bf16", 128, False), ("f32", 96, False), ("bf16", 128, True)])
def test_segment_scan_and_segmented_forward_write_nothing_outside(dtype, V, many):
    """MFMA and vector-ALU shapes, and a chain of 39 maps."""
    lib = gdn.load_library()
    Hqk, Hv, K = 2, 4, 128
    T = 600
    in_dt = gdn.BF16 if dtype == "bf16" else gdn.F32
    d, t = _inputs([T], Hqk, Hv, K, V, dtype=dtype, s0=True)
    off = np.array([0, 64, 64, 333, 600], dtype=np.int32)  # an empty and a ragged segment
    if many:
        off = np.concatenate([[0], np.arange(1, 40) * 15, [600]]).astype(np.int32)
        off[20] = off[19]
    P = len(off) - 1
    off_dev = dev(off, "i32")
    M = Guarded(P * Hv * K * K * 4)
    b = Guarded(P * Hv * K * V * 4)
    starts = Guarded(P * Hv * K * V * 4)
    fin = Guarded(Hv * K * V * 4)
    ws_bytes = lib.gdn_segment_state_scan_workspace_bytes(T, P, Hv, K, V)
    ws = Guarded(ws_bytes)
    st = lib.gdn_segment_state_scan(t["k"].data_ptr(), t["v"].data_ptr(), in_dt, 0, 0, t["g"].data_ptr(),
                                    t["beta"].data_ptr(), off_dev.data_ptr(), _host_cu(off), P,
                                    t["s0"].data_ptr(), T, Hqk, Hv, K, V, M.ptr, b.ptr, starts.ptr, fin.ptr,
                                    ws.ptr, ws_bytes, _stream())
    assert st == 0
    for buf, name in ((M, "M"), (b, "b"), (starts, "starts"), (fin, "final_state"), (ws, "workspace")):
        buf.check("segment scan " + name)
    o = Guarded(T * Hv * V * 4)
    fin2 = Guarded(Hv * K * V * 4)
    ws_bytes = lib.gdn_segmented_workspace_bytes(T, P, Hv, K, V)
    ws2 = Guarded(ws_bytes)
    st = lib.gdn_chunk_fwd_segmented(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), in_dt, 0, 0, 0,
                                     t["g"].data_ptr(), t["beta"].data_ptr(), 0.1, t["s0"].data_ptr(),
                                     off_dev.data_ptr(), _host_cu(off), P, T, Hqk, Hv, K, V, o.ptr, gdn.F32,
                                     fin2.ptr, ws2.ptr, ws_bytes, _stream())
    assert st == 0
    for buf, name in ((o, "o"), (fin2, "final_state"), (ws2, "workspace")):
        buf.check("segmented forward " + name)


def test_gated_norm_writes_nothing_outside():
    lib = gdn.load_library()
    Hqk, Hv, K, V = 2, 4, 128, 128
    d, t = _inputs(LENGTHS, Hqk, Hv, K, V)
    T, N = sum(LENGTHS), len(LENGTHS)
    z = dev(np.random.default_rng(4).standard_normal((T, Hv, V)).astype(np.float32), "bf16")
    # fused into the scan's write-out (V = 128), bf16 y
    y = Guarded(T * Hv * V * 2)
    fin = Guarded(N * Hv * K * V * 4)
    ws_bytes = lib.gdn_chunk_fwd_workspace_bytes(gdn.BF16, T, N, Hv, K, V)
    ws = Guarded(ws_bytes)
    st = lib.gdn_chunk_fwd_gated_norm(
        t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), gdn.BF16, 0, 0, 0, t["g"].data_ptr(),
        t["beta"].data_ptr(), 0.1, t["s0"].data_ptr(), t["cu"].data_ptr(), _host_cu(t["cu_np"]), N, 1, T, Hqk, Hv, K,
        V, z.data_ptr(), gdn.BF16, None, 1e-6, y.ptr, gdn.BF16, fin.ptr, ws.ptr, ws_bytes, _stream())
    assert st == 0
    for buf, name in ((y, "y"), (fin, "final_state"), (ws, "workspace")):
        buf.check("fused gated norm " + name)
    # the norm kernel alone
    o = torch.randn((T * Hv, V), device="cuda:0")
    y2 = Guarded(T * Hv * V * 2)
    st = lib.gdn_gated_rmsnorm_fwd(o.data_ptr(), gdn.F32, z.data_ptr(), gdn.BF16, None, 1e-6, T * Hv, V, y2.ptr,
                                   gdn.BF16, _stream())
    assert st == 0
    y2.check("gated norm y")


def test_decode_writes_nothing_outside():
    lib = gdn.load_library()
    Hqk, Hv, K, V = 2, 4, 128, 128
    N, R = 5, 9
    d = gdn_inputs.small(92, [1] * N, Hqk, Hv, K, V, "bf16", s0_std=0.05)
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    q, k, v = dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(d["v"], "bf16")
    state = Guarded(R * Hv * K * V * 4, torch.float32)
    state.payload().normal_()
    before = state.payload((R, Hv * K * V)).clone()
    idx = dev(np.array([3, -1, 0, 8, 5], dtype=np.int32), "i32")  # one padding slot; rows 1, 2, 4, 6, 7 unused
    o = Guarded(N * Hv * V * 4)
    st = lib.gdn_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), gdn.BF16, g.data_ptr(), beta.data_ptr(), 0.1,
                             state.ptr, idx.data_ptr(), R, N, Hqk, Hv, K, V, o.ptr, gdn.F32, _stream())
    assert st == 0
    state.check("decode state")
    o.check("decode o")
    after = state.payload((R, Hv * K * V))
    for r in (1, 2, 4, 6, 7):
        assert torch.equal(after[r], before[r]), "state row %d not named by any sequence was written" % r
