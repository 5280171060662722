"""The C ABI library: loads, exports every symbol include/gdn.h declares, and
rejects bad arguments on the host before touching a GPU (so these run without
one: validation happens before any HIP call)."""

import ctypes
import os
import re

import pytest

import gated_deltanet_linear_chunk_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULLP, SHAPE, DTYPE, UNSUP, SEQ, HIP, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.library_path()):
        from gated_deltanet_linear_chunk_amd import build

        build.build()
    return gdn.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(gdn.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for s in range(8):
        assert lib.gdn_status_string(s)
    assert b"unknown" in lib.gdn_status_string(99)
    assert lib.gdn_abi_version() == 3


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def _chunk(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=1, qs=0, ks=0, vs=0, g=FAKE, beta=FAKE, scale=1.0, s0=None, cu=None,
                cu_host=None,
                n_seqs=0, B=1, T=64, Hqk=16, Hv=32, K=128, V=128, o=FAKE, o_dt=0, fin=None, ws=FAKE,
                ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return lib.gdn_chunk_fwd(*args.values())


def test_chunk_validation(lib):
    assert _chunk(lib, q=None) == NULLP
    assert _chunk(lib, o=None) == NULLP
    assert _chunk(lib, in_dt=7) == DTYPE
    assert _chunk(lib, o_dt=5) == DTYPE
    assert _chunk(lib, B=0) == SHAPE
    assert _chunk(lib, T=-1) == SHAPE
    assert _chunk(lib, qs=100) == SHAPE  # below the dense 16 * 128
    assert _chunk(lib, vs=32 * 128 + 4) == SHAPE  # not a multiple of 8
    assert _chunk(lib, ks=8192, qs=8192, vs=8192, q=None) == NULLP  # a wide stride itself is fine
    big = (1 << 24) - 8  # largest stride accepted: the kernels form in-chunk offsets with 24-bit multiplies
    assert _chunk(lib, ks=big, qs=big, vs=big, q=None) == NULLP
    assert _chunk(lib, ks=1 << 24) == SHAPE
    assert _chunk(lib, qs=1 << 24) == SHAPE
    assert _chunk(lib, vs=1 << 24) == SHAPE
    assert _chunk(lib, Hqk=3) == SHAPE  # 32 % 3 != 0
    assert _chunk(lib, K=96) == UNSUP  # K in {32, 64, 128}
    assert _chunk(lib, V=100) == UNSUP  # V a multiple of 32
    assert _chunk(lib, in_dt=0, K=96) == UNSUP
    assert _chunk(lib, in_dt=0, K=32, V=48) == UNSUP
    # bf16 K = 32 / 64, V = 32 and fp32 K = 128 run the vector-ALU kernel: supported, no workspace
    assert _chunk(lib, K=64, V=32, ws=None, q=None) == NULLP
    assert _chunk(lib, in_dt=0, K=128, ws=None, q=None) == NULLP
    assert lib.gdn_chunk_fwd_workspace_bytes(1, 64, 1, 32, 64, 128) == 0
    assert _chunk(lib, cu=FAKE, n_seqs=2, B=2) == SEQ  # cu_seqlens needs B == 1
    assert _chunk(lib, cu=FAKE, n_seqs=0) == SEQ
    bad = (ctypes.c_int32 * 3)(0, 40, 30)  # decreasing
    assert _chunk(lib, cu=FAKE, cu_host=bad, n_seqs=2) == SEQ
    short = (ctypes.c_int32 * 3)(0, 30, 60)  # does not end at T
    assert _chunk(lib, cu=FAKE, cu_host=short, n_seqs=2) == SEQ
    start = (ctypes.c_int32 * 3)(4, 30, 64)
    assert _chunk(lib, cu=FAKE, cu_host=start, n_seqs=2) == SEQ
    assert _chunk(lib, ws=None) == NULLP  # the bf16 path needs its T workspace
    need = lib.gdn_chunk_fwd_workspace_bytes(1, 64, 1, 32, 128, 128)
    record = 4 * 10 * 256 * 2 + 2 * 64 * 4  # per (chunk slot, v-head)
    plain = record * (1 + 1) * 32  # records of every chunk slot; the query adds room for splitting
    assert need >= plain
    assert _chunk(lib, ws_bytes=plain - 1) == SHAPE
    assert lib.gdn_chunk_fwd_workspace_bytes(0, 64, 1, 2, 32, 32) == 0  # fp32 path needs none
    # nothing to do: no tokens and no state requested
    assert _chunk(lib, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def _chunk_noalloc(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=1, qs=0, ks=0, vs=0, g=FAKE, beta=FAKE, scale=1.0, s0=None, cu=None,
                cu_host=None, n_seqs=0, B=1, T=64, Hqk=16, Hv=32, K=128, V=128, o=FAKE, o_dt=0, fin=None, stream=None)
    args.update(kw)
    return lib.gdn_chunk_fwd_noalloc(*args.values())


def test_chunk_noalloc_validation(lib):
    # every argument check runs before the fixed array is looked up (no HIP call here)
    assert _chunk_noalloc(lib, q=None) == NULLP
    assert _chunk_noalloc(lib, in_dt=7) == DTYPE
    assert _chunk_noalloc(lib, B=0) == SHAPE
    assert _chunk_noalloc(lib, qs=100) == SHAPE
    assert _chunk_noalloc(lib, K=96) == UNSUP
    assert _chunk_noalloc(lib, cu=FAKE, n_seqs=2, B=2) == SEQ
    # the records of 20992 bytes per (chunk slot, v-head) must fit GDN_NOALLOC_SCRATCH_BYTES
    record = 4 * 10 * 256 * 2 + 2 * 64 * 4
    assert record == 20992
    slots_max = gdn.NOALLOC_SCRATCH_BYTES // (record * 32)
    assert slots_max == 199
    T = 64 * (slots_max - 1)  # 198 chunks + 1 sequence = 199 slots, the most that fit
    assert _chunk_noalloc(lib, T=T + 64) == SCRATCH
    assert _chunk_noalloc(lib, B=2, T=T) == SCRATCH  # 2 rows: two more slots than one row
    cu_host = (ctypes.c_int32 * 3)(0, 64, 128)
    assert _chunk_noalloc(lib, T=64 * 198, cu=FAKE, cu_host=None, n_seqs=2) == SCRATCH
    assert _chunk_noalloc(lib, T=128, cu=FAKE, cu_host=cu_host, n_seqs=2, Hv=32 * 100) == SCRATCH
    # fp32 inputs use no records: the size limit does not apply
    assert _chunk_noalloc(lib, in_dt=0, K=32, V=32, Hqk=2, Hv=4, T=1 << 20, q=None) == NULLP


def _chunk_norm(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=1, qs=0, ks=0, vs=0, g=FAKE, beta=FAKE, scale=1.0, s0=None, cu=None,
                cu_host=None, n_seqs=0, B=1, T=64, Hqk=16, Hv=32, K=128, V=128, z=FAKE, z_dt=1, nw=None, eps=1e-6,
                o=FAKE, o_dt=0, fin=None, ws=FAKE, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return lib.gdn_chunk_fwd_gated_norm(*args.values())


def test_chunk_gated_norm_validation(lib):
    assert _chunk_norm(lib, z_dt=3) == DTYPE
    assert _chunk_norm(lib, o_dt=3) == DTYPE
    assert _chunk_norm(lib, eps=-1.0) == SHAPE
    assert _chunk_norm(lib, eps=float("nan")) == SHAPE
    assert _chunk_norm(lib, z=None) == NULLP  # fused path (bf16, V = 128)
    assert _chunk_norm(lib, z=None, V=256) == NULLP  # chunk forward + norm kernel
    assert _chunk_norm(lib, in_dt=0, K=32, V=96) == UNSUP  # no norm kernel for V = 96
    # more norm rows than the norm kernel's grid holds: refused before the chunk forward is enqueued
    assert _chunk_norm(lib, V=256, T=(1 << 31) - 1) == UNSUP
    assert _chunk_norm(lib, q=None) == NULLP  # the chunk forward's own checks still apply
    assert _chunk_norm(lib, K=96) == UNSUP
    assert _chunk_norm(lib, ws=None) == NULLP
    assert _chunk_norm(lib, T=0, q=None, k=None, v=None, g=None, beta=None, o=None, z=None) == OK
    assert _chunk_norm(lib, T=0, V=256, q=None, k=None, v=None, g=None, beta=None, o=None, z=None) == OK


def test_conv_validation(lib):
    def conv(**kw):
        a = dict(x=FAKE, w=FAKE, bias=None, dt=1, cu=None, cu_host=None, n=0, B=1, T=32, C=8192, W=4, silu=1,
                 l2=4096, hd=128, eps=1e-6, rounding=0, y=FAKE, stream=None)
        a.update(kw)
        return lib.gdn_conv1d_fwd(*a.values())

    assert conv(x=None) == NULLP
    assert conv(dt=3) == DTYPE
    assert conv(C=100) == SHAPE  # channels % 8
    assert conv(W=5) == UNSUP
    assert conv(W=0) == UNSUP
    assert conv(l2=100) == SHAPE
    assert conv(hd=96) == UNSUP
    assert conv(cu=FAKE, n=2, B=2) == SEQ
    assert conv(cu=FAKE, n=2, cu_host=(ctypes.c_int32 * 3)(0, 10, 31)) == SEQ
    assert conv(T=0, x=None, w=None, y=None) == OK
    assert conv(rounding=2) == SHAPE  # GDN_ROUND_FAST (0) or GDN_ROUND_EXACT (1)
    assert conv(rounding=1, x=None) == NULLP


def test_conv_chunk_validation(lib):
    def cc(**kw):
        a = dict(x=FAKE, w=FAKE, bias=None, in_dt=1, W=4, eps=1e-6, ga=FAKE, gb=FAKE, A_log=FAKE, dt_bias=FAKE,
                 scale=1.0, s0=None, cu=None,
                 cu_host=None, n_seqs=0, B=1, T=64, Hqk=16, Hv=32, K=128, V=128, o=FAKE, o_dt=0, fin=None,
                 ws=FAKE, ws_bytes=1 << 40, stream=None)
        a.update(kw)
        return lib.gdn_conv_chunk_fwd(*a.values())

    assert cc(x=None) == NULLP
    assert cc(w=None) == NULLP
    assert cc(ga=None) == NULLP
    assert cc(gb=None) == NULLP
    assert cc(A_log=None) == NULLP
    assert cc(dt_bias=None) == NULLP
    assert cc(o=None) == NULLP
    assert cc(in_dt=3) == DTYPE
    assert cc(o_dt=3) == DTYPE
    assert cc(B=0) == SHAPE
    assert cc(Hv=24) == SHAPE  # H_v % H_qk
    assert cc(eps=0.0) == SHAPE
    assert cc(eps=float("nan")) == SHAPE
    assert cc(W=5) == UNSUP
    assert cc(W=0) == UNSUP
    assert cc(K=96) == UNSUP
    assert cc(V=100) == UNSUP
    assert cc(cu=FAKE, n_seqs=2, B=2) == SEQ
    assert cc(cu=FAKE, n_seqs=2, cu_host=(ctypes.c_int32 * 3)(0, 10, 63)) == SEQ  # must end at T
    assert cc(cu=FAKE, n_seqs=0) == SEQ
    assert cc(T=0, x=None, w=None, ga=None, gb=None, A_log=None, dt_bias=None, o=None) == OK  # nothing to do
    # bf16 with the MFMA head sizes needs the workspace its query names
    need = lib.gdn_conv_chunk_fwd_workspace_bytes(1, 64, 1, 16, 32, 128, 128)
    assert need > 64 * (2 * 16 * 128 + 32 * 128) * 2
    assert cc(ws=None) == NULLP
    assert cc(ws_bytes=need - 1) == SHAPE
    # the vector-ALU shapes need none
    assert lib.gdn_conv_chunk_fwd_workspace_bytes(0, 64, 1, 16, 32, 128, 128) == 0  # fp32
    assert lib.gdn_conv_chunk_fwd_workspace_bytes(1, 64, 1, 16, 32, 64, 64) == 0  # K = 64
    assert lib.gdn_conv_chunk_fwd_workspace_bytes(1, 64, 1, 4, 32, 128, 128) == 0  # 8 v-heads per q/k head


def test_gate_and_segment_validation(lib):
    assert lib.gdn_gate_fwd(FAKE, FAKE, FAKE, FAKE, 10, 0, FAKE, FAKE, None) == SHAPE
    assert lib.gdn_gate_fwd(None, FAKE, FAKE, FAKE, 10, 4, FAKE, FAKE, None) == NULLP
    assert lib.gdn_gate_fwd(None, None, None, None, 0, 4, None, None, None) == OK

    def scan(**kw):
        a = dict(k=FAKE, v=FAKE, dt=1, ks=0, vs=0, g=FAKE, beta=FAKE, off=FAKE, off_host=None, P=8, s0=None, T=4096,
                 Hqk=16,
                 Hv=32, K=128, V=128, M=FAKE, b=FAKE, starts=FAKE, fin=None, ws=FAKE, ws_bytes=1 << 40,
                 stream=None)
        a.update(kw)
        return lib.gdn_segment_state_scan(*a.values())

    assert scan(off=None) == NULLP
    assert scan(ks=12) == SHAPE
    assert scan(vs=1 << 24) == SHAPE
    assert scan(M=None) == NULLP
    assert scan(ws=None) == NULLP
    assert scan(ws_bytes=lib.gdn_segment_state_scan_workspace_bytes(4096, 8, 32, 128, 128) - 4) == SHAPE
    # K = 128 only; bf16 with V % 128 == 0 on the MFMA kernels, otherwise fp32 or
    # V % 32 == 0 on the vector-ALU kernel (which needs no workspace)
    assert scan(dt=0, K=64) == UNSUP
    assert scan(dt=1, K=32, V=32) == UNSUP
    assert scan(dt=0, V=200) == UNSUP
    assert scan(dt=0, M=None, ws=None) == NULLP  # fp32 accepted; the outputs are still required
    assert scan(V=96, starts=None, ws=None) == NULLP  # bf16 with V = 96 accepted
    assert scan(P=0) == SHAPE
    assert scan(V=200) == UNSUP
    off = (ctypes.c_int32 * 3)(0, 5000, 4096)
    assert scan(P=2, off_host=off) == SEQ
    # segmented forward: records of all P segments, then M, b and starts of the
    # P - 1 segments that precede another, then 2 P ints of start/final maps
    def a256(x):
        return (x + 255) // 256 * 256
    rec = lib.gdn_segment_state_scan_workspace_bytes(4096, 8, 32, 128, 128)
    assert lib.gdn_segmented_workspace_bytes(4096, 8, 32, 128, 128) == \
        a256(rec) + a256(4 * 7 * 32 * 128 * 128) + 2 * a256(4 * 7 * 32 * 128 * 128) + a256(4 * 16)
    assert lib.gdn_segmented_workspace_bytes(4096, 0, 32, 128, 128) == 0

    def seg(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dt=1, qs=0, ks=0, vs=0, g=FAKE, beta=FAKE, scale=1.0, s0=None, off=FAKE,
                 off_host=(ctypes.c_int32 * 3)(0, 2048, 4096), P=2, T=4096, Hqk=16, Hv=32, K=128, V=128, o=FAKE,
                 o_dt=0, fin=None, ws=FAKE, ws_bytes=lib.gdn_segmented_workspace_bytes(4096, 2, 32, 128, 128),
                 stream=None)
        a.update(kw)
        return lib.gdn_chunk_fwd_segmented(*a.values())

    ws = lib.gdn_segmented_workspace_bytes(4096, 2, 32, 128, 128)
    assert seg(ws_bytes=ws - 1) == SHAPE
    assert seg(ws=None) == NULLP
    assert seg(off_host=(ctypes.c_int32 * 3)(0, 2048, 4000)) == SEQ
    # every argument is checked before pass 1 writes anything, the q stride included
    assert seg(qs=100) == SHAPE
    assert seg(qs=1 << 24) == SHAPE
    assert seg(o=None) == NULLP
    assert seg(q=None) == NULLP
    assert seg(o_dt=4) == DTYPE
    assert seg(dt=0, K=64) == UNSUP
    assert seg(dt=0, q=None) == NULLP  # fp32 accepted
    assert seg(V=96, o=None) == NULLP  # bf16 with V = 96 accepted
    assert seg(K=64) == UNSUP
    assert seg(Hqk=3) == SHAPE
    assert seg(P=0) == SHAPE
    # no tokens and no final state requested: nothing to do
    assert seg(T=0, off_host=(ctypes.c_int32 * 3)(0, 0, 0), q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def test_decode_validation(lib):
    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dt=1, g=FAKE, beta=FAKE, scale=1.0, state=FAKE, idx=None, rows=64, N=64,
                 Hqk=16, Hv=32, K=128, V=128, o=FAKE, o_dt=1, stream=None)
        a.update(kw)
        return lib.gdn_decode_step(*a.values())

    assert dec(dt=7) == DTYPE
    assert dec(o_dt=7) == DTYPE
    assert dec(N=-1) == SHAPE
    assert dec(Hv=24) == SHAPE  # not a multiple of H_qk
    assert dec(rows=63) == SHAPE  # fewer state rows than sequences, no indices
    assert dec(K=96) == UNSUP
    assert dec(V=100) == UNSUP
    assert dec(N=70000, rows=70000) == UNSUP
    assert dec(state=None) == NULLP
    assert dec(o=None) == NULLP
    assert dec(N=0, q=None, k=None, v=None, g=None, beta=None, state=None, o=None) == OK


def test_gated_norm_validation(lib):
    def gn(**kw):
        a = dict(o=FAKE, o_dt=0, z=FAKE, z_dt=1, w=None, eps=1e-6, rows=100, V=128, y=FAKE, y_dt=1, stream=None)
        a.update(kw)
        return lib.gdn_gated_rmsnorm_fwd(*a.values())

    assert gn(o_dt=9) == DTYPE
    assert gn(y_dt=9) == DTYPE
    assert gn(rows=-1) == SHAPE
    assert gn(eps=-1.0) == SHAPE
    assert gn(eps=float("nan")) == SHAPE
    assert gn(V=96) == UNSUP
    assert gn(z=None) == NULLP
    assert gn(rows=0, o=None, z=None, y=None) == OK


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        gdn.gdn_conv1d_fwd(x, torch.zeros(8, 4))
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros(1, 64, 4, 128, dtype=torch.bfloat16)
    g = torch.zeros(1, 64, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_chunk_fwd_gated_norm(q, q, v, g, g, v)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_gated_rmsnorm_fwd(v, v)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_conv_chunk_fwd(torch.zeros(1, 64, 1024), torch.zeros(1024, 4), g, g, torch.zeros(4), torch.zeros(4),
                               Hqk=2, K=128)
