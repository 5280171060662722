"""GPU parity at small sizes: every kernel against the fp64 oracle on the same
seeded inputs (sizes span several 64-token chunks and ragged tails), plus the
bit-exact properties (packed == per-sample, determinism, untouched memory).

The GPU side derives g and beta with its own gate kernel; the oracle derives
them in fp64 from the same raw draws.
"""

import numpy as np
import pytest

import gdn_inputs
import oracle
from parity_util import assert_units_bf16, TOL_F32_ABS, assert_bf16, assert_f32, dev, host, stats

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402


def _gpu_gates(d):
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    return g, beta


def _oracle_gates(d):
    return oracle.gates(d["a"], d["b"], d["A_log"], d["dt_bias"])


def _run_chunk(d, dtype, s0=None, o_dtype=None, use_cu=True):
    q = dev(d["q"], dtype)[None]
    k = dev(d["k"], dtype)[None]
    v = dev(d["v"], dtype)[None]
    g, beta = _gpu_gates(d)
    cu = dev(d["cu_seqlens"], "i32") if use_cu else None
    o, fin = gdn.gdn_chunk_fwd(
        q, k, v, g[None], beta[None], initial_state=None if s0 is None else dev(s0),
        cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens"] if use_cu else None, o_dtype=o_dtype,
    )
    torch.cuda.synchronize()
    return o[0], fin


def _oracle_chunk(d, s0=None):
    g, beta = _oracle_gates(d)
    return oracle.recurrence(d["q"], d["k"], d["v"], g, beta, s0, d["cu_seqlens"])


# --------------------------------------------------------------------------- #
def test_gate_kernel():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal((300, 8)) * 4).astype(np.float32)
    b = (rng.standard_normal((300, 8)) * 4).astype(np.float32)
    A_log = rng.uniform(-3, 3, 8).astype(np.float32)
    dt = rng.uniform(-1, 1, 8).astype(np.float32)
    g, beta = gdn.gdn_gate_fwd(dev(a), dev(b), dev(A_log), dev(dt))
    go, bo = oracle.gates(a, b, A_log, dt)
    np.testing.assert_allclose(host(g), go, rtol=2e-6, atol=1e-30)
    np.testing.assert_allclose(host(beta), bo, rtol=2e-6, atol=1e-30)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("l2", [False, True])
def test_conv1d_packed(dtype, l2):
    w = gdn_inputs.Workload("conv", 11, 300, 5, 2, 4, 128, 64, dtype, conv_width=4, lengths=[1, 63, 64, 2, 170])
    d = gdn_inputs.draw(w)
    C = d["x"].shape[1]
    l2ch = 2 * 2 * 128 if l2 else 0
    ref = oracle.conv1d(d["x"], d["conv_w"], d["conv_bias"], d["cu_seqlens"])
    if l2:
        q, k, _ = oracle.split_channels(ref, 2, 4, 128, 64)
        ref = ref.copy()
        ref[:, :l2ch] = np.concatenate([oracle.l2norm(q).reshape(300, -1), oracle.l2norm(k).reshape(300, -1)], 1)
    for exact in (False, True):
        y = gdn.gdn_conv1d_fwd(dev(d["x"], dtype), dev(d["conv_w"], dtype), dev(d["conv_bias"], dtype),
                               cu_seqlens=dev(d["cu_seqlens"], "i32"), cu_seqlens_host=d["cu_seqlens"],
                               l2norm_channels=l2ch, head_dim=128, exact_rounding=exact)
        got = host(y)
        assert got.shape == (300, C)
        if dtype == "f32":
            np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
            continue
        # the fp32 evaluation rounded once to bf16: within half a bf16 unit plus the fp32 error
        err = np.abs(got - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), float((err - 2.0 ** -8 * np.abs(ref)).max())
        if exact:
            # every output, normalised or not, is the bf16 nearest to the exact value
            np.testing.assert_array_equal(got, oracle.round_bf16(ref))


def test_conv1d_bf16_rounding_is_exact_at_scale():
    """Every unnormalised bf16 output equals the oracle's fp64 value rounded once to bf16, over
    enough values (about 2M) that the fp64 settling of doubtful roundings runs many times."""
    w = gdn_inputs.Workload("conv_big", 13, 2048, 3, 1, 8, 64, 128, "bf16", conv_width=4, lengths=[700, 1000, 348])
    d = gdn_inputs.draw(w)
    y = gdn.gdn_conv1d_fwd(dev(d["x"], "bf16"), dev(d["conv_w"], "bf16"), dev(d["conv_bias"], "bf16"),
                           cu_seqlens=dev(d["cu_seqlens"], "i32"), cu_seqlens_host=d["cu_seqlens"],
                           exact_rounding=True)
    ref = oracle.conv1d(d["x"], d["conv_w"], d["conv_bias"], d["cu_seqlens"])
    np.testing.assert_array_equal(host(y), oracle.round_bf16(ref))


def test_conv1d_batched_rows_and_width():
    rng = np.random.default_rng(12)
    B, T, C = 3, 70, 256
    x = gdn_inputs.bf16_round(rng.standard_normal((B, T, C)).astype(np.float32))
    for W in (1, 2, 3, 4):
        wt = gdn_inputs.bf16_round(rng.standard_normal((C, W)).astype(np.float32))
        cu = np.arange(B + 1) * T
        ref = oracle.conv1d(x.reshape(B * T, C), wt, None, cu, silu=False).reshape(B, T, C)
        y = gdn.gdn_conv1d_fwd(dev(x, "bf16"), dev(wt, "bf16"), None, apply_silu=False, exact_rounding=True)
        np.testing.assert_array_equal(host(y), oracle.round_bf16(ref))
        y = gdn.gdn_conv1d_fwd(dev(x, "bf16"), dev(wt, "bf16"), None, apply_silu=False)
        err = np.abs(host(y) - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), W


# --------------------------------------------------------------------------- #
def test_chunk_fp32_tiny_workload():
    d = gdn_inputs.draw(gdn_inputs.WORKLOADS["tiny_fp32_T256_H2_K32"])
    o, fin = _run_chunk(d, "f32")
    oref, fref = _oracle_chunk(d)
    assert_f32(host(o), oref, "o")
    assert_f32(host(fin), fref, "final")


@pytest.mark.parametrize("K,V", [(32, 32), (64, 64), (32, 96), (128, 32), (128, 128)])
def test_chunk_fp32_packed_with_state(K, V):
    d = gdn_inputs.small(21, [1, 64, 65, 130, 7], 2, 4, K, V, "f32")
    N = 5
    s0 = (np.random.default_rng(3).standard_normal((N, 4, K, V)) * 0.5).astype(np.float32)
    o, fin = _run_chunk(d, "f32", s0)
    oref, fref = _oracle_chunk(d, s0)
    assert_f32(host(o), oref, "o")
    assert_f32(host(fin), fref, "final")


@pytest.mark.parametrize("K,V", [(32, 32), (64, 128), (128, 32)])
@pytest.mark.parametrize("o_dtype", ["f32", "bf16"])
def test_chunk_bf16_small_heads_vector_kernel(K, V, o_dtype):
    """bf16 inputs of head sizes outside the MFMA kernel's (K = 128, V % 128 == 0) run the fp32
    vector-ALU kernel on the given bf16 values: fp32 arithmetic, so the fp32 bound holds (bf16 o
    adds its own rounding)."""
    d = gdn_inputs.small(22, [1, 64, 65, 130, 0, 7], 2, 4, K, V, "bf16")
    N = 6
    s0 = (np.random.default_rng(4).standard_normal((N, 4, K, V)) * 0.5).astype(np.float32)
    od = torch.float32 if o_dtype == "f32" else torch.bfloat16
    o, fin = _run_chunk(d, "bf16", s0, o_dtype=od)
    oref, fref = _oracle_chunk(d, s0)
    assert_f32(host(fin), fref, "final")
    if o_dtype == "f32":
        assert_f32(host(o), oref, "o")
    else:
        excess = np.abs(host(o) - oref) - (TOL_F32_ABS + 2.0 ** -8 * np.abs(oref))
        assert excess.max() <= 0, float(excess.max())


GATES = {
    "fast": dict(A_log_range=(0.0, float(np.log(16.0)))),
    "slow": dict(A_log_range=(-2.0, 0.0)),
    "very_slow": dict(A_log_range=(-8.0, -4.0)),
    "zero_decay": dict(gate_kind="zero_decay"),
}


@pytest.mark.parametrize("gates", list(GATES))
@pytest.mark.parametrize("V", [128, 256])
def test_chunk_bf16_packed(gates, V):
    lengths = [1, 63, 64, 65, 127, 300]
    d = gdn_inputs.small(31, lengths, 2, 4, 128, V, "bf16", **GATES[gates])
    s0 = (np.random.default_rng(4).standard_normal((len(lengths), 4, 128, V)) * 0.05).astype(np.float32)
    o, fin = _run_chunk(d, "bf16", s0, o_dtype=torch.float32)
    oref, fref = _oracle_chunk(d, s0)
    so = assert_bf16(host(o), oref, "o")
    sf = assert_bf16(host(fin), fref, "final")
    print("\nbf16 %s V=%d o %s final %s" % (gates, V, so, sf))


@pytest.mark.parametrize("gates", ["slow", "zero_decay", "fast"])
@pytest.mark.parametrize("V", [128, 256])
def test_chunk_bf16_split_long_samples(gates, V):
    """Packed samples of very different lengths with host offsets: the long ones are cut into
    segments (pass 1: first segments forward and the middle segments' maps; fp32 chains; pass 2
    from the composed starts); outputs and final states match the oracle, and the unsplit run
    (no host offsets) within the same bound."""
    lengths = [2500, 0, 700, 64, 1, 1350]
    d = gdn_inputs.small(38, lengths, 2, 4, 128, V, "bf16", **GATES[gates])
    s0 = (np.random.default_rng(8).standard_normal((len(lengths), 4, 128, V)) * 0.05).astype(np.float32)
    o, fin = _run_chunk(d, "bf16", s0, o_dtype=torch.float32)
    oref, fref = _oracle_chunk(d, s0)
    so = assert_bf16(host(o), oref, "o")
    sf = assert_bf16(host(fin), fref, "final")
    np.testing.assert_array_equal(host(fin)[1], s0[1])  # zero-length sample keeps its state
    print("\nsplit %s V=%d o %s final %s" % (gates, V, so, sf))
    q = dev(d["q"], "bf16")[None]
    k = dev(d["k"], "bf16")[None]
    v = dev(d["v"], "bf16")[None]
    g, beta = _gpu_gates(d)
    o2, f2 = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], initial_state=dev(s0),
                               cu_seqlens=dev(d["cu_seqlens"], "i32"), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_bf16(host(o2[0]), oref, "o unsplit")
    # Pass 1 runs the forward arithmetic, so where the decay drives a segment's start state below
    # fp32 rounding its map's b is the sequential state bit for bit, and the paths can agree
    # exactly; without decay the composed starts differ in the last bits.
    if gates == "zero_decay":
        assert not torch.equal(o2[0], o)  # the split path really ran


@pytest.mark.parametrize("V", [384, 512])
def test_chunk_bf16_three_and_four_column_tiles(V):
    """V = 384 and 512: three and four 128-column workgroups per head, in the split packed run
    (forward and map blocks of pass 1 over 4 and 5 tiles), the unsplit run and batched rows; every
    unit against the oracle."""
    lengths = [2500, 0, 700, 64, 1, 1350]
    d = gdn_inputs.small(40 + V, lengths, 2, 4, 128, V, "bf16", **GATES["slow"])
    s0 = (np.random.default_rng(12).standard_normal((len(lengths), 4, 128, V)) * 0.05).astype(np.float32)
    oref, fref = _oracle_chunk(d, s0)
    cu = d["cu_seqlens"]
    o, fin = _run_chunk(d, "bf16", s0, o_dtype=torch.float32)
    assert_units_bf16(host(o), oref, cu, "split V=%d" % V, fin=host(fin), fref=fref)
    q, k, v = (dev(d[n], "bf16")[None] for n in ("q", "k", "v"))
    g, beta = _gpu_gates(d)
    o2, f2 = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], initial_state=dev(s0), cu_seqlens=dev(cu, "i32"),
                               o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_units_bf16(host(o2[0]), oref, cu, "unsplit V=%d" % V, fin=host(f2), fref=fref)
    # batched rows: two rows of 300 tokens
    db = gdn_inputs.small(41 + V, [300, 300], 2, 4, 128, V, "bf16", **GATES["slow"])
    s0b = s0[:2]
    q, k, v = (dev(db[n], "bf16").reshape(2, 300, *db[n].shape[1:]) for n in ("q", "k", "v"))
    g, beta = _gpu_gates(db)
    o3, f3 = gdn.gdn_chunk_fwd(q, k, v, g.reshape(2, 300, 4), beta.reshape(2, 300, 4), initial_state=dev(s0b),
                               o_dtype=torch.float32)
    torch.cuda.synchronize()
    orefb, frefb = _oracle_chunk(db, s0b)
    assert_units_bf16(host(o3).reshape(600, 4, V), orefb, db["cu_seqlens"], "batched V=%d" % V, fin=host(f3),
                      fref=frefb)


def test_chunk_bf16_gqa_ratio_three():
    """Three v-heads per q/k head (H_qk = 8, H_v = 24): the prep builds one v-head per wave and the
    scan places each q/k head's three v-heads on one XCD; packed samples with host offsets and
    start states match the oracle."""
    lengths = [3000, 1, 130, 64]
    d = gdn_inputs.small(39, lengths, 8, 24, 128, 128, "bf16", A_log_range=(-2.0, 0.0))
    s0 = (np.random.default_rng(9).standard_normal((len(lengths), 24, 128, 128)) * 0.05).astype(np.float32)
    o, fin = _run_chunk(d, "bf16", s0, o_dtype=torch.float32)
    oref, fref = _oracle_chunk(d, s0)
    so = assert_bf16(host(o), oref, "o")
    sf = assert_bf16(host(fin), fref, "final")
    print("\ngqa 3: o %s final %s" % (so, sf))


def test_chunk_bf16_store_o_bf16():
    d = gdn_inputs.small(32, [200, 57], 1, 2, 128, 128, "bf16")
    o, _ = _run_chunk(d, "bf16", o_dtype=torch.bfloat16)
    oref, _ = _oracle_chunk(d)
    assert_bf16(host(o), oref, "o bf16", bf16_store=True)


def test_chunk_bf16_batched_rows_equal_packed():
    """B rows without cu_seqlens give the same bits as the packed form."""
    lengths = [128, 128, 128]
    d = gdn_inputs.small(33, lengths, 2, 4, 128, 128, "bf16")
    s0 = (np.random.default_rng(5).standard_normal((3, 4, 128, 128)) * 0.02).astype(np.float32)
    o_p, f_p = _run_chunk(d, "bf16", s0, o_dtype=torch.float32)
    g, beta = _gpu_gates(d)
    q = dev(d["q"], "bf16").reshape(3, 128, 2, 128)
    k = dev(d["k"], "bf16").reshape(3, 128, 2, 128)
    v = dev(d["v"], "bf16").reshape(3, 128, 4, 128)
    o_b, f_b = gdn.gdn_chunk_fwd(q, k, v, g.reshape(3, 128, 4), beta.reshape(3, 128, 4),
                                 initial_state=dev(s0), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_b.reshape(o_p.shape), o_p)
    assert torch.equal(f_b, f_p)


def test_chunk_bf16_packed_equals_per_sample_bitwise():
    lengths = [65, 1, 130, 64]
    d = gdn_inputs.small(34, lengths, 2, 4, 128, 128, "bf16", A_log_range=(-2.0, 0.0))
    o, fin = _run_chunk(d, "bf16", o_dtype=torch.float32)
    cu = d["cu_seqlens"]
    g, beta = _gpu_gates(d)
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        on, fn = gdn.gdn_chunk_fwd(dev(d["q"][a:b], "bf16")[None], dev(d["k"][a:b], "bf16")[None],
                                   dev(d["v"][a:b], "bf16")[None], g[a:b][None].contiguous(),
                                   beta[a:b][None].contiguous(), o_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(on[0], o[a:b]), n
        assert torch.equal(fn[0], fin[n]), n


def test_chunk_bf16_deterministic_and_leak_free():
    lengths = [100, 150]
    d = gdn_inputs.small(35, lengths, 2, 4, 128, 128, "bf16", A_log_range=(-2.0, 0.0))
    o1, f1 = _run_chunk(d, "bf16", o_dtype=torch.float32)
    o2, f2 = _run_chunk(d, "bf16", o_dtype=torch.float32)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    d2 = dict(d)
    d2["v"] = d["v"].copy()
    d2["v"][100:] = gdn_inputs.bf16_round(d2["v"][100:] + 1.0)
    o3, f3 = _run_chunk(d2, "bf16", o_dtype=torch.float32)
    assert torch.equal(o3[:100], o1[:100]) and torch.equal(f3[0], f1[0])
    assert not torch.equal(o3[100:], o1[100:])


def test_chunk_zero_length_samples_keep_state():
    lengths = [0, 70, 0]
    d = gdn_inputs.small(36, lengths, 1, 2, 128, 128, "bf16")
    s0 = (np.random.default_rng(6).standard_normal((3, 2, 128, 128))).astype(np.float32)
    o, fin = _run_chunk(d, "bf16", s0, o_dtype=torch.float32)
    f = host(fin)
    np.testing.assert_array_equal(f[0], s0[0])
    np.testing.assert_array_equal(f[2], s0[2])
    oref, fref = _oracle_chunk(d, s0)
    assert_bf16(host(o), oref, "o")


def test_chunk_scale_argument():
    d = gdn_inputs.small(37, [90], 1, 2, 128, 128, "bf16")
    g, beta = _gpu_gates(d)
    args = (dev(d["q"], "bf16")[None], dev(d["k"], "bf16")[None], dev(d["v"], "bf16")[None], g[None], beta[None])
    o1, _ = gdn.gdn_chunk_fwd(*args, o_dtype=torch.float32)
    o2, _ = gdn.gdn_chunk_fwd(*args, scale=0.25, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1 * 0.25)


# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("gates", ["zero_decay", "very_slow", "fast"])
def test_segment_state_scan(gates):
    T = 512
    d = gdn_inputs.small(41, [T], 2, 4, 128, 128, "bf16", **GATES[gates])
    off = np.array([0, 64, 100, 256, 257, 512], dtype=np.int32)
    s0 = (np.random.default_rng(8).standard_normal((4, 128, 128)) * 0.1).astype(np.float32)
    g, beta = _gpu_gates(d)
    M, b, starts, fin = gdn.gdn_segment_state_scan(dev(d["k"], "bf16"), dev(d["v"], "bf16"), g, beta,
                                                   dev(off, "i32"), off, initial_state=dev(s0))
    torch.cuda.synchronize()
    go, bo = _oracle_gates(d)
    Mref, bref = oracle.segment_affine(d["k"], d["v"], go, bo, off, Hqk=2)
    sref, fref = oracle.chain(Mref, bref, s0)
    for i in range(len(off) - 1):
        if gates != "fast":  # fast gates drive M below the fp32 range; nothing to compare
            assert_bf16(host(M[i]), Mref[i], "M[%d]" % i)
        assert_bf16(host(b[i]), bref[i], "b[%d]" % i)
        assert_bf16(host(starts[i]), sref[i], "start[%d]" % i)
    assert_bf16(host(fin), fref, "final")


@pytest.mark.parametrize("gates", ["zero_decay", "slow"])
def test_segmented_forward_matches_oracle(gates):
    T = 640
    d = gdn_inputs.small(42, [T], 2, 4, 128, 128, "bf16", **GATES[gates])
    off = np.array([0, 128, 320, 321, 640], dtype=np.int32)
    s0 = (np.random.default_rng(9).standard_normal((1, 4, 128, 128)) * 0.05).astype(np.float32)
    g, beta = _gpu_gates(d)
    o, fin = gdn.gdn_chunk_fwd_segmented(dev(d["q"], "bf16")[None], dev(d["k"], "bf16")[None],
                                         dev(d["v"], "bf16")[None], g[None], beta[None], dev(off, "i32"), off,
                                         initial_state=dev(s0[0]), o_dtype=torch.float32)
    torch.cuda.synchronize()
    oref, fref = _oracle_chunk(d, s0)
    assert_bf16(host(o[0]), oref, "o")
    assert_bf16(host(fin), fref[0], "final")
    # one segment is exactly the plain path
    one = np.array([0, T], dtype=np.int32)
    o1, _ = gdn.gdn_chunk_fwd_segmented(dev(d["q"], "bf16")[None], dev(d["k"], "bf16")[None],
                                        dev(d["v"], "bf16")[None], g[None], beta[None], dev(one, "i32"), one,
                                        initial_state=dev(s0[0]), o_dtype=torch.float32)
    o2, f2 = gdn.gdn_chunk_fwd(dev(d["q"], "bf16")[None], dev(d["k"], "bf16")[None], dev(d["v"], "bf16")[None],
                               g[None], beta[None], initial_state=dev(s0), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    # two segments cut at a chunk boundary: pass 1 runs segment 0 forward and segment 1 starts from
    # its end state, with no map and no chain, so the result is the plain path's bit for bit
    two = np.array([0, 256, T], dtype=np.int32)
    o3, f3 = gdn.gdn_chunk_fwd_segmented(dev(d["q"], "bf16")[None], dev(d["k"], "bf16")[None],
                                         dev(d["v"], "bf16")[None], g[None], beta[None], dev(two, "i32"), two,
                                         initial_state=dev(s0[0]), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o3, o2) and torch.equal(f3, f2[0])


@pytest.mark.parametrize("dtype,V,gates", [("f32", 128, "slow"), ("f32", 32, "zero_decay"), ("bf16", 96, "slow"),
                                            ("f32", 64, "fast")])
def test_segment_state_scan_vector_alu(dtype, V, gates):
    """K = 128 segment scans outside the MFMA shapes (fp32 inputs, or bf16 with V % 128 != 0): pass 1
    on the vector-ALU kernel, M, b, the chained starts and the final state against the oracle."""
    T = 512
    d = gdn_inputs.small(43, [T], 2, 4, 128, V, dtype, **GATES[gates])
    off = np.array([0, 64, 100, 256, 257, 512], dtype=np.int32)
    s0 = (np.random.default_rng(8).standard_normal((4, 128, V)) * 0.1).astype(np.float32)
    g, beta = _gpu_gates(d)
    M, b, starts, fin = gdn.gdn_segment_state_scan(dev(d["k"], dtype), dev(d["v"], dtype), g, beta,
                                                   dev(off, "i32"), off, initial_state=dev(s0))
    torch.cuda.synchronize()
    go, bo = _oracle_gates(d)
    Mref, bref = oracle.segment_affine(d["k"], d["v"], go, bo, off, Hqk=2)
    sref, fref = oracle.chain(Mref, bref, s0)
    check = assert_f32 if dtype == "f32" else assert_bf16
    for i in range(len(off) - 1):
        check(host(M[i]), Mref[i], "M[%d]" % i)
        check(host(b[i]), bref[i], "b[%d]" % i)
        check(host(starts[i]), sref[i], "start[%d]" % i)
    check(host(fin), fref, "final")


@pytest.mark.parametrize("dtype,V", [("f32", 128), ("bf16", 32), ("f32", 96)])
def test_segmented_forward_vector_alu(dtype, V):
    """The segmented forward on the vector-ALU kernel (pass 1, fp32 chain, pass 2 from the chained
    starts through the start/final-state maps) against the oracle; one segment equals the plain call."""
    T = 640
    d = gdn_inputs.small(44, [T], 2, 4, 128, V, dtype, **GATES["slow"])
    off = np.array([0, 128, 320, 321, 640], dtype=np.int32)
    s0 = (np.random.default_rng(9).standard_normal((1, 4, 128, V)) * 0.05).astype(np.float32)
    g, beta = _gpu_gates(d)
    q, k, v = dev(d["q"], dtype)[None], dev(d["k"], dtype)[None], dev(d["v"], dtype)[None]
    o, fin = gdn.gdn_chunk_fwd_segmented(q, k, v, g[None], beta[None], dev(off, "i32"), off,
                                         initial_state=dev(s0[0]), o_dtype=torch.float32)
    torch.cuda.synchronize()
    oref, fref = _oracle_chunk(d, s0)
    check = assert_f32 if dtype == "f32" else assert_bf16
    check(host(o[0]), oref, "o")
    check(host(fin), fref[0], "final")
    one = np.array([0, T], dtype=np.int32)
    o1, f1 = gdn.gdn_chunk_fwd_segmented(q, k, v, g[None], beta[None], dev(one, "i32"), one,
                                         initial_state=dev(s0[0]), o_dtype=torch.float32)
    o2, f2 = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], initial_state=dev(s0), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2[0])


def _many_offsets(T, P, seed):
    """P chunk-unaligned segments of T tokens, a few of them empty."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(0, T + 1, P - 1))
    off = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    off[P // 2] = off[P // 2 - 1]  # at least one empty segment
    return np.maximum.accumulate(off).astype(np.int32)


@pytest.mark.parametrize("dtype,V,P", [("bf16", 128, 17), ("bf16", 128, 18), ("bf16", 128, 64), ("f32", 64, 40)])
def test_segment_state_scan_long_chains(dtype, V, P):
    """Long serial chains of maps (up to 64, with empty and ragged segments): every start and the
    final state against the oracle's chain."""
    T = 1536
    d = gdn_inputs.small(45 + P, [T], 2, 4, 128, V, dtype, **GATES["slow"])
    off = _many_offsets(T, P, P)
    s0 = (np.random.default_rng(10).standard_normal((4, 128, V)) * 0.1).astype(np.float32)
    g, beta = _gpu_gates(d)
    M, b, starts, fin = gdn.gdn_segment_state_scan(dev(d["k"], dtype), dev(d["v"], dtype), g, beta,
                                                   dev(off, "i32"), off, initial_state=dev(s0))
    torch.cuda.synchronize()
    go, bo = _oracle_gates(d)
    Mref, bref = oracle.segment_affine(d["k"], d["v"], go, bo, off, Hqk=2)
    sref, fref = oracle.chain(Mref, bref, s0)
    check = assert_f32 if dtype == "f32" else assert_bf16
    for i in range(P):
        check(host(starts[i]), sref[i], "start[%d]" % i)
    check(host(fin), fref, "final")


@pytest.mark.parametrize("dtype,V,P", [("bf16", 128, 40), ("f32", 32, 33)])
def test_segmented_forward_long_chains(dtype, V, P):
    T = 1600
    d = gdn_inputs.small(46 + P, [T], 2, 4, 128, V, dtype, **GATES["slow"])
    off = _many_offsets(T, P, 100 + P)
    s0 = (np.random.default_rng(11).standard_normal((1, 4, 128, V)) * 0.05).astype(np.float32)
    g, beta = _gpu_gates(d)
    o, fin = gdn.gdn_chunk_fwd_segmented(dev(d["q"], dtype)[None], dev(d["k"], dtype)[None], dev(d["v"], dtype)[None],
                                         g[None], beta[None], dev(off, "i32"), off, initial_state=dev(s0[0]),
                                         o_dtype=torch.float32)
    torch.cuda.synchronize()
    oref, fref = _oracle_chunk(d, s0)
    check = assert_f32 if dtype == "f32" else assert_bf16
    check(host(o[0]), oref, "o")
    check(host(fin), fref[0], "final")


# --------------------------------------------------------------------------- #
# Recurrent decode step (one new token per sequence, state updated in place)
# --------------------------------------------------------------------------- #
def _decode_inputs(seed, N, Hqk, Hv, K, V, dtype):
    """N one-token samples of the usual recipe, plus N fp32 states."""
    d = gdn_inputs.small(seed, [1] * N, Hqk, Hv, K, V, dtype, s0_std=0.5)
    return d, d["s0"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 32), (32, 256)])
def test_decode_step_matches_oracle(dtype, K, V):
    N, Hqk, Hv = 40, 2, 4
    d, s0 = _decode_inputs(41, N, Hqk, Hv, K, V, dtype)
    g, beta = _gpu_gates(d)
    state = dev(s0)
    o = gdn.gdn_decode_step(dev(d["q"], dtype), dev(d["k"], dtype), dev(d["v"], dtype), g, beta, state,
                            scale=0.75, o_dtype=torch.float32)
    torch.cuda.synchronize()
    og, bg = _oracle_gates(d)
    oref, sref = oracle.decode_step(d["q"], d["k"], d["v"], og, bg, s0, scale=0.75)
    check = assert_f32 if dtype == "f32" else assert_bf16
    so = check(host(o), oref, "o")
    ss = check(host(state), sref, "state")
    print("\ndecode %s K=%d V=%d o %s state %s" % (dtype, K, V, so, ss))


def test_decode_step_state_rows_skips_and_bf16_o():
    """Rows picked by index; negative and out-of-range indices skip their sequence (o = 0, no
    state row touched); bf16 o is the fp32 result rounded."""
    N, Hqk, Hv, K, V, R = 6, 1, 2, 128, 128, 10
    d, _ = _decode_inputs(42, N, Hqk, Hv, K, V, "bf16")
    s0 = (np.random.default_rng(43).standard_normal((R, Hv, K, V)) * 0.5).astype(np.float32)
    idx = np.array([7, 2, -1, 9, 0, 15], dtype=np.int32)
    g, beta = _gpu_gates(d)
    state = dev(s0)
    o = gdn.gdn_decode_step(dev(d["q"], "bf16"), dev(d["k"], "bf16"), dev(d["v"], "bf16"), g, beta, state,
                            state_indices=dev(idx, "i32"), o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    og, bg = _oracle_gates(d)
    ref_idx = np.where(idx < R, idx, -1)
    oref, sref = oracle.decode_step(d["q"], d["k"], d["v"], og, bg, s0, state_indices=ref_idx)
    got_o, got_s = host(o), host(state)
    live = ref_idx >= 0
    assert np.all(got_o[~live] == 0)
    untouched = np.setdiff1d(np.arange(R), ref_idx[live])
    np.testing.assert_array_equal(got_s[untouched], s0[untouched].astype(np.float64))
    assert_bf16(got_s[ref_idx[live]], sref[ref_idx[live]], "state")
    rms = np.sqrt(np.mean(oref[live] ** 2))
    assert np.all(np.abs(got_o[live] - oref[live]) <= 2e-2 * rms + 2.0 ** -8 * np.abs(oref[live]))


def test_decode_continues_a_chunk_prefill():
    """gdn_chunk_fwd over packed samples hands its final states to the decode step; one more token
    per sample then matches the oracle recurrence over the longer samples."""
    lengths = [300, 1, 64, 129]
    N, Hqk, Hv, K, V = len(lengths), 2, 4, 128, 128
    full = gdn_inputs.small(44, [n + 1 for n in lengths], Hqk, Hv, K, V, "bf16")
    cu = full["cu_seqlens"]
    last = cu[1:] - 1
    keep = np.setdiff1d(np.arange(cu[-1]), last)
    pre = {key: full[key][keep] for key in ("q", "k", "v", "a", "b")}
    pre.update(A_log=full["A_log"], dt_bias=full["dt_bias"], cu_seqlens=np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    _, fin = _run_chunk(pre, "bf16", o_dtype=torch.float32)
    g, beta = gdn.gdn_gate_fwd(dev(full["a"][last]), dev(full["b"][last]), dev(full["A_log"]), dev(full["dt_bias"]))
    o = gdn.gdn_decode_step(dev(full["q"][last], "bf16"), dev(full["k"][last], "bf16"), dev(full["v"][last], "bf16"),
                            g, beta, fin, o_dtype=torch.float32)
    torch.cuda.synchronize()
    oref, fref = _oracle_chunk(full)
    so = assert_bf16(host(o), oref[last], "o")
    sf = assert_bf16(host(fin), fref, "state")
    print("\ndecode after prefill o %s state %s" % (so, sf))


# --------------------------------------------------------------------------- #
# Output norm gated by z
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("o_dt,z_dt", [("f32", "bf16"), ("bf16", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("V", [32, 128, 256])
def test_gated_norm_matches_oracle(o_dt, z_dt, V):
    rng = np.random.default_rng(61)
    rows = 1003  # not a multiple of any rows-per-workgroup count
    o = (rng.standard_normal((rows, V)) * 0.3).astype(np.float32)
    z = (rng.standard_normal((rows, V)) * 2.0).astype(np.float32)
    w = rng.uniform(0.5, 1.5, V).astype(np.float32)
    if o_dt == "bf16":
        o = oracle.round_bf16(o).astype(np.float32)
    if z_dt == "bf16":
        z = oracle.round_bf16(z).astype(np.float32)
    y = gdn.gdn_gated_rmsnorm_fwd(dev(o, o_dt), dev(z, z_dt), dev(w), eps=1e-5, y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(o, z, w, 1e-5)
    s = assert_f32(host(y), ref, "y")
    print("\ngated norm o %s z %s V=%d %s" % (o_dt, z_dt, V, s))


def test_gated_norm_bf16_in_place_and_without_weight():
    """bf16 y written over o (each row is read before it is written), no weight: the fp32 result rounded."""
    rng = np.random.default_rng(62)
    rows, V = 4099, 128
    o = oracle.round_bf16(rng.standard_normal((rows, V))).astype(np.float32)
    z = oracle.round_bf16(rng.standard_normal((rows, V)) * 2.0).astype(np.float32)
    ot = dev(o, "bf16")
    y = gdn.gdn_gated_rmsnorm_fwd(ot, dev(z, "bf16"), None, eps=1e-6, out=ot)
    torch.cuda.synchronize()
    assert y.data_ptr() == ot.data_ptr()
    ref = oracle.gated_rmsnorm(o, z, None, 1e-6)
    got = host(y)
    assert np.all(np.abs(got - ref) <= 1e-5 + 2.0 ** -8 * np.abs(ref))


def test_gated_norm_after_the_chunk_rule():
    """gdn_chunk_fwd's o (fp32, [T, H_v, V]) through the norm matches the oracle recurrence's o normed."""
    d = gdn_inputs.small(63, [200, 57, 130], 2, 4, 128, 128, "bf16")
    o, _ = _run_chunk(d, "bf16", o_dtype=torch.float32)
    z = (np.random.default_rng(64).standard_normal(o.shape) * 2.0).astype(np.float32)
    z = oracle.round_bf16(z).astype(np.float32)
    w = np.random.default_rng(65).uniform(0.5, 1.5, 128).astype(np.float32)
    y = gdn.gdn_gated_rmsnorm_fwd(o, dev(z, "bf16"), dev(w), eps=1e-6, y_dtype=torch.float32)
    torch.cuda.synchronize()
    oref, _ = _oracle_chunk(d)
    ref = oracle.gated_rmsnorm(oref, z, w, 1e-6)
    s = assert_bf16(host(y), ref, "y")
    print("\nnorm after chunk %s" % (s,))


def _run_chunk_norm(d, dtype, z, w, eps, s0=None, o_dtype=None, use_cu=True):
    q = dev(d["q"], dtype)[None]
    k = dev(d["k"], dtype)[None]
    v = dev(d["v"], dtype)[None]
    g, beta = _gpu_gates(d)
    cu = dev(d["cu_seqlens"], "i32") if use_cu else None
    o, fin = gdn.gdn_chunk_fwd_gated_norm(
        q, k, v, g[None], beta[None], z[None], norm_weight=w, eps=eps,
        initial_state=None if s0 is None else dev(s0), cu_seqlens=cu,
        cu_seqlens_host=d["cu_seqlens"] if use_cu else None, o_dtype=o_dtype,
    )
    torch.cuda.synchronize()
    return o[0], fin


@pytest.mark.parametrize("o_dt,z_dt,weighted", [("f32", "bf16", True), ("bf16", "bf16", False), ("f32", "f32", False)])
def test_chunk_gated_norm_fused(o_dt, z_dt, weighted):
    """bf16 inputs, V = 128: the scan applies the gated norm as it writes o (packed samples that
    the planner splits, start states).  Matches the oracle's recurrence followed by its norm,
    and with fp32 o the unfused pair gdn_chunk_fwd + gdn_gated_rmsnorm_fwd to fp32 rounding."""
    lengths = [2500, 0, 700, 64, 1, 1350]
    d = gdn_inputs.small(66, lengths, 2, 4, 128, 128, "bf16", A_log_range=(-2.0, 0.0))
    s0 = (np.random.default_rng(67).standard_normal((len(lengths), 4, 128, 128)) * 0.05).astype(np.float32)
    z = (np.random.default_rng(68).standard_normal((sum(lengths), 4, 128)) * 2.0).astype(np.float32)
    if z_dt == "bf16":
        z = oracle.round_bf16(z).astype(np.float32)
    w = np.random.default_rng(69).uniform(0.5, 1.5, 128).astype(np.float32) if weighted else None
    o_t = torch.float32 if o_dt == "f32" else torch.bfloat16
    y, fin = _run_chunk_norm(d, "bf16", dev(z, z_dt), None if w is None else dev(w), 1e-6, s0, o_dtype=o_t)
    oref, fref = _oracle_chunk(d, s0)
    ref = oracle.gated_rmsnorm(oref, z, w, 1e-6)
    s = assert_bf16(host(y), ref, "y", bf16_store=o_dt == "bf16")
    assert_bf16(host(fin), fref, "final")
    print("\nfused norm o %s z %s weight %s: %s" % (o_dt, z_dt, weighted, s))
    if o_dt == "f32":
        o2, _ = _run_chunk(d, "bf16", s0, o_dtype=torch.float32)
        y2 = gdn.gdn_gated_rmsnorm_fwd(o2, dev(z, z_dt), None if w is None else dev(w), eps=1e-6)
        torch.cuda.synchronize()
        diff = np.abs(host(y) - host(y2))
        assert diff.max() <= 1e-6 * max(1.0, float(np.abs(host(y2)).max())), float(diff.max())
        print("fused vs unfused: max |diff| %.3g" % diff.max())


def test_chunk_gated_norm_wide_v_and_fp32_paths():
    """Shapes the scan does not fuse run the chunk forward, then the norm kernel over o in place:
    bf16 with V = 256, and the fp32 kernel (K = V = 32)."""
    lengths = [300, 1, 129]
    d = gdn_inputs.small(70, lengths, 2, 4, 128, 256, "bf16")
    z = oracle.round_bf16(np.random.default_rng(71).standard_normal((sum(lengths), 4, 256)) * 2.0)
    z = z.astype(np.float32)
    w = np.random.default_rng(72).uniform(0.5, 1.5, 256).astype(np.float32)
    y, _ = _run_chunk_norm(d, "bf16", dev(z, "bf16"), dev(w), 1e-6, o_dtype=torch.float32)
    oref, _ = _oracle_chunk(d)
    s = assert_bf16(host(y), oracle.gated_rmsnorm(oref, z, w, 1e-6), "y V=256")
    print("\nnorm V=256 %s" % (s,))

    d = gdn_inputs.small(73, [1, 64, 65, 130], 2, 4, 32, 32, "f32")
    z = (np.random.default_rng(74).standard_normal((260, 4, 32)) * 2.0).astype(np.float32)
    y, _ = _run_chunk_norm(d, "f32", dev(z), None, 1e-6)
    oref, _ = _oracle_chunk(d)
    ref = oracle.gated_rmsnorm(oref, z, None, 1e-6)
    # an fp32 error e in o moves the normed row by at most about 2 e / rms(row) times |silu(z)|
    rms = np.sqrt(np.mean(oref * oref, axis=-1, keepdims=True) + 1e-6)
    bound = 2.0 * TOL_F32_ABS / rms * np.abs(z / (1.0 + np.exp(-z.astype(np.float64)))) + 1e-6
    err = np.abs(host(y).astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / bound).max())
    print("norm fp32 path: worst error / bound %.3g" % float((err / bound).max()))


def test_chunk_gated_norm_fused_gqa_three_batched():
    """Fused norm with three v-heads per q/k head, on batched rows (no cu_seqlens) with start
    states: matches the oracle's recurrence per row followed by its norm."""
    lengths = [192, 192]
    d = gdn_inputs.small(77, lengths, 2, 6, 128, 128, "bf16", A_log_range=(-2.0, 0.0))
    s0 = (np.random.default_rng(78).standard_normal((2, 6, 128, 128)) * 0.05).astype(np.float32)
    z = oracle.round_bf16(np.random.default_rng(79).standard_normal((384, 6, 128)) * 2.0).astype(np.float32)
    g, beta = _gpu_gates(d)
    q = dev(d["q"], "bf16").reshape(2, 192, 2, 128)
    k = dev(d["k"], "bf16").reshape(2, 192, 2, 128)
    v = dev(d["v"], "bf16").reshape(2, 192, 6, 128)
    y, fin = gdn.gdn_chunk_fwd_gated_norm(q, k, v, g.reshape(2, 192, 6), beta.reshape(2, 192, 6),
                                          dev(z, "bf16").reshape(2, 192, 6, 128), eps=1e-6,
                                          initial_state=dev(s0), o_dtype=torch.float32)
    torch.cuda.synchronize()
    oref, fref = _oracle_chunk(d, s0)
    ref = oracle.gated_rmsnorm(oref, z, None, 1e-6)
    s = assert_bf16(host(y).reshape(384, 6, 128), ref, "y")
    assert_bf16(host(fin), fref, "final")
    print("\nfused norm gqa 3 batched: %s" % (s,))


def test_chunk_calls_from_two_host_threads():
    """Split packed calls from two host threads on two streams at once (the planner's cache and the
    LDS-limit flag are the library's shared host state) give what the same calls give one at a time,
    bit for bit."""
    import threading

    Hqk, Hv, K, V = 2, 4, 128, 128
    sets = []
    for seed, lengths in ((61, [2000, 64, 130, 7]), (62, [50, 1900, 300])):
        d = gdn_inputs.small(seed, lengths, Hqk, Hv, K, V, "bf16", s0_std=0.05)
        g, beta = _gpu_gates(d)
        sets.append(dict(q=dev(d["q"], "bf16")[None], k=dev(d["k"], "bf16")[None], v=dev(d["v"], "bf16")[None],
                         g=g[None], beta=beta[None], s0=dev(d["s0"]), cu=dev(d["cu_seqlens"], "i32"),
                         cu_host=d["cu_seqlens"]))
    torch.cuda.synchronize()

    def call(t):
        return gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["s0"],
                                 cu_seqlens=t["cu"], cu_seqlens_host=t["cu_host"], o_dtype=torch.float32)

    ref = [call(t) for t in sets]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = [[None] * 8, [None] * 8]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for r in range(8):
                    results[i][r] = call(sets[i])
            streams[i].synchronize()
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for o, fin in results[i]:
            assert torch.equal(o, ref[i][0]) and torch.equal(fin, ref[i][1])
