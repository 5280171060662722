"""Packed calls with more samples than a wavefront has lanes.

Up to 64 samples, the chunk prep finds a chunk slot's sample with one wave-wide
ballot over the offsets and the conv finds a run's first sample the same way;
beyond that both switch to a binary search.  These cases hold 100-166 samples
(empty, one-token and partial-chunk ones among them) and check the results
against the oracle: the chunk call (MFMA and vector-ALU kernels), a split run
(one long sample beside many short ones, which the planner cuts), the conv in
both rounding modes, and the fused conv + chunk call against the unfused pair.
Samples never see each other (LlamaFactory PR "[v1] support GDN Ulysses cp",
Design decisions 5-6).
"""

import numpy as np
import pytest

import gdn_inputs
import oracle
from parity_util import assert_f32, assert_units_bf16, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402

# one long sample among many short ones: the planner splits it (shown on the CPU by
# tests/test_split_plan_cpu.py for these lengths at H_v = 4, V = 128 on 256 compute units)
SPLIT_LENGTHS = [1] * 150 + [0] * 5 + [4000] + [37] * 10


def _random_lengths(n, seed):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(0, 100, n)
    lengths[::17] = 0
    lengths[5::23] = 1
    return [int(x) for x in lengths]


def _chunk(d, dtype, s0):
    q, k, v = (dev(d[n], dtype)[None] for n in ("q", "k", "v"))
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    cu = d["cu_seqlens"]
    o, fin = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], initial_state=dev(s0), cu_seqlens=dev(cu, "i32"),
                               cu_seqlens_host=cu, o_dtype=torch.float32)
    torch.cuda.synchronize()
    return host(o[0]), host(fin)


def _oracle(d, s0):
    g, beta = oracle.gates(d["a"], d["b"], d["A_log"], d["dt_bias"])
    return oracle.recurrence(d["q"], d["k"], d["v"], g, beta, s0, d["cu_seqlens"], threads=oracle.max_threads())


@pytest.mark.parametrize("case", ["bf16_random", "bf16_split", "f32_random"])
def test_chunk_fwd_many_samples(case):
    if case == "f32_random":
        dtype, K, V, lengths = "f32", 64, 64, _random_lengths(120, 1)
    else:
        dtype, K, V = "bf16", 128, 128
        lengths = _random_lengths(120, 2) if case == "bf16_random" else SPLIT_LENGTHS
    d = gdn_inputs.small(60 + len(lengths), lengths, 2, 4, K, V, dtype, s0_std=0.05)
    o, fin = _chunk(d, dtype, d["s0"])
    oref, fref = _oracle(d, d["s0"])
    cu = d["cu_seqlens"]
    if dtype == "f32":
        assert_f32(o, oref, "o")
        assert_f32(fin, fref, "final state")
    else:
        assert_units_bf16(o, oref, cu, case, fin=fin, fref=fref)
    # empty samples keep their start state bit for bit
    for n in np.flatnonzero(np.diff(cu) == 0):
        assert np.array_equal(fin[n], d["s0"][n]), "empty sample %d" % n


def test_conv_many_samples_both_roundings():
    Hqk, Hv, K, V = 2, 4, 128, 128
    lengths = _random_lengths(100, 3)
    d = gdn_inputs.small(70, lengths, Hqk, Hv, K, V, "bf16", conv_width=4)
    cu = d["cu_seqlens"]
    T = int(cu[-1])
    l2ch = 2 * Hqk * K
    ref = oracle.conv1d(d["x"], d["conv_w"], d["conv_bias"], cu)
    ref[:, :l2ch] = oracle.l2norm(ref[:, :l2ch].reshape(T, -1, K)).reshape(T, -1)
    args = (dev(d["x"], "bf16"), dev(d["conv_w"], "bf16"), dev(d["conv_bias"], "bf16"))
    kw = dict(cu_seqlens=dev(cu, "i32"), cu_seqlens_host=cu, l2norm_channels=l2ch, head_dim=K)
    got = host(gdn.gdn_conv1d_fwd(*args, **kw))
    excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-5)
    assert excess.max() <= 0, float(excess.max())
    got = host(gdn.gdn_conv1d_fwd(*args, exact_rounding=True, **kw))
    assert np.array_equal(got, oracle.round_bf16(ref))


@pytest.mark.parametrize("lengths", [_random_lengths(100, 4), SPLIT_LENGTHS], ids=["random", "split"])
def test_conv_chunk_many_samples_equals_unfused(lengths):
    Hqk, Hv, K, V = 2, 4, 128, 128
    d = gdn_inputs.small(80 + len(lengths), lengths, Hqk, Hv, K, V, "bf16", conv_width=4, s0_std=0.05)
    cu = d["cu_seqlens"]
    T, C = d["x"].shape
    x, w, bias = dev(d["x"], "bf16"), dev(d["conv_w"], "bf16"), dev(d["conv_bias"], "bf16")
    a, b, A_log, dt_bias = dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"])
    s0, cu_d = dev(d["s0"]), dev(cu, "i32")
    o1, f1 = gdn.gdn_conv_chunk_fwd(x[None], w, a[None], b[None], A_log, dt_bias, Hqk=Hqk, K=K, bias=bias,
                                    initial_state=s0, cu_seqlens=cu_d, cu_seqlens_host=cu, o_dtype=torch.float32)
    y = gdn.gdn_conv1d_fwd(x, w, bias, cu_seqlens=cu_d, cu_seqlens_host=cu, l2norm_channels=2 * Hqk * K,
                           head_dim=K)[None]
    g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
    q = y[..., : Hqk * K].unflatten(-1, (Hqk, K))
    k = y[..., Hqk * K : 2 * Hqk * K].unflatten(-1, (Hqk, K))
    v = y[..., 2 * Hqk * K :].unflatten(-1, (Hv, V))
    o2, f2 = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], initial_state=s0, cu_seqlens=cu_d,
                               cu_seqlens_host=cu, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
