"""conv1d + SiLU + q/k L2 norm fused into the chunk kernels (gdn_conv_chunk_fwd)
against the oracle's pipeline: conv1d, SiLU, the per-head L2 norm of q and k,
and the token recurrence, in fp64.

- Vector-ALU shapes (fp32 inputs, or head sizes the MFMA kernels do not take):
  the kernel keeps the activations in fp32 and never stores them, so the
  oracle leaves them unrounded, and outputs and final states are held to the
  fp32 bound (1e-4 absolute), bf16-stored o additionally to its own rounding
  (2^-8 relative).
- MFMA shapes (bf16, K = 128, V a multiple of 128, at most four v-heads per
  q/k head): the chunk prep forms the activations and stores them in bf16
  exactly as the separate conv's fast rounding does (the fp32 evaluation
  rounded once), so o and the final states must equal the unfused pair
  (gdn_conv1d_fwd, then gdn_chunk_fwd on its output) bit for bit.  Against the
  oracle, that rounding can land one bf16 unit away from the oracle's rounding
  of the exact activation, and one such v value moves o at its token by up to
  a few percent of RMS(o); so the oracle bound is checked on the same case
  through the unfused pipeline with the conv's exact rounding, whose
  activations are the oracle's bit for bit, while the fast conv itself is
  held to 2^-8 |y| + 1e-5 per output (tests/test_gpu_workloads.py).

The layer runs the short convolution over the concatenated q | k | v
channels and feeds the chunk rule on the same token-major layout
(LlamaFactory PR "[v1] support GDN Ulysses cp", Design).
"""

import numpy as np
import pytest

import gdn_inputs
import oracle
from parity_util import TOL_F32_ABS, assert_bf16, assert_f32, assert_units_bf16, dev, host, stats

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402


def _mfma(dtype, Hqk, Hv, K, V):
    return dtype == "bf16" and K == 128 and V % 128 == 0 and Hv // Hqk <= 4


def _oracle(d, Hqk, Hv, K, V, scale=1.0, s0=None, threads=0, act_round="none"):
    q, k, v = oracle.pipeline_activations(d["x"], d["conv_w"], d.get("conv_bias"), d["cu_seqlens"], Hqk, Hv, K, V,
                                          act_round=act_round, threads=threads)
    g, beta = oracle.gates(d["a"], d["b"], d["A_log"], d["dt_bias"])
    return oracle.recurrence(q, k, v, g, beta, s0, d["cu_seqlens"], scale=scale, threads=threads)


def _fused(d, dtype, Hqk, K, B=1, packed=True, bias=True, scale=1.0, s0=None, o_dtype=None):
    """The fused call on the raw conv input and the raw gate inputs."""
    T, C = d["x"].shape
    Hv = d["a"].shape[-1]
    x = dev(d["x"], dtype).reshape(B, T // B, C)
    o, fin = gdn.gdn_conv_chunk_fwd(
        x, dev(d["conv_w"], dtype), dev(d["a"]).reshape(B, T // B, Hv), dev(d["b"]).reshape(B, T // B, Hv),
        dev(d["A_log"]), dev(d["dt_bias"]), Hqk=Hqk, K=K,
        bias=dev(d["conv_bias"], dtype) if bias else None, scale=scale, initial_state=None if s0 is None else dev(s0),
        cu_seqlens=dev(d["cu_seqlens"], "i32") if packed else None,
        cu_seqlens_host=d["cu_seqlens"] if packed else None, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o.reshape(T, Hv, -1), fin


def _assert_o(got, ref, bf16_store, what):
    if not bf16_store:
        return assert_f32(got, ref, what)
    s = stats(got, ref)
    excess = np.abs(got - ref) - (TOL_F32_ABS + 2.0 ** -8 * np.abs(ref))
    assert s["nonfinite"] == 0 and excess.max() <= 0, (what, s, float(excess.max()))
    return s


LENGTHS = [1, 63, 64, 2, 170, 0, 33, 129]

CASES = [
    # dtype, Hqk, Hv, K, V, width, bias, s0, o_dtype
    ("f32", 1, 2, 32, 32, 4, True, False, "f32"),
    ("bf16", 2, 4, 64, 64, 3, False, True, "f32"),
    ("bf16", 2, 4, 128, 128, 4, True, True, "bf16"),
    ("bf16", 2, 6, 128, 128, 2, True, True, "f32"),
    ("bf16", 1, 1, 128, 256, 4, False, False, "f32"),
    ("f32", 1, 3, 128, 32, 2, True, True, "f32"),
    ("bf16", 2, 2, 64, 96, 1, True, False, "f32"),
    ("bf16", 1, 2, 32, 256, 4, True, False, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_Hqk%d_Hv%d_K%d_V%d_W%d" % c[:6])
def test_conv_chunk_packed_matches_oracle(case):
    dtype, Hqk, Hv, K, V, W, bias, with_s0, o_dt = case
    d = gdn_inputs.small(41 + K + V + W, LENGTHS, Hqk, Hv, K, V, dtype, conv_width=W,
                         s0_std=0.05 if with_s0 else 0.0)
    if not bias:
        d.pop("conv_bias")
    scale = K ** -0.5
    print("conv_chunk packed %s" % (case,), flush=True)
    o, fin = _fused(d, dtype, Hqk, K, bias=bias, scale=scale, s0=d.get("s0"),
                    o_dtype=torch.bfloat16 if o_dt == "bf16" else torch.float32)
    if _mfma(dtype, Hqk, Hv, K, V):
        od = torch.bfloat16 if o_dt == "bf16" else torch.float32
        o2, f2 = _unfused(d, Hqk, K, bias=bias, s0=d.get("s0"), o_dtype=od, scale=scale)
        assert torch.equal(o, o2) and torch.equal(fin, f2)
        o3, f3 = _unfused(d, Hqk, K, bias=bias, s0=d.get("s0"), o_dtype=od, scale=scale, exact=True)
        oref, fref = _oracle(d, Hqk, Hv, K, V, scale=scale, s0=d.get("s0"), act_round="bf16")
        assert_bf16(host(o3), oref, "o (exact conv)", bf16_store=o_dt == "bf16")
        assert_bf16(host(f3), fref, "final (exact conv)")
    else:
        oref, fref = _oracle(d, Hqk, Hv, K, V, scale=scale, s0=d.get("s0"))
        _assert_o(host(o), oref, o_dt == "bf16", "o")
        assert_f32(host(fin), fref, "final")
    # zero-length samples hand the start state (or zero) straight through
    N = len(LENGTHS)
    start = d["s0"] if with_s0 else np.zeros((N, Hv, K, V))
    for n, L in enumerate(LENGTHS):
        if L == 0:
            np.testing.assert_array_equal(host(fin)[n], start[n])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_chunk_batched_rows(dtype):
    """B rows of equal length without offsets: each row starts with zero conv history."""
    B, L, Hqk, Hv, K, V = 3, 150, 2, 4, 64, 64
    d = gdn_inputs.small(77, [L] * B, Hqk, Hv, K, V, dtype, conv_width=4)
    o, fin = _fused(d, dtype, Hqk, K, B=B, packed=False, o_dtype=torch.float32)
    oref, fref = _oracle(d, Hqk, Hv, K, V)
    assert_f32(host(o), oref, "o")
    assert_f32(host(fin), fref, "final")


def test_conv_chunk_agrees_with_the_separate_fp32_pipeline():
    """fp32 inputs: the separate conv stores fp32 activations, so the unfused
    pipeline (gdn_conv1d_fwd, then gdn_chunk_fwd on strided views) computes the
    same values in another order; both stay within the fp32 bound of the oracle
    and within 1e-5 of each other."""
    Hqk, Hv, K, V = 2, 4, 128, 64
    d = gdn_inputs.small(5, LENGTHS, Hqk, Hv, K, V, "f32", conv_width=4)
    T, C = d["x"].shape
    cu = dev(d["cu_seqlens"], "i32")
    y = gdn.gdn_conv1d_fwd(dev(d["x"]), dev(d["conv_w"]), dev(d["conv_bias"]), cu_seqlens=cu,
                           cu_seqlens_host=d["cu_seqlens"], l2norm_channels=2 * Hqk * K, head_dim=K)
    y = y.reshape(1, T, C)
    q = y[..., : Hqk * K].unflatten(-1, (Hqk, K))
    k = y[..., Hqk * K : 2 * Hqk * K].unflatten(-1, (Hqk, K))
    v = y[..., 2 * Hqk * K :].unflatten(-1, (Hv, V))
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    o1, f1 = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens"])
    o2, f2 = _fused(d, "f32", Hqk, K, o_dtype=torch.float32)
    oref, fref = _oracle(d, Hqk, Hv, K, V)
    assert_f32(host(o1[0]), oref, "unfused o")
    assert_f32(host(o2), oref, "fused o")
    np.testing.assert_allclose(host(o2), host(o1[0]), rtol=0, atol=1e-5)
    np.testing.assert_allclose(host(f2), host(f1), rtol=0, atol=1e-5)


@pytest.mark.parametrize("name", ["packed_varlen_bf16_T8192_N8_Hv32_K128", "batched_prefill_bf16_B8_T4096_Hv32_K128"])
def test_conv_chunk_full_workload(name):
    """The whole layer input of the packed and the batched workload through the
    fused call (MFMA path, the packed one split): bit for bit the unfused fast
    pipeline, and the same input through the exact pipeline within the bound
    of every (sequence, head) unit."""
    w = gdn_inputs.WORKLOADS[name]
    d = gdn_inputs.draw(w, with_qkv=False)
    print("conv_chunk full %s" % name, flush=True)
    B = w.batch_rows
    o, fin = _fused(d, "bf16", w.Hqk, w.K, B=B, packed=B == 1, s0=d.get("s0"), o_dtype=torch.float32)
    o2, f2 = _unfused(d, w.Hqk, w.K, B=B, packed=B == 1, s0=d.get("s0"), scale=1.0)
    assert torch.equal(o, o2) and torch.equal(fin, f2)
    # the unfused pipeline with exactly rounded activations against the oracle: every unit
    o3, f3 = _unfused(d, w.Hqk, w.K, B=B, packed=B == 1, s0=d.get("s0"), scale=1.0, exact=True)
    oref, fref = _oracle(d, w.Hqk, w.Hv, w.K, w.V, s0=d.get("s0"), threads=oracle.max_threads(), act_round="bf16")
    worst = assert_units_bf16(host(o3), oref, d["cu_seqlens"], name, fin=host(f3), fref=fref)
    print("%s: fused = unfused bit for bit; exact pipeline worst unit %.2e of its RMS" % (name, worst))


def _unfused(d, Hqk, K, B=1, packed=True, bias=True, s0=None, o_dtype=torch.float32, scale=None, exact=False):
    """gdn_conv1d_fwd (fast rounding unless exact), then gdn_chunk_fwd on views of its output."""
    T, C = d["x"].shape
    cu = dev(d["cu_seqlens"], "i32") if packed else None
    cuh = d["cu_seqlens"] if packed else None
    x = dev(d["x"], "bf16").reshape(B, T // B, C)
    y = gdn.gdn_conv1d_fwd(x, dev(d["conv_w"], "bf16"), dev(d["conv_bias"], "bf16") if bias else None,
                           cu_seqlens=cu, cu_seqlens_host=cuh, l2norm_channels=2 * Hqk * K, head_dim=K,
                           exact_rounding=exact)
    y = y.reshape(B, T // B, C)
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    Hv = g.shape[-1]
    V = (C - 2 * Hqk * K) // Hv
    q = y[..., : Hqk * K].unflatten(-1, (Hqk, K))
    k = y[..., Hqk * K : 2 * Hqk * K].unflatten(-1, (Hqk, K))
    v = y[..., 2 * Hqk * K :].unflatten(-1, (Hv, V))
    o, fin = gdn.gdn_chunk_fwd(q, k, v, g.reshape(B, T // B, Hv), beta.reshape(B, T // B, Hv),
                               scale=K ** -0.5 if scale is None else scale,
                               initial_state=None if s0 is None else dev(s0), cu_seqlens=cu, cu_seqlens_host=cuh,
                               o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o.reshape(T, Hv, -1), fin


@pytest.mark.parametrize("lengths,W,bias,Hv", [
    ([2500, 0, 700, 64, 1, 1350], 4, True, 4),  # long samples: the planner splits them
    (LENGTHS, 3, False, 4),
    ([300, 5, 1000], 1, True, 6),
    ([700, 64, 1, 190], 4, True, 8),  # four v-heads per q/k head: the widest prep workgroup
])
def test_conv_chunk_mfma_equals_unfused_bitwise(lengths, W, bias, Hv):
    """The conv in the chunk prep computes every activation as the separate conv does, so the fused
    call equals the unfused pair bit for bit: packed with host offsets (split and unsplit runs),
    with start states, and without bias."""
    Hqk, K, V = 2, 128, 128
    d = gdn_inputs.small(91 + W + len(lengths), lengths, Hqk, Hv, K, V, "bf16", conv_width=W, s0_std=0.05)
    print("conv_chunk mfma bitwise %s W=%d bias=%s Hv=%d" % (lengths, W, bias, Hv), flush=True)
    o1, f1 = _fused(d, "bf16", Hqk, K, bias=bias, scale=K ** -0.5, s0=d["s0"], o_dtype=torch.float32)
    o2, f2 = _unfused(d, Hqk, K, bias=bias, s0=d["s0"])
    assert torch.equal(o1, o2)
    assert torch.equal(f1, f2)


def test_conv_chunk_mfma_batched_equals_unfused_bitwise():
    """B rows without offsets (each row starts with zero conv history), bf16 o."""
    B, L, Hqk, Hv, K, V = 3, 200, 2, 4, 128, 128
    d = gdn_inputs.small(97, [L] * B, Hqk, Hv, K, V, "bf16", conv_width=4)
    o1, f1 = _fused(d, "bf16", Hqk, K, B=B, packed=False, scale=K ** -0.5, o_dtype=torch.bfloat16)
    o2, f2 = _unfused(d, Hqk, K, B=B, packed=False, o_dtype=torch.bfloat16)
    assert torch.equal(o1, o2)
    assert torch.equal(f1, f2)
