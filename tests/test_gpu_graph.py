"""The layer step (gates, conv1d + SiLU + L2 norm, chunk rule) captured into a HIP
graph and replayed: every replay, with eager work and synchronisations between
the replays, must equal the eager step bit for bit.  The split path of packed
calls hands its plan to the device inside kernel arguments and the library
enqueues no memset or copy, so the captured launches are the eager ones.
"""

import numpy as np
import pytest

import gdn_inputs
from parity_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402


def _step_fn(d, w, out):
    T, C = d["x"].shape
    Hqk, Hv, K, V = w.Hqk, w.Hv, w.K, w.V
    x, cw, cb = dev(d["x"], "bf16"), dev(d["conv_w"], "bf16"), dev(d["conv_bias"], "bf16")
    a, b = dev(d["a"])[None], dev(d["b"])[None]
    A_log, dt_bias = dev(d["A_log"]), dev(d["dt_bias"])
    cu = dev(d["cu_seqlens"], "i32")
    s0 = dev(d["s0"]) if "s0" in d else None

    def step():
        y = gdn.gdn_conv1d_fwd(x, cw, cb, cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens"],
                               l2norm_channels=2 * Hqk * K, head_dim=K).reshape(1, T, C)
        q = y[..., : Hqk * K].unflatten(-1, (Hqk, K))
        k = y[..., Hqk * K : 2 * Hqk * K].unflatten(-1, (Hqk, K))
        v = y[..., 2 * Hqk * K :].unflatten(-1, (Hv, V))
        g, beta = gdn.gdn_gate_fwd(a, b, A_log, dt_bias)
        o, fin = gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu,
                                   cu_seqlens_host=d["cu_seqlens"], o_dtype=torch.float32)
        out["o"], out["fin"] = o, fin

    return step


@pytest.mark.parametrize("lengths", [[3000, 64, 1, 900, 0, 2131], [700, 700]])
def test_step_graph_replays_equal_the_eager_step(lengths):
    """Long samples take the segment-split path (several kernels, plan in kernel arguments);
    balanced ones the plain path."""
    w = gdn_inputs.Workload("graph_step", 71, sum(lengths), len(lengths), 4, 8, 128, 128, "bf16", conv_width=4,
                            s0_std=0.05, lengths=lengths)
    d = gdn_inputs.draw(w, with_qkv=False)
    eager = {}
    step = _step_fn(d, w, eager)
    step()
    torch.cuda.synchronize()
    o_ref, fin_ref = eager["o"].clone(), eager["fin"].clone()

    captured = {}
    gstep = _step_fn(d, w, captured)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gstep()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gstep()
    for rep in range(4):
        captured["o"].zero_()
        captured["fin"].zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(captured["o"], o_ref), rep
        assert torch.equal(captured["fin"], fin_ref), rep
        step()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(eager["o"], o_ref) and torch.equal(eager["fin"], fin_ref)


def _replays_equal_eager(make_step):
    """make_step(out) -> a function that runs the calls and stores their results in out."""
    eager = {}
    step = make_step(eager)
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items()}
    captured = {}
    gstep = make_step(captured)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gstep()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gstep()
    for rep in range(3):
        for t in captured.values():
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(captured[k], ref[k]), (k, rep)
        step()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(eager[k], ref[k]), (k, rep)


def test_fused_conv_chunk_graph_replays_equal_eager():
    """gdn_conv_chunk_fwd on the MFMA path with a split (the plan and the gates formed in the prep)."""
    lengths = [3000, 64, 1, 900, 0, 2131]
    w = gdn_inputs.Workload("graph_fused", 72, sum(lengths), len(lengths), 4, 8, 128, 128, "bf16", conv_width=4,
                            s0_std=0.05, lengths=lengths)
    d = gdn_inputs.draw(w, with_qkv=False)
    x, cw, cb = dev(d["x"], "bf16")[None], dev(d["conv_w"], "bf16"), dev(d["conv_bias"], "bf16")
    a, b, A_log, dt_bias = dev(d["a"])[None], dev(d["b"])[None], dev(d["A_log"]), dev(d["dt_bias"])
    cu, s0 = dev(d["cu_seqlens"], "i32"), dev(d["s0"])

    def make_step(out):
        def step():
            out["o"], out["fin"] = gdn.gdn_conv_chunk_fwd(x, cw, a, b, A_log, dt_bias, Hqk=w.Hqk, K=w.K, bias=cb,
                                                          initial_state=s0, cu_seqlens=cu,
                                                          cu_seqlens_host=d["cu_seqlens"], o_dtype=torch.float32)
        return step

    _replays_equal_eager(make_step)


def test_segmented_forward_graph_replays_equal_eager():
    """gdn_chunk_fwd_segmented (maps in the prep's kernel arguments, mixed pass 1, chain, pass 2)."""
    T = 2000
    d = gdn_inputs.small(73, [T], 2, 4, 128, 128, "bf16", s0_std=0.05)
    q, k, v = (dev(d[n], "bf16")[None] for n in ("q", "k", "v"))
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    off = np.array([0, 300, 301, 1000, 1000, 1700, T], dtype=np.int32)
    off_d, s0 = dev(off, "i32"), dev(d["s0"][0])

    def make_step(out):
        def step():
            out["o"], out["fin"] = gdn.gdn_chunk_fwd_segmented(q, k, v, g[None], beta[None], off_d, off,
                                                               initial_state=s0, o_dtype=torch.float32)
        return step

    _replays_equal_eager(make_step)
