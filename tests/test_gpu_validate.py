"""GDN_VALIDATE=1: offsets given on the device alone are copied back and checked
like a host mirror before anything is enqueued.

Malformed offsets (decreasing, or not ending at T) must be refused with
GDN_ERR_BAD_SEQLENS and leave the outputs untouched; well-formed ones must give
the same results as without the check.  Without the variable, device-only
offsets are not read on the host (the kernels clamp them), which the canary
test covers.  Packed samples never see each other (LlamaFactory PR "[v1]
support GDN Ulysses cp", Design decisions 5-6), so a malformed array is an
argument error, not a layout.
"""

import os

import numpy as np
import pytest

import gdn_inputs
from parity_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402

BAD_SEQLENS = 5


@pytest.fixture
def validate():
    old = os.environ.get("GDN_VALIDATE")
    os.environ["GDN_VALIDATE"] = "1"
    yield
    os.environ.pop("GDN_VALIDATE", None)
    if old is not None:
        os.environ["GDN_VALIDATE"] = old


def _bad_offsets(cu):
    dec = cu.copy()
    dec[2] = dec[1] - 1  # decreasing
    short = cu.copy()
    short[-1] -= 1  # does not end at T
    return [dec, short]


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f32", 64)])
def test_chunk_fwd_refuses_bad_device_offsets(validate, dtype, K):
    lengths = [70, 130, 60]
    d = gdn_inputs.small(31, lengths, 2, 4, K, K, dtype)
    q, k, v = (dev(d[n], dtype)[None] for n in ("q", "k", "v"))
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    cu = d["cu_seqlens"]
    ref_o, ref_f = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], cu_seqlens=dev(cu, "i32"),
                                     o_dtype=torch.float32)
    torch.cuda.synchronize()
    for bad in _bad_offsets(cu):
        with pytest.raises(gdn.GdnError) as exc:
            gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], cu_seqlens=dev(bad, "i32"), o_dtype=torch.float32)
        assert exc.value.status == BAD_SEQLENS
    os.environ.pop("GDN_VALIDATE")
    o2, f2 = gdn.gdn_chunk_fwd(q, k, v, g[None], beta[None], cu_seqlens=dev(cu, "i32"), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref_o) and torch.equal(f2, ref_f)


def test_conv_and_fused_refuse_bad_device_offsets(validate):
    lengths = [70, 130, 60]
    Hqk, Hv, K, V = 2, 4, 128, 128
    d = gdn_inputs.small(32, lengths, Hqk, Hv, K, V, "bf16", conv_width=4)
    T, C = d["x"].shape
    x = dev(d["x"], "bf16")
    lib = gdn.load_library()
    for bad in _bad_offsets(d["cu_seqlens"]):
        y = torch.full((T, C), 7.0, dtype=torch.bfloat16, device="cuda:0")
        st = lib.gdn_conv1d_fwd(x.data_ptr(), dev(d["conv_w"], "bf16").data_ptr(), None, gdn.BF16,
                                dev(bad, "i32").data_ptr(), None, len(bad) - 1, 1, T, C, 4, 1, 2 * Hqk * K, K, 1e-6,
                                0, y.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == BAD_SEQLENS, lib.gdn_status_string(st)
        assert bool((y == 7.0).all())
        with pytest.raises(gdn.GdnError) as exc:
            gdn.gdn_conv_chunk_fwd(x[None], dev(d["conv_w"], "bf16"), dev(d["a"])[None], dev(d["b"])[None],
                                   dev(d["A_log"]), dev(d["dt_bias"]), Hqk=Hqk, K=K,
                                   cu_seqlens=dev(bad, "i32"))
        assert exc.value.status == BAD_SEQLENS


def test_segment_entry_points_refuse_bad_device_offsets(validate):
    T, Hqk, Hv, K, V = 300, 2, 4, 128, 128
    d = gdn_inputs.small(33, [T], Hqk, Hv, K, V, "bf16")
    k, v = dev(d["k"], "bf16"), dev(d["v"], "bf16")
    q = dev(d["q"], "bf16")
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    bad = np.array([0, 128, 64, T], dtype=np.int32)  # decreasing
    with pytest.raises(gdn.GdnError) as exc:
        gdn.gdn_segment_state_scan(k, v, g, beta, dev(bad, "i32"))
    assert exc.value.status == BAD_SEQLENS
    with pytest.raises(gdn.GdnError) as exc:
        gdn.gdn_chunk_fwd_segmented(q[None], k[None], v[None], g[None], beta[None], dev(bad, "i32"))
    assert exc.value.status == BAD_SEQLENS
    good = np.array([0, 64, 200, T], dtype=np.int32)
    o, f = gdn.gdn_chunk_fwd_segmented(q[None], k[None], v[None], g[None], beta[None], dev(good, "i32"), good)
    o2, f2 = gdn.gdn_chunk_fwd_segmented(q[None], k[None], v[None], g[None], beta[None], dev(good, "i32"))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(f, f2)
