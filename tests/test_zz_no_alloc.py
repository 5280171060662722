"""gdn_chunk_fwd_noalloc -- the chunk forward whose per-chunk records sit in the
library's fixed device array -- against gdn_chunk_fwd, through the C ABI.

Both calls run the same kernels: without host offsets gdn_chunk_fwd takes the
unsplit path, the only one the no-allocation variant has, so the two agree bit
for bit.  Against the default (segment-split) gdn_chunk_fwd they agree within
the bf16 tolerance, and the small call is also held to the oracle.  Two calls
in a row, the second smaller, show that whatever the array keeps from the last
call does not leak into the next.
"""

import numpy as np
import pytest

import gdn_inputs
import oracle
from parity_util import assert_bf16, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402

HQK, HV, K, V = 16, 32, 128, 128


def _inputs(seed, lengths, s0_std):
    d = gdn_inputs.small(seed, lengths, HQK, HV, K, V, "bf16", s0_std=s0_std)
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    t = dict(q=dev(d["q"], "bf16")[None], k=dev(d["k"], "bf16")[None], v=dev(d["v"], "bf16")[None],
             g=g[None], beta=beta[None], cu=dev(d["cu_seqlens"], "i32"), cu_host=d["cu_seqlens"],
             s0=dev(d["s0"]) if "s0" in d else None)
    return d, t


def _call_pair(t, o_dtype):
    kw = dict(scale=K ** -0.5, initial_state=t["s0"], cu_seqlens=t["cu"], o_dtype=o_dtype)
    o_n, f_n = gdn.gdn_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens_host=t["cu_host"],
                                         **kw)
    o_p, f_p = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens_host=None, **kw)
    o_s, f_s = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens_host=t["cu_host"], **kw)
    torch.cuda.synchronize()
    return (o_n, f_n), (o_p, f_p), (o_s, f_s)


@pytest.mark.parametrize("o_dtype", ["f32", "bf16"])
def test_noalloc_matches_chunk_fwd_two_calls(o_dtype):
    od = torch.float32 if o_dtype == "f32" else torch.bfloat16
    # first call: the packed 8-sample workload at full size (8192 tokens, H_v = 32)
    rng = np.random.default_rng(2024)
    big = gdn_inputs.dirichlet_lengths(rng, 8192, 8, 64)
    # second call: fewer tokens and samples, other values, a zero-length and a one-token sample
    small = [700, 0, 64, 1, 333]
    for call, (seed, lengths, s0_std) in enumerate([(31, big, 0.0), (32, small, 0.02)]):
        print("noalloc call %d: lengths %s o=%s" % (call, lengths, o_dtype), flush=True)
        d, t = _inputs(seed, lengths, s0_std)
        (o_n, f_n), (o_p, f_p), (o_s, f_s) = _call_pair(t, od)
        assert torch.equal(o_n, o_p) and torch.equal(f_n, f_p), "call %d differs from the unsplit gdn_chunk_fwd" % call
        ref_o, ref_f = host(o_s)[0], host(f_s)
        assert_bf16(host(o_n)[0], ref_o, "o vs split call %d" % call, bf16_store=(o_dtype == "bf16"))
        assert_bf16(host(f_n), ref_f, "final state vs split call %d" % call)
        if call == 1:
            g64, b64 = oracle.gates(d["a"], d["b"], d["A_log"], d["dt_bias"])
            oo, of = oracle.recurrence(d["q"], d["k"], d["v"], g64, b64, d["s0"], d["cu_seqlens"], scale=K ** -0.5)
            assert_bf16(host(o_n)[0], oo, "o vs oracle", bf16_store=(o_dtype == "bf16"))
            assert_bf16(host(f_n), of, "final state vs oracle")


def test_noalloc_rejects_inputs_beyond_the_array():
    # 3 x 8192 tokens in 8 samples at H_v = 32 need 392 chunk slots of records; the array holds 199
    T = 3 * 8192
    lengths = [T // 8] * 8
    q = torch.zeros((1, T, HQK, K), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, T, HV, V), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, T, HV), dtype=torch.float32, device="cuda")
    cu_host = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    o = torch.full((1, T, HV, V), 7.0, dtype=torch.float32, device="cuda")
    fin = torch.full((8, HV, K, V), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd_noalloc(q, q, v, g, g, cu_seqlens=dev(cu_host, "i32"), cu_seqlens_host=cu_host, o=o,
                                  final_state=fin)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((fin == 7.0).all())


def test_noalloc_fp32_inputs_need_no_array():
    d = gdn_inputs.small(33, [130, 64, 1], 2, 4, 32, 64, "f32")
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    args = (dev(d["q"])[None], dev(d["k"])[None], dev(d["v"])[None], g[None], beta[None])
    cu = dev(d["cu_seqlens"], "i32")
    o_n, f_n = gdn.gdn_chunk_fwd_noalloc(*args, cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens"])
    o_p, f_p = gdn.gdn_chunk_fwd(*args, cu_seqlens=cu, cu_seqlens_host=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_p) and torch.equal(f_n, f_p)
