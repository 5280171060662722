"""Calls from several host threads at once, each on its own stream.

The library's host state is the cache of split plans (behind a mutex), the
per-device flag that raises the scan's LDS limit and the per-device compute-unit
count.  Four threads run split packed calls over ten different offset sets
(more than the cache holds, so entries are evicted while other threads look
them up), and every result must equal the same call made alone, bit for bit:
the kernels are deterministic and a plan depends only on the offsets and sizes.
"""

import threading

import numpy as np
import pytest

import gdn_inputs
from parity_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only machines skip via -m "not gpu"
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_deltanet_linear_chunk_amd as gdn  # noqa: E402

N_SETS, N_THREADS, ROUNDS = 10, 4, 3


def _case(i):
    rng = np.random.default_rng(500 + i)
    lengths = [int(x) for x in rng.integers(0, 200, 5)] + [1500 + 64 * i]  # one long sample: split
    d = gdn_inputs.small(600 + i, lengths, 2, 4, 128, 128, "bf16", s0_std=0.05)
    g, beta = gdn.gdn_gate_fwd(dev(d["a"]), dev(d["b"]), dev(d["A_log"]), dev(d["dt_bias"]))
    return dict(q=dev(d["q"], "bf16")[None], k=dev(d["k"], "bf16")[None], v=dev(d["v"], "bf16")[None],
                g=g[None], beta=beta[None], s0=dev(d["s0"]), cu=dev(d["cu_seqlens"], "i32"), cu_np=d["cu_seqlens"])


def _call(c):
    return gdn.gdn_chunk_fwd(c["q"], c["k"], c["v"], c["g"], c["beta"], initial_state=c["s0"], cu_seqlens=c["cu"],
                             cu_seqlens_host=c["cu_np"], o_dtype=torch.float32)


def test_concurrent_calls_from_threads_match_sequential():
    cases = [_case(i) for i in range(N_SETS)]
    ref = [_call(c) for c in cases]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                stream.wait_stream(torch.cuda.default_stream())  # inputs were made on the default stream
                for r in range(ROUNDS):
                    for j in range(N_SETS):
                        i = (j + 3 * t + r) % N_SETS
                        o, fin = _call(cases[i])
                        stream.synchronize()
                        if not (torch.equal(o, ref[i][0]) and torch.equal(fin, ref[i][1])):
                            errors.append("thread %d round %d set %d differs" % (t, r, i))
        except Exception as e:  # reported below, in the main thread
            errors.append("thread %d: %r" % (t, e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(N_THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors[:5]
