"""Host logic of bench.py on the CPU: the traffic figures it takes from the committed rocprofv3
summaries, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("workload,key", [
    (bench.MAIN, "traffic_bytes_per_launch"),
    (bench.MAIN + "_bf16o", "traffic_bytes_per_launch"),
    (bench.BATCHED, "traffic_bytes_per_launch"),
    (bench.LONG, "traffic_bytes_per_launch_segmented"),
    (bench.LONG, "traffic_bytes_per_launch_split"),
    (bench.WIDE, "traffic_bytes_per_launch"),
])
def test_profiled_traffic_reads_every_summary(workload, key):
    """Each summary's figure is read while its source digest matches the tree, and is at least the
    call's algorithmic bytes (traffic below them would mean a wrong calibration or parse)."""
    path = os.path.join(ROOT, "profiles", "chunk_fwd_%s.md" % workload)
    with open(path) as f:
        text = f.read()
    if "chunk_sources_sha256_16: %s" % bench.sources_digest(bench.CHUNK_SOURCES) not in text:
        pytest.skip("the kernel sources changed since this summary's counters were taken")
    got = bench.profiled_traffic(workload, key)
    assert isinstance(got, int) and got > 0
    base = workload[: -len("_bf16o")] if workload.endswith("_bf16o") else workload
    w = bench.gdn_inputs.WORKLOADS[base]
    N = w.batch_rows if w.batch_rows > 1 else w.n_samples
    o_bytes = 2 if workload.endswith("_bf16o") else 4
    alg = bench.chunk_alg_bytes(w.total_tokens, N, w.Hqk, w.Hv, w.K, w.V, o_bytes, s0=w.s0_std > 0)
    assert got >= alg


def test_profiled_traffic_missing_summary_or_key():
    assert bench.profiled_traffic("no_such_workload") is None
    assert bench.profiled_traffic(bench.MAIN, "no_such_key") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
