"""Host logic of the segment split of packed runs (csrc/split_plan.cpp), on the CPU.

The planner is compiled with g++ together with a small driver (split_plan_main.cpp) and run on
sample lengths shaped like the workloads; every plan is checked for what pass 1, the fp32 chains
and pass 2 rely on: the segments tile every sample in order and are chunk-aligned from its start;
pass 1 runs the first segment of every split sample forward (from the sample's start state, its
end state going to the start row of the second segment) and forms the maps of the segments
between the first and the last; each segment after the second gets its start from its sample's
chain, which begins at the second segment's start row and runs through the maps in order; pass 2
runs every other segment; every sample's final state comes from its last segment.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_linear_chunk_amd", "csrc")


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = str(tmp_path_factory.mktemp("plan") / "split_plan")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", CSRC, os.path.join(ROOT, "tests", "split_plan_main.cpp"),
                    os.path.join(CSRC, "split_plan.cpp"), "-o", exe], check=True)

    def run(lengths, Hv, V, has_s0=True, cus=256):
        inp = "%d %d %d %d %d %s" % (Hv, V, int(has_s0), cus, len(lengths), " ".join(map(str, lengths)))
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
        split, n_seg, n_prefix, n_chain, n_fwd = map(int, out[0].split())
        ints = np.array(out[1].split(), dtype=np.int64)
        return dict(split=bool(split), n_seg=n_seg, n_prefix=n_prefix, n_chain=n_chain, n_fwd=n_fwd, ints=ints,
                    pmax=int(out[2]))
    return run


def check_plan(p, lengths, has_s0):
    n_seg, n_prefix, n_chain, I = p["n_seg"], p["n_prefix"], p["n_chain"], p["ints"]
    assert len(I) == (n_seg + 1) + 3 * n_seg + n_prefix + 4 * n_chain + n_seg
    cu = np.concatenate([[0], np.cumsum(lengths)])
    seg_cu = I[: n_seg + 1]
    o = n_seg + 1
    order, s0_ref, sf_map = I[o: o + n_seg], I[o + n_seg: o + 2 * n_seg], I[o + 2 * n_seg: o + 3 * n_seg]
    pre = I[o + 3 * n_seg: o + 3 * n_seg + n_prefix]
    o2 = o + 3 * n_seg + n_prefix
    chains = I[o2: o2 + 4 * n_chain].reshape(n_chain, 4)
    seg_sample = I[o2 + 4 * n_chain:]
    assert seg_cu[0] == 0 and seg_cu[-1] == cu[-1] and np.all(np.diff(seg_cu) >= 0)
    # segments tile the samples: every sample boundary is a segment boundary
    assert set(cu.tolist()) <= set(seg_cu.tolist())
    sample = np.searchsorted(cu, seg_cu[:-1], side="right") - 1
    # zero-length samples own one empty segment each: attribute by final-state map instead
    owners = {}
    for i in range(n_seg):
        a, b = seg_cu[i], seg_cu[i + 1]
        if b > a:
            n = int(sample[i])
            assert cu[n] <= a and b <= cu[n + 1]
            assert seg_sample[i] == n  # the segment reads the chunk records of its sample
            assert (a - cu[n]) % 64 == 0  # chunk-aligned from the sample start
            owners.setdefault(n, []).append(i)
    assert sorted(order.tolist()) == list(range(n_seg))
    seg_len = np.diff(seg_cu)
    n_fwd = p["n_fwd"]
    pass2, fwd1 = order[: n_seg - n_fwd], order[n_seg - n_fwd:]
    assert np.all(np.diff(seg_len[pass2]) <= 0)  # longest first
    # an empty segment is the one segment of a zero-length sample (its final-state row)
    for i in range(n_seg):
        if seg_cu[i + 1] == seg_cu[i]:
            assert sf_map[i] == seg_sample[i]
    # final states: one per sample, from its last segment
    assert sorted(x for x in sf_map.tolist() if x >= 0) == list(range(len(lengths)))
    later = []
    split = {n: segs for n, segs in owners.items() if len(segs) > 1}
    for n, segs in owners.items():
        assert segs == list(range(segs[0], segs[-1] + 1))
        assert sf_map[segs[-1]] == n and all(sf_map[i] == -1 for i in segs[:-1])
        assert s0_ref[segs[0]] == ((-2 - n) if has_s0 else -1)
        later += [int(s0_ref[i]) for i in segs[1:]]
        for i in segs[:-1]:
            assert seg_len[i] % 64 == 0
    assert sorted(later) == list(range(n_prefix))
    # pass 1: the first segment of every split sample forward, then the middle segments' maps
    assert n_fwd == len(split) and len(pre) == n_prefix
    assert sorted(fwd1.tolist()) == sorted(segs[0] for segs in split.values())
    assert pre[:n_fwd].tolist() == sorted(segs[0] for segs in split.values())
    maps = pre[n_fwd:].tolist()
    assert maps == sorted(i for segs in split.values() for i in segs[1:-1])
    assert all(sf_map[i] == -1 for i in pre)
    # a forward pass-1 segment ends where the next segment's start row is read (s0_ref of i + 1)
    for i in pre[:n_fwd]:
        assert seg_sample[i + 1] == seg_sample[i] and s0_ref[i + 1] >= 0
    # chains: from the second segment's start row through the sample's maps, in order, to the
    # start rows of its later segments
    assert len(chains) == sum(1 for segs in split.values() if len(segs) > 2)
    for start, p0, count, out0 in chains:
        n = int(sample[maps[p0]])
        segs = split[n]
        assert count == len(segs) - 2
        assert start == s0_ref[segs[1]]
        assert maps[p0: p0 + count] == segs[1:-1]
        assert [int(s0_ref[i]) for i in segs[2:]] == list(range(out0, out0 + count))
    assert n_prefix <= p["pmax"]


def test_packed_workload_is_split(planner):
    lengths = [1097, 99, 338, 1601, 835, 265, 3540, 417]
    for has_s0 in (False, True):
        p = planner(lengths, 32, 128, has_s0)
        assert p["split"] and p["n_prefix"] >= 1
        check_plan(p, lengths, has_s0)
        seg_len = np.diff(p["ints"][: p["n_seg"] + 1])
        assert seg_len.max() < 3540 * 0.6  # the longest sample no longer bounds the scan


def test_one_long_sample_among_many_short_ones_is_split(planner):
    """The lengths the GPU test of packed calls with more than 64 samples runs through the split
    path (tests/test_gpu_many_samples.py): the long sample is cut, the short ones run whole."""
    lengths = [1] * 150 + [0] * 5 + [4000] + [37] * 10
    for has_s0 in (False, True):
        p = planner(lengths, 4, 128, has_s0)
        assert p["split"] and p["n_fwd"] == 1 and p["n_seg"] > len(lengths)
        check_plan(p, lengths, has_s0)


@pytest.mark.parametrize("lengths,Hv,V", [
    ([2500, 0, 700, 64, 1, 1350], 4, 128),
    ([2500, 0, 700, 64, 1, 1350], 4, 256),
    ([32768], 16, 128),
    ([0, 9000, 0], 8, 128),
    ([64 * 40, 64 * 40 + 1], 2, 128),
])
def test_plans_are_consistent(planner, lengths, Hv, V):
    for has_s0 in (False, True):
        p = planner(lengths, Hv, V, has_s0)
        if p["split"]:
            check_plan(p, lengths, has_s0)


@pytest.mark.parametrize("lengths,Hv,V", [
    ([4096] * 8, 32, 128),           # batched rows: balanced already
    ([100, 300, 64, 1], 32, 128),    # short samples
    ([139, 2655, 12374, 17600], 64, 256),  # many heads: no room for pass-1 blocks
])
def test_balanced_or_crowded_runs_are_not_split(planner, lengths, Hv, V):
    assert not planner(lengths, Hv, V)["split"]


def test_planner_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The planner is host C++ that runs on every split call: build it (host only, g++) with
    AddressSanitizer and UBSan and plan length mixes with empty samples, one long sample, many
    short ones and the workloads' shapes; any out-of-bounds access, leak or undefined operation
    aborts the driver or prints a report."""
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = str(tmp_path / "split_plan_san")
    build = subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                            "-fno-sanitize-recover=undefined", "-I", CSRC, os.path.join(ROOT, "tests", "split_plan_main.cpp"),
                            os.path.join(CSRC, "split_plan.cpp"), "-o", exe], capture_output=True, text=True)
    if build.returncode != 0:
        pytest.skip("sanitizer runtimes not available: " + build.stderr[-200:])
    rng = np.random.default_rng(3)
    cases = [
        (32, 128, [8192]),
        (32, 128, [0, 0, 8192, 0]),
        (32, 128, [1] * 300 + [20000]),
        (32, 256, [3000, 200, 64, 1, 700, 2500, 1000, 727]),
        (64, 256, [int(x) for x in rng.integers(0, 20000, 4)]),
        (32, 128, [int(x) for x in rng.integers(0, 3000, 90)]),
        (16, 128, [32768]),
    ]
    for Hv, V, lengths in cases:
        for has_s0 in (0, 1):
            inp = "%d %d %d %d %d %s" % (Hv, V, has_s0, 256, len(lengths), " ".join(map(str, lengths)))
            r = subprocess.run([exe], input=inp, capture_output=True, text=True,
                               env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
            assert r.returncode == 0, (Hv, V, lengths[:8], r.stderr[-2000:])
            assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
