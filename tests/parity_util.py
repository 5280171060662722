"""Helpers shared by the GPU parity tests: device transfer, error statistics and
the tolerance rules.

Tolerances (on outputs o and final states, separately):
- fp32 inputs: max |gpu - oracle| <= 1e-4 (absolute);
- bf16 inputs: max |gpu - oracle| <= 2e-2 * RMS(oracle), with fp32-stored o;
- bf16-stored o additionally carries its own rounding: the bound becomes
  2e-2 * RMS(oracle) + 2^-8 |oracle| elementwise (round-to-nearest-even moves a
  value by at most half a bf16 unit in the last place, 2^-8 relative).
"""

from __future__ import annotations

import numpy as np

TOL_F32_ABS = 1e-4
TOL_BF16_REL_RMS = 2e-2


def torch_mod():
    import torch

    return torch


def dev(x, dtype="f32", device="cuda"):
    """numpy -> torch on the GPU; dtype 'bf16' casts exactly-representable values."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.float32).to(torch.bfloat16)
    elif dtype == "f32":
        t = t.to(torch.float32)
    elif dtype == "i32":
        t = t.to(torch.int32)
    return t.to(device)


def host(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def stats(got, ref) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    mx = float(err.max()) if err.size else 0.0
    return {
        "max_abs": mx,
        "rms_ref": rms,
        "max_over_rms": mx / rms if rms > 0 else (0.0 if mx == 0 else float("inf")),
        "rms_err_over_rms": (float(np.sqrt(np.mean(err * err))) / rms) if rms > 0 else 0.0,
        "nonfinite": int(np.count_nonzero(~np.isfinite(got))),
    }


def assert_f32(got, ref, what=""):
    s = stats(got, ref)
    assert s["nonfinite"] == 0, (what, s)
    assert s["max_abs"] <= TOL_F32_ABS, (what, s)
    return s


def assert_bf16(got, ref, what="", bf16_store=False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    s = stats(got, ref)
    assert s["nonfinite"] == 0, (what, s)
    bound = TOL_BF16_REL_RMS * s["rms_ref"]
    if bf16_store:
        excess = np.abs(got - ref) - (bound + 2.0 ** -8 * np.abs(ref))
        assert excess.max() <= 0, (what, s, float(excess.max()))
    else:
        assert s["max_abs"] <= bound, (what, s)
    return s


def assert_units_bf16(o, ref, cu, what="", bf16_store=False, fin=None, fref=None):
    """Every (sequence, head) unit of a packed or batched run against the oracle, each to the bf16
    bound of its own RMS: o, ref [T, H, V]; cu [N + 1] offsets; fin, fref [N, H, K, V] optional."""
    o = np.asarray(o)
    ref = np.asarray(ref)
    assert o.shape == ref.shape, (o.shape, ref.shape)
    assert np.all(np.isfinite(o)), what
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            err = np.abs(o[a:b] - ref[a:b])  # [L, H, V]
            rms = np.sqrt(np.mean(ref[a:b] * ref[a:b], axis=(0, 2)))  # per head
            bound = TOL_BF16_REL_RMS * rms[None, :, None]
            if bf16_store:
                bound = bound + 2.0 ** -8 * np.abs(ref[a:b])
            excess = (err - bound).max(axis=(0, 2))
            h = int(np.argmax(excess))
            assert excess[h] <= 0, "%s: o unit (%d, %d) exceeds its bound by %.3e (max err %.3e, rms %.3e)" % (
                what, n, h, excess[h], err[:, h].max(), rms[h])
            worst = max(worst, float((err.max(axis=(0, 2)) / np.maximum(rms, 1e-300)).max()))
        if fin is not None:
            f, fr = np.asarray(fin[n]), np.asarray(fref[n])
            assert np.all(np.isfinite(f)), what
            err = np.abs(f - fr).max(axis=(1, 2))
            rms = np.sqrt(np.mean(fr * fr, axis=(1, 2)))
            h = int(np.argmax(err - TOL_BF16_REL_RMS * rms))
            assert err[h] <= TOL_BF16_REL_RMS * rms[h], "%s: final state (%d, %d): max err %.3e, rms %.3e" % (
                what, n, h, err[h], rms[h])
    return worst
