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
