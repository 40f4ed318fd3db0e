"""Helpers shared by the GPU parity tests (not a test module).

Tolerance rule: max|y_gpu - y_oracle| <= tau * RMS(y_oracle), with RMS over the
whole oracle tensor of the call and the max over all elements; tau = 1e-4 for
float32 inputs and 2e-2 for bf16 inputs (float32 accumulation and state).

A bf16 output also carries the round-to-nearest-even step of its own storage
format, up to 2^-8·|y| per element.  On the 2.7B-layer shape that step alone,
applied to the exact result, reaches 0.032·RMS(y) with the D skip and 0.043
without it, so no bf16 output could meet the bar with it counted.  For outputs
stored in bf16 the check therefore allows each element that rounding step on
top of tau·RMS:  max(|err_i| - 2^-8·|y_i|) <= tau·RMS.  States are float32 and
are held to the plain rule.
"""
from __future__ import annotations

import numpy as np

BF16_UNIT_ROUNDOFF = 2.0 ** -8
TAU_F32 = 1e-4
TAU_BF16 = 2e-2


def to_dev(t, device="cuda"):
    """gen.Tensor -> torch tensor on `device` (bf16 and float8 bits reinterpreted,
    no rounding)."""
    import torch
    if t is None:
        return None
    if t.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)
    if t.dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device).view(torch.float8_e4m3fn)
    return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)


def to_f64(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.double().numpy()


def stats(gpu, ref, bf16_output: bool):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    allow = BF16_UNIT_ROUNDOFF * np.abs(r) if bf16_output else 0.0
    excess = float(np.max(err - allow)) if err.size else 0.0
    return dict(rms=rms, max_err_over_rms=float(err.max()) / rms if err.size else 0.0,
                excess_over_rms=excess / rms if err.size else 0.0,
                rms_err_over_rms=float(np.sqrt(np.mean(err * err))) / rms if err.size else 0.0)


def assert_parity(gpu, ref, tau, bf16_output, what=""):
    g = np.asarray(gpu, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    s = stats(g, ref, bf16_output)
    print(f"[parity] {what}: " + ", ".join(f"{k}={v:.3e}" for k, v in s.items()), flush=True)
    assert s["excess_over_rms"] <= tau, f"{what}: {s} exceeds tau={tau}"
    return s
