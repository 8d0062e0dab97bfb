"""Comparison helpers shared by the GPU parity tests (test code only).

bf16 tolerance: max-abs 3e-2 and relative L2 1e-2. bf16 itself cannot place a
value of magnitude >= 8 within 3e-2 (its half-ulp there is 2^-5), so the
max-abs bound is applied elementwise to |got - ref| / max(1, |ref|): for
outputs of magnitude up to 1 it is the plain absolute bound.
"""
import numpy as np
import torch

BF16_MAX_ABS = 3e-2
BF16_REL_L2 = 1e-2


def to_np(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy() if t.dtype.is_floating_point \
            else t.detach().cpu().numpy()
    return np.asarray(t)


def bf16_round(a):
    """Round-to-nearest-even bf16 of float64 values (via float32, exact for the
    integer-valued cases this is used on)."""
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .to(torch.float64).numpy()


def rel_l2(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_close_bf16(got, ref, max_abs=BF16_MAX_ABS, rel=BF16_REL_L2, what=""):
    got, ref = to_np(got), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if got.size == 0:
        return 0.0, 0.0
    scaled = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    err = float(np.max(scaled))
    r = rel_l2(got, ref)
    assert err <= max_abs and r <= rel, \
        f"{what}: max|d|/max(1,|ref|)={err:.3e} (<= {max_abs}), relL2={r:.3e} (<= {rel})"
    return err, r
