"""Helpers for the GPU parity tests: move seeded bf16 inputs to the device and back."""
from __future__ import annotations

import numpy as np

from synth import bf16_bits_to_f64


def to_dev_bf16(bits: np.ndarray):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev(arr: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def from_dev_bf16_bits(t) -> np.ndarray:
    return t.detach().view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)


def from_dev_f64(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(from_dev_bf16_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_close(got: np.ndarray, ref: np.ndarray, max_abs=2e-2, mean_abs=2e-3, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e} (<= {max_abs}), mean-abs {mn:.3e} (<= {mean_abs})"
    return mx, mn


def assert_within_one_ulp(got: np.ndarray, ref: np.ndarray, what=""):
    """Prologue outputs: one bf16 ulp of the exact value, plus the fp32 rounding
    of the rotation a*cos - b*sin, which is relative to the row's magnitude and
    shows where the two products nearly cancel; 99% within half an ulp."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    row_scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    tol = bf16_ulp(ref) + 2.0 ** -20 * row_scale
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} beyond tolerance, max err/ulp {np.max(err / bf16_ulp(ref)):.3f}"
    assert np.mean(err <= bf16_ulp(ref) * 0.5 + 2.0 ** -20 * row_scale) > 0.99, what
