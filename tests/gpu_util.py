"""Helpers for the GPU parity tests (comparison of HIP results with oracle results)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f16_bits(scales) -> np.ndarray:
    """Scale plane as raw fp16 bit patterns (uint16) from a torch int16 tensor or numpy float16."""
    if isinstance(scales, torch.Tensor):
        return scales.cpu().numpy().view(np.uint16)
    return np.asarray(scales, dtype=np.float16).view(np.uint16)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in f32 units-in-the-last-place between two f32 arrays (monotone int mapping)."""
    def key(x):
        i = np.asarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(key(a) - key(b))


def assert_f32_match(got, want, max_ulp=1, max_frac_inexact=1e-3, what=""):
    """The GPU node rounds f64-accurate results to f32 like the oracle: nearly all elements are
    identical, the rest differ by one ulp (an f64 rounding at an f32 tie)."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(want)), what
    d = ulp_diff(got, want)
    frac = float(np.mean(d != 0)) if d.size else 0.0
    say(f"  {what}: {d.size} values, identical {1 - frac:.6f}, max ulp {int(d.max()) if d.size else 0}")
    assert int(d.max()) <= max_ulp, f"{what}: max ulp diff {int(d.max())}"
    assert frac <= max_frac_inexact, f"{what}: {frac} of values differ"


def assert_codes_match(gc, gs, oc, os_, max_frac_code_diff=0.0, what=""):
    gc = gc.cpu().numpy() if isinstance(gc, torch.Tensor) else gc
    gsb, osb = f16_bits(gs), f16_bits(os_)
    dc = np.abs(gc.astype(np.int32) - oc.astype(np.int32))
    frac_c = float(np.mean(dc != 0))
    frac_s = float(np.mean(gsb != osb))
    say(f"  {what}: codes differ {frac_c:.2e} (max {int(dc.max())}), scales differ {frac_s:.2e}")
    if max_frac_code_diff == 0.0:
        np.testing.assert_array_equal(gc, oc, err_msg=what)
        np.testing.assert_array_equal(gsb, osb, err_msg=what)
    else:
        assert frac_c <= max_frac_code_diff and int(dc.max()) <= 1, what
        assert frac_s <= max_frac_code_diff * 32, what
