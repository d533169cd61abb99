"""The bf16 post-attention kernel evaluates GELU with a fitted sigmoid form instead of the erf
form. This reads the fit's coefficients and clamp from the kernel source, evaluates the same
expression in fp32 on the CPU, and checks it against the erf form over the range the hidden
activations can take and far beyond (host-only: no GPU, no oracle)."""

import os
import re

import numpy as np
from scipy.special import erf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POST = os.path.join(ROOT, "unified_transformer_recommender_amd", "csrc", "post.hip")


def _coefficients():
    src = open(POST).read()
    c = {k: float(v) for k, v in re.findall(r"constexpr float (GELU_FIT_A[135]) = ([-0-9.eE]+)f;", src)}
    clamp = re.search(r"fmed3f\(x, -([0-9.]+)f, ([0-9.]+)f\)", src)
    assert len(c) == 3 and clamp and clamp.group(1) == clamp.group(2)
    return c["GELU_FIT_A1"], c["GELU_FIT_A3"], c["GELU_FIT_A5"], float(clamp.group(1))


def _gelu_fit_f32(x):
    a1, a3, a5, lim = _coefficients()
    f = np.float32
    L = f(-1.4426950408889634)
    x = x.astype(np.float32)
    xc = np.clip(x, f(-lim), f(lim))
    x2 = xc * xc
    z = xc * (x2 * (x2 * (f(a5) * L) + f(a3) * L) + f(a1) * L)
    with np.errstate(over="ignore"):
        return x * (f(1) / (f(1) + np.exp2(z)))


def _gelu_erf(x):
    x = x.astype(np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def test_fit_error_bound():
    x = np.linspace(-40.0, 40.0, 400001)
    err = np.abs(_gelu_fit_f32(x).astype(np.float64) - _gelu_erf(x))
    assert err.max() < 8.0e-5, err.max()


def test_fit_tails_and_special_values():
    x = np.array([-1e30, -1e4, -50.0, -10.0, 0.0, 10.0, 50.0, 1e4, 1e30], dtype=np.float32)
    y = _gelu_fit_f32(x)
    assert np.all(np.isfinite(y))
    assert y[4] == 0.0
    np.testing.assert_allclose(y[5:], x[5:], rtol=1e-6)          # identity for large positive x
    # large negative x: sigma(z(-10)) is about 4.4e-16, so the result is zero to fp32 precision
    # relative to x (and below 1e-5 in absolute terms up to |x| = 1e10)
    assert np.all(np.abs(y[:4]) <= 5e-16 * np.abs(x[:4]))
