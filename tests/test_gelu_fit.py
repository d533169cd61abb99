"""The bf16 kernels (post-attention FFN, tokenizer MLPs) evaluate GELU with a fitted sigmoid form instead of the erf
form. This reads the fit's coefficients from the kernel source, evaluates the same expression in
fp32 on the CPU, and checks it against the erf form over the range the hidden activations can
take and far beyond (host-only: no GPU, no oracle)."""

import os
import re

import numpy as np
from scipy.special import erf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POST = os.path.join(ROOT, "unified_transformer_recommender_amd", "csrc", "common.hpp")

# the bf16 activation this feeds is rounded to 8 significant bits right after; the fit's error
# stays below half a bf16 step of every activation of magnitude >= 0.14
BOUND = 2.8e-4


def _coefficients():
    src = open(POST).read()
    c = {k: float(v) for k, v in re.findall(r"constexpr float (GELU_FIT_A[13]) = ([-0-9.eE]+)f;", src)}
    assert len(c) == 2
    return c["GELU_FIT_A1"], c["GELU_FIT_A3"]


def _gelu_fit_f32(x):
    a1, a3 = _coefficients()
    f = np.float32
    L = f(-1.4426950408889634)
    x = x.astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        x2 = x * x
        z = x * (x2 * (f(a3) * L) + f(a1) * L)
        return x * (f(1) / (f(1) + np.exp2(z)))


def _gelu_erf(x):
    x = x.astype(np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def test_fit_error_bound():
    x = np.linspace(-40.0, 40.0, 400001)
    err = np.abs(_gelu_fit_f32(x).astype(np.float64) - _gelu_erf(x))
    assert err.max() < BOUND, err.max()


def test_fit_below_half_bf16_step_of_the_activation():
    # where |GELU(x)| >= 0.14 the fit's error is below half the bf16 rounding step of the result
    x = np.linspace(-12.0, 12.0, 240001)
    g = _gelu_erf(x)
    m = np.abs(g) >= 0.14
    half_step = np.abs(g[m]) * 2.0 ** -9
    err = np.abs(_gelu_fit_f32(x[m]).astype(np.float64) - g[m])
    assert np.all(err < half_step)


def test_fit_tails_and_special_values():
    x = np.array([-1e30, -1e4, -50.0, -10.0, 0.0, 10.0, 50.0, 1e4, 1e30], dtype=np.float32)
    y = _gelu_fit_f32(x)
    assert np.all(np.isfinite(y))
    assert y[4] == 0.0
    np.testing.assert_allclose(y[5:], x[5:], rtol=1e-6)          # identity for large positive x
    # large negative x: sigma(z) underflows to 0, so the result is (signed) zero
    assert np.all(np.abs(y[:4]) <= 1e-20)
