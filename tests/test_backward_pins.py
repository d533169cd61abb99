"""Pins of the oracle's backward (oracle/onetrans_backward.py) against facts fixed outside it:
torch.autograd in fp64 through an independent torch-functional build of the stack (library layers
F.rms_norm / F.layer_norm, F.linear, F.scaled_dot_product_attention, F.gelu), and central finite
differences of the oracle's own forward."""

from dataclasses import replace

import numpy as np
import pytest

import oracle as O
import synth
from oracle import onetrans_backward as OB
from oracle_refs import torch_functional_grads


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def _case(norm="rms", sched=(32, 20, 8), seed=5):
    w = synth.test_workload("tiny3_fwd")
    m = replace(w.model, norm=norm, norm_eps=1e-6 if norm == "rms" else 1e-5, weight_seed=1100 + seed)
    ws = synth.make_weights(m)
    x0 = synth.forward_sample(replace(w, model=m), 0)
    rng = np.random.default_rng(seed)
    d_out = rng.standard_normal((sched[-1] + m.l_ns, m.d_model))
    return m, ws, x0, d_out, sched


@pytest.mark.parametrize("norm", ["rms", "layer"])
@pytest.mark.parametrize("sched", [(32, 20, 8), (32, 32, 32), (32, 7, 1)])
def test_backward_matches_torch_autograd(norm, sched):
    """Every gradient (the input rows and each parameter of each block, the shared S set and every NS
    set separately) equals torch.autograd's to fp64 rounding, with a pyramid, without one, and with a
    pyramid down to one S query."""
    m, ws, x0, d_out, sched = _case(norm, sched)
    dx, grads = OB.backward(x0, ws, m, sched, d_out)
    tdx, tgrads = torch_functional_grads(x0, ws, m, sched, d_out)
    assert _rel(dx, tdx) < 1e-10
    for n, (g, tg) in enumerate(zip(grads, tgrads)):
        for f in OB.FIELDS:
            if norm == "rms" and f.endswith("_b"):
                assert np.all(g[f] == 0)                   # RMSNorm has no shift
            elif f.startswith("norm"):
                assert _rel(g[f], tg[f]) < 1e-9, (n, f)
            else:                                          # each weight set on its own: S set 0, NS sets 1 + j
                for gset in range(g[f].shape[0]):
                    assert _rel(g[f][gset], tg[f][gset]) < 1e-9, (n, f, gset, _rel(g[f][gset], tg[f][gset]))


def _loss(x0, ws, m, sched, d_out):
    return float(np.sum(O.forward(x0, ws, m, sched) * d_out))


def test_backward_matches_finite_differences():
    """Central differences of the oracle's forward loss for single entries of a Q, K, V, O, W1 and W2
    matrix in the S set and in NS sets, biases of both kinds of set, norm gains and shifts, and entries of
    S and NS input rows match the analytic gradient."""
    m, ws, x0, d_out, sched = _case("layer", (32, 20, 8), seed=7)
    ws = [type(p)(**{f: np.asarray(getattr(p, f), np.float64) for f in OB.FIELDS}) for p in ws]
    x0 = np.asarray(x0, np.float64)                  # fp64 copies: a step of h must not be rounded away
    dx, grads = OB.backward(x0, ws, m, sched, d_out)
    h = 1e-5
    picks = [(0, "wq", (0, 3, 5)), (0, "wk", (2, 1, 7)), (1, "wv", (0, 9, 4)), (1, "wo", (3, 0, 2)),
             (2, "w1", (0, 11, 6)), (2, "w2", (4, 5, 17)), (0, "b1", (1, 13)), (2, "b2", (0, 3)),
             (1, "norm1_g", (8,)), (2, "norm2_b", (1,)), (0, "norm2_g", (30,))]
    for n, f, idx in picks:
        wp = [p.copy() for p in ws]
        wm = [p.copy() for p in ws]
        getattr(wp[n], f)[idx] += h
        getattr(wm[n], f)[idx] -= h
        fd = (_loss(x0, wp, m, sched, d_out) - _loss(x0, wm, m, sched, d_out)) / (2 * h)
        assert abs(fd - grads[n][f][idx]) <= 1e-6 * max(1.0, abs(fd)), (n, f, idx, fd, grads[n][f][idx])
    for idx in [(0, 0), (11, 3), (31, 63), (33, 7), (35, 60)]:     # S rows and NS rows of X(0)
        xp, xm = x0.copy(), x0.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (_loss(xp, ws, m, sched, d_out) - _loss(xm, ws, m, sched, d_out)) / (2 * h)
        assert abs(fd - dx[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, dx[idx])


def test_backward_batch_sums_parameter_gradients():
    m, ws, _, _, sched = _case()
    w = replace(synth.test_workload("tiny3_fwd"), model=m)
    x = synth.forward_batch(w)[:3]
    rng = np.random.default_rng(3)
    d_out = rng.standard_normal((3, sched[-1] + m.l_ns, m.d_model))
    dxs, tot = OB.backward_batch(x, ws, m, sched, d_out)
    for b in range(3):
        dx, _ = OB.backward(x[b], ws, m, sched, d_out[b])
        np.testing.assert_array_equal(dxs[b], dx)
    parts = [OB.backward(x[b], ws, m, sched, d_out[b])[1] for b in range(3)]
    for n in range(m.n_blocks):
        for f in OB.FIELDS:
            np.testing.assert_allclose(tot[n][f], sum(p[n][f] for p in parts), rtol=1e-13, atol=1e-15)
