"""Pins of the tokenizer oracle (fun-rec-mdbook "OneTrans", section 7.5.0) against facts fixed
outside it: table values of the standard normal CDF, closed forms of the MLP in regimes where the
GELU is exactly linear or exactly zero, the merge's row arithmetic, and the Split order."""

import numpy as np
import pytest

import oracle
import synth

# Standard normal CDF Phi(x) from printed tables (GELU(x) = x Phi(x)).
PHI = {1.0: 0.8413447460685429, -1.0: 0.15865525393145707, 2.0: 0.9772498680518208, 0.5: 0.6914624612740131}


def _one_hot(shape, i, j):
    a = np.zeros(shape)
    a[i, j] = 1.0
    return a


@pytest.mark.parametrize("x", sorted(PHI))
def test_mlp_one_hot_path_is_gelu_of_one_input(x):
    # W1 picks input k0 into hidden unit h0, W2 copies h0 to output n0: the output is GELU(x_k0)
    # at n0 and the bias elsewhere. Non-square shapes pin the (out, in) orientation of both.
    d_in, hid, d_out, k0, h0, n0 = 5, 7, 3, 3, 4, 1
    e = np.full(d_in, -9.0)
    e[k0] = x
    b2 = np.array([0.25, 0.0, -0.5])
    y = oracle.mlp(e, _one_hot((hid, d_in), h0, k0), np.zeros(hid), _one_hot((d_out, hid), n0, h0), b2)
    expect = b2.copy()
    expect[n0] += x * PHI[x]
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=1e-15)


def test_mlp_linear_regime_is_the_composed_affine_map():
    # With b1 = +40 every pre-activation is >= 30, where GELU(z) = z to within z * Phi(-30) (< 1e-196),
    # so MLP(x) = (W2 W1) x + W2 b1 + b2 exactly in fp64.
    rng = np.random.default_rng(5)
    w1, w2 = rng.standard_normal((6, 4)) * 0.5, rng.standard_normal((3, 6))
    b1, b2 = np.full(6, 40.0), rng.standard_normal(3)
    x = rng.standard_normal((9, 4))
    expect = x @ (w2 @ w1).T + (w2 @ b1 + b2)
    np.testing.assert_allclose(oracle.mlp(x, w1, b1, w2, b2), expect, rtol=1e-12, atol=1e-12)
    # b1 = -40: every hidden unit is GELU(z <= -30) = 0 to within 1e-196, the output is b2
    np.testing.assert_allclose(oracle.mlp(x, w1, -b1, w2, b2), np.broadcast_to(b2, (9, 3)), atol=1e-150)


def _tok(key="tok_mid"):
    w = synth.tok_workload(key)
    return w, synth.tokenizer_weights(w), synth.tokenizer_sample(w, 1)


def test_merge_rows_and_sep_positions():
    # L_S = sum L_i + n (one [SEP] after each sequence, the empty one included); with W2 = 0 every
    # event row of sequence i is b2_i and row off_i + L_i is SEP_i
    w, tw, (ev, ns) = _tok()
    for p in tw["seq"]:
        p["w2"] = np.zeros_like(p["w2"])
    x = oracle.tokenize(ev, ns, tw, w.model.l_ns)
    assert x.shape == (w.l_s + w.model.l_ns, w.model.d_model)
    assert w.l_s == sum(w.seq_lens) + w.n_seq
    off = 0
    for i, L in enumerate(w.seq_lens):
        np.testing.assert_array_equal(x[off:off + L], np.broadcast_to(tw["seq"][i]["b2"], (L, w.model.d_model)))
        np.testing.assert_array_equal(x[off + L], tw["sep"][i])
        off += L + 1
    assert off == w.l_s


def test_split_order_of_ns_tokens():
    # W2 = 0 and b2 = 0, 1, 2, ...: NS token j must hold values [j d, (j + 1) d)
    w, tw, (ev, ns) = _tok()
    d, l_ns = w.model.d_model, w.model.l_ns
    tw["ns"]["w2"] = np.zeros_like(tw["ns"]["w2"])
    tw["ns"]["b2"] = np.arange(l_ns * d, dtype=np.float64)
    x = oracle.tokenize(ev, ns, tw, l_ns)
    for j in range(l_ns):
        np.testing.assert_array_equal(x[w.l_s + j], np.arange(j * d, (j + 1) * d))


def test_event_rows_depend_only_on_their_own_event():
    # MLP_i acts row by row: changing event 3 of sequence 2 changes exactly its own row of X(0),
    # and reversing a sequence's events reverses its rows
    w, tw, (ev, ns) = _tok()
    base = oracle.tokenize(ev, ns, tw, w.model.l_ns)
    ev2 = [e.copy() for e in ev]
    ev2[2][3] += 1.0
    changed = np.nonzero(np.any(oracle.tokenize(ev2, ns, tw, w.model.l_ns) != base, axis=1))[0]
    off2 = (w.seq_lens[0] + 1) + (w.seq_lens[1] + 1)
    assert changed.tolist() == [off2 + 3]
    ev3 = [e.copy() for e in ev]
    ev3[0] = ev3[0][::-1].copy()
    x3 = oracle.tokenize(ev3, ns, tw, w.model.l_ns)
    L0 = w.seq_lens[0]
    np.testing.assert_array_equal(x3[:L0], base[:L0][::-1])
    np.testing.assert_array_equal(x3[L0:], base[L0:])


def test_ns_rows_depend_only_on_ns_features():
    w, tw, (ev, ns) = _tok()
    base = oracle.tokenize(ev, ns, tw, w.model.l_ns)
    x = oracle.tokenize(ev, ns + 0.5, tw, w.model.l_ns)
    np.testing.assert_array_equal(x[:w.l_s], base[:w.l_s])
    assert np.all(np.any(x[w.l_s:] != base[w.l_s:], axis=1))


def test_no_ns_tokens():
    w, tw, (ev, ns) = _tok("tok_tiny")
    x = oracle.tokenize(ev, ns, tw, 0)
    assert x.shape == (w.l_s, w.model.d_model)
