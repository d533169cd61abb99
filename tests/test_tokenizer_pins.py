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


# --- timestamp-aware merge (events interleaved by time, type embedding added, no [SEP]) ---------

def _identity_mlp():
    # D_in = hidden = 1, d = 2: in the linear regime (b1 = +40) MLP(x) = [x, 0] to within 1e-12
    return {"w1": np.array([[1.0]]), "b1": np.array([40.0]), "w2": np.array([[1.0], [0.0]]),
            "b2": np.array([-40.0, 0.0])}


def test_time_merge_hand_example():
    # A: values 10, 11, 12 at times 1, 4, 9; B: values 20, 21, 22 at times 2, 3, 10. The type
    # embeddings [0, 1] and [0, 2] mark the type in the second column. Worked by hand: time order
    # 1 (A0), 2 (B0), 3 (B1), 4 (A1), 9 (A2), 10 (B2).
    ev = [np.array([[10.0], [11.0], [12.0]]), np.array([[20.0], [21.0], [22.0]])]
    t = [np.array([1, 4, 9]), np.array([2, 3, 10])]
    emb = np.array([[0.0, 1.0], [0.0, 2.0]])
    got = oracle.s_tokens_by_time(ev, t, [_identity_mlp(), _identity_mlp()], emb)
    expect = [[10, 1], [20, 2], [21, 2], [11, 1], [12, 1], [22, 2]]
    np.testing.assert_allclose(got, expect, atol=1e-12)


def test_time_merge_ties_keep_type_then_position_order():
    # equal times: type order first (A before B), then the order inside the sequence
    ev = [np.array([[1.0], [2.0]]), np.array([[3.0], [4.0]])]
    t = [np.array([5, 5]), np.array([5, 7])]
    emb = np.zeros((2, 2))
    got = oracle.s_tokens_by_time(ev, t, [_identity_mlp(), _identity_mlp()], emb)
    np.testing.assert_allclose(got[:, 0], [1, 2, 3, 4], atol=1e-12)
    t = [np.array([6, 6]), np.array([5, 6])]
    got = oracle.s_tokens_by_time(ev, t, [_identity_mlp(), _identity_mlp()], emb)
    np.testing.assert_allclose(got[:, 0], [3, 1, 2, 4], atol=1e-12)


def test_time_merge_disjoint_ranges_concatenate():
    w, tw, (ev, ns) = _tok("tok_mid")
    times = [np.arange(L) + 10_000 * (w.n_seq - i) for i, L in enumerate(w.seq_lens)]   # last type oldest
    x = oracle.tokenize(ev, ns, tw, w.model.l_ns, times=times)
    parts = [oracle.mlp(e, p["w1"], p["b1"], p["w2"], p["b2"]) + tw["sep"][i]
             for i, (e, p) in enumerate(zip(ev, tw["seq"]))]
    np.testing.assert_array_equal(x[:sum(w.seq_lens)], np.concatenate(parts[::-1], axis=0))


def test_time_merge_is_a_sorted_permutation():
    w = synth.tok_workload("tok_mid_time")
    tw = synth.tokenizer_weights(w)
    ev, ns = synth.tokenizer_sample(w, 2)
    times = synth.tokenizer_times(w, 2)
    x = oracle.tokenize(ev, ns, tw, w.model.l_ns, times=times)
    assert w.l_s == sum(w.seq_lens) and x.shape[0] == w.l_s + w.model.l_ns
    rows = np.concatenate([oracle.mlp(e, p["w1"], p["b1"], p["w2"], p["b2"]) + tw["sep"][i]
                           for i, (e, p) in enumerate(zip(ev, tw["seq"]))], axis=0)
    t_all = np.concatenate(times)
    # every merged row is one aligned row, each used once, and the times along the merge never fall
    idx = [int(np.argmin(np.abs(rows - r).sum(axis=1))) for r in x[:w.l_s]]
    np.testing.assert_array_equal(x[:w.l_s], rows[idx])
    assert sorted(idx) == list(range(w.l_s))
    assert np.all(np.diff(t_all[idx]) >= 0)


# --- the batched form used as the expectation of the GPU tokenizer tests ------------------------

def test_tokenize_batch_hand_worked_two_samples():
    # Two samples, two types, identity-like MLPs (MLP(x) = [x, 0] in the linear regime), so X(0)
    # is written out by hand. Intent merge: [A events; SEP_A; B events; SEP_B; NS rows]. The Auto-
    # Split MLP is the identity on its 4 features (linear regime again), so NS row j of a sample is
    # its feature pair j. Samples differ in every entry, so a swapped sample, a shifted row or a
    # mixed-up time fails.
    ident = _identity_mlp()
    ns_mlp = {"w1": np.eye(4), "b1": np.full(4, 40.0), "w2": np.eye(4), "b2": np.full(4, -40.0)}
    tw = {"seq": [ident, ident], "sep": np.array([[0.0, 7.0], [0.0, 8.0]]), "ns": ns_mlp}
    ev = [np.array([[[1.0], [2.0]], [[3.0], [4.0]]]),          # type A: [B=2][L=2][1]
          np.array([[[5.0]], [[6.0]]])]                        # type B: [B=2][L=1][1]
    ns = np.array([[0.1, 0.2, 0.3, 0.4], [0.5, 0.6, 0.7, 0.8]])
    got = oracle.tokenize_batch(ev, ns, tw, 2)
    expect = [[[1, 0], [2, 0], [0, 7], [5, 0], [0, 8], [0.1, 0.2], [0.3, 0.4]],
              [[3, 0], [4, 0], [0, 7], [6, 0], [0, 8], [0.5, 0.6], [0.7, 0.8]]]
    np.testing.assert_allclose(got, expect, atol=1e-12)
    # timestamp-aware: sample 0 has B's event first (time 0 < 1 < 2), sample 1 last (time 9)
    times = [np.array([[1, 2], [1, 2]]), np.array([[0], [9]])]
    got = oracle.tokenize_batch(ev, ns, tw, 2, times=times)
    expect = [[[5, 8], [1, 7], [2, 7], [0.1, 0.2], [0.3, 0.4]],
              [[3, 7], [4, 7], [6, 8], [0.5, 0.6], [0.7, 0.8]]]
    np.testing.assert_allclose(got, expect, atol=1e-12)


@pytest.mark.parametrize("key", ["tok_mid", "tok_mid_time"])
def test_tokenize_batch_is_per_sample_tokenize(key):
    # Every sample of the batched form equals the (pinned) single-sample form on that sample's own
    # events, features and times, and permuting the batch permutes the result.
    w = synth.tok_workload(key)
    tw = synth.tokenizer_weights(w)
    samples = [0, 3, 1]
    ev, ns = synth.tokenizer_batch(w, samples)
    times = synth.tokenizer_times_batch(w, samples) if w.merge == "time" else None
    got = oracle.tokenize_batch(ev, ns, tw, w.model.l_ns, times=times)
    for i, b in enumerate(samples):
        e1, n1 = synth.tokenizer_sample(w, b)
        t1 = synth.tokenizer_times(w, b) if times is not None else None
        np.testing.assert_array_equal(got[i], oracle.tokenize(e1, n1, tw, w.model.l_ns, times=t1))
    assert not np.array_equal(got[0], got[1])
    perm = [2, 0, 1]
    got_p = oracle.tokenize_batch([e[perm] for e in ev], ns[perm], tw, w.model.l_ns,
                                  times=None if times is None else [t[perm] for t in times])
    np.testing.assert_array_equal(got_p, got[perm])
