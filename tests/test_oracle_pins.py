"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test names the property it checks and where it comes from; the oracle is
only trusted because these hold.
"""

import math
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth
from oracle_refs import gelu_scalar, torch_encoder_layer_stack, torch_functional_forward

TINY = synth.workload("tiny")
T3 = synth.test_workload("tiny3_fwd")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def _shared_weights(ws):
    """Every NS parameter set replaced by the shared S set (W_NS,j = W_S)."""
    out = []
    for p in ws:
        q = p.copy()
        for f in ("wq", "wk", "wv", "wo", "w1", "b1", "w2", "b2"):
            a = getattr(q, f)
            a[1:] = a[0]
        out.append(q)
    return out


# --- elementary pieces against library routines ------------------------------------------------

def test_norms_and_gelu_match_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 64)) * 3 + 0.5
    g = 1 + 0.1 * rng.standard_normal(64)
    b = 0.1 * rng.standard_normal(64)
    t = torch.as_tensor
    assert _rel(O.rms_norm(x, g, 1e-6), F.rms_norm(t(x), (64,), weight=t(g), eps=1e-6).numpy()) < 1e-14
    assert _rel(O.layer_norm(x, g, b, 1e-5),
                F.layer_norm(t(x), (64,), weight=t(g), bias=t(b), eps=1e-5).numpy()) < 1e-14
    z = np.linspace(-6, 6, 1001)
    assert _rel(O.gelu(z), F.gelu(t(z), approximate="none").numpy()) < 1e-15
    # GELU special values: phi(0) = 0, phi(x) -> x for large x, phi(-x) -> 0
    assert O.gelu(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu(np.array([10.0]))[0] - 10.0) < 1e-12
    assert abs(O.gelu(np.array([-10.0]))[0]) < 1e-12


def test_weight_group_indexing():
    # [en] 7.5.1: rows 0..L_S-1 share set 0; NS token j (row L_S + j) owns set 1 + j.
    assert [O.weight_group(t, 5) for t in range(8)] == [0, 0, 0, 0, 0, 1, 2, 3]


# --- P5: reduction to a textbook pre-norm causal Transformer ----------------------------------

def test_textbook_reduction_torch_encoder_layer():
    """W_NS,j = W_S and no pyramid: the stack is torch's own pre-LN causal encoder layer."""
    m = TINY.model
    ws = _shared_weights(synth.make_weights(m))
    for b in range(3):
        x0 = synth.forward_sample(TINY, b)
        got = O.forward(x0, ws, m, TINY.s_queries)
        ref = torch_encoder_layer_stack(x0, ws, m)
        assert _rel(got, ref) < 1e-12


def test_textbook_reduction_multiblock_layernorm():
    m = replace(T3.model, norm="layer", norm_eps=1e-5)
    w = replace(T3, model=m, s_queries=(32, 32, 32))
    ws = _shared_weights(synth.make_weights(m))
    x0 = synth.forward_sample(w, 0)
    assert _rel(O.forward(x0, ws, m, w.s_queries), torch_encoder_layer_stack(x0, ws, m)) < 1e-12


@pytest.mark.parametrize("norm_kind", ["rms", "layer"])
def test_mixed_stack_matches_torch_functional(norm_kind):
    """Distinct NS parameter sets, pyramid 32 -> 20 -> 8: library attention with a bottom-right mask."""
    m = replace(T3.model, norm=norm_kind)
    w = replace(T3, model=m)
    ws = synth.make_weights(m)
    for b in range(2):
        x0 = synth.forward_sample(w, b)
        got = O.forward(x0, ws, m, w.s_queries)
        ref = torch_functional_forward(x0, ws, m, w.s_queries)
        assert got.shape == (w.s_queries[-1] + m.l_ns, m.d_model)
        assert _rel(got, ref) < 1e-12


# --- P1: S rows never see NS rows ------------------------------------------------------------

def test_s_rows_invariant_to_ns_inputs_and_weights():
    m = T3.model
    w = replace(T3, s_queries=(32, 32, 32))
    ws = synth.make_weights(m)
    x0 = synth.forward_sample(w, 0)
    base = O.forward(x0, ws, m, w.s_queries)
    rng = np.random.default_rng(5)
    x1 = x0.copy()
    x1[w.l_s:] = rng.standard_normal(x1[w.l_s:].shape).astype(np.float32)
    ws1 = [p.copy() for p in ws]
    for p in ws1:
        for f in ("wq", "wk", "wv", "wo", "w1", "b1", "w2", "b2"):
            a = getattr(p, f)
            a[1:] = rng.standard_normal(a[1:].shape).astype(np.float32) * 0.05
    pert = O.forward(x1, ws1, m, w.s_queries)
    np.testing.assert_array_equal(pert[: w.l_s], base[: w.l_s])
    assert np.max(np.abs(pert[w.l_s:] - base[w.l_s:])) > 1e-3     # NS rows do change


# --- P2: pyramid tail equality per block ------------------------------------------------------

def test_pyramid_tail_equals_full_query_block():
    m = T3.model
    ws = synth.make_weights(m)
    x0 = synth.forward_sample(T3, 1)
    s = T3.l_s
    for q in (32, 20, 8, 1):
        tail = O.block_forward(x0, s, q, ws[0], m)
        full = O.block_forward(x0, s, s, ws[0], m)
        assert tail.shape[0] == q + m.l_ns
        assert _rel(tail, full[s - q:]) < 1e-13


# --- P3: two-stage serving equals the monolithic forward ---------------------------------------

def test_two_stage_equals_forward():
    w = synth.test_workload("tiny3_two_stage")
    m = w.model
    ws = synth.make_weights(m)
    for u in range(w.n_users):
        xs = synth.user_sequence(w, u)
        cache, s_out = O.prefill_user(xs, ws, m, w.s_queries)
        assert [c["k"].shape[0] for c in cache] == [32, 32, 20]
        for c in range(w.n_cand):
            xn = synth.candidate_tokens(w, u, c)
            mono = O.forward(np.concatenate([xs, xn]), ws, m, w.s_queries)
            assert _rel(O.score_candidate(cache, xn, ws, m), mono[-m.l_ns:]) < 1e-12
            assert _rel(s_out, mono[: -m.l_ns]) < 1e-12


# --- P4: cross-request append equals full recompute ---------------------------------------------

def test_append_equals_recompute():
    w = synth.test_workload("tiny3_append")
    m = w.model
    ws = synth.make_weights(m)
    for u in range(w.n_users):
        old, new = synth.append_rows(w, u)
        full_cache, full_out = O.prefill_user(np.concatenate([old, new]), ws, m, w.s_queries)
        old_cache, _ = O.prefill_user(old, ws, m, (w.l_old,) * m.n_blocks)
        new_cache, new_out = O.append_events(old_cache, new, ws, m)
        for a, b in zip(new_cache, full_cache):
            assert _rel(a["k"], b["k"]) < 1e-12 and _rel(a["v"], b["v"]) < 1e-12
        assert _rel(new_out, full_out[w.l_old:]) < 1e-12
        xn = synth.candidate_tokens(w, u, 0)
        assert _rel(O.score_candidate(new_cache, xn, ws, m), O.score_candidate(full_cache, xn, ws, m)) < 1e-12


def test_padded_prefill_caches_each_users_own_rows():
    """Ragged users (reading R25): with the causal mask, rows past a user's own length (padding in
    a shared-length prefill) change none of the rows before them, so the first L rows of every
    block's cache and output equal those of the user's own L-row sequence. Rows of the padded
    run past L do differ from the unpadded ones (there are none), so the check is on the prefix."""
    w = synth.test_workload("tiny3_append")
    m = w.model
    ws = synth.make_weights(m)
    seq = synth.user_sequence(w, 0)                       # 32 rows
    full = seq.shape[0]
    pad_cache, pad_out = O.prefill_user(seq, ws, m, (full,) * m.n_blocks)
    for n_rows in (1, 9, 24):
        own_cache, own_out = O.prefill_user(seq[:n_rows], ws, m, (n_rows,) * m.n_blocks)
        for a, b in zip(own_cache, pad_cache):
            assert _rel(a["k"], b["k"][:n_rows]) < 1e-12 and _rel(a["v"], b["v"][:n_rows]) < 1e-12
        assert _rel(own_out, pad_out[:n_rows]) < 1e-12
    # the padding does matter to the rows after it: a changed padding row moves the last row
    alt = seq.copy()
    alt[24] += 1.0
    _, alt_out = O.prefill_user(alt, ws, m, (full,) * m.n_blocks)
    assert _rel(alt_out[:24], pad_out[:24]) < 1e-12 and _rel(alt_out[24:], pad_out[24:]) > 1e-6


def test_append_refuses_pyramided_cache():
    w = synth.test_workload("tiny3_two_stage")
    ws = synth.make_weights(w.model)
    cache, _ = O.prefill_user(synth.user_sequence(w, 0), ws, w.model, w.s_queries)
    with pytest.raises(ValueError):
        O.append_events(cache, np.zeros((2, w.model.d_model), np.float32), ws, w.model)


# --- cross-request append on a pyramided cache ------------------------------------------------

def test_grown_schedule_hand_examples():
    # leading blocks that keep every row grow with the sequence; from the first pruning block on the
    # kept counts stay (the OneTransS schedule after appending 32 rows to 1158)
    assert O.grown_schedule(1158, (1158, 955, 719, 484, 248, 12), 32) == (1190, 955, 719, 484, 248, 12)
    assert O.grown_schedule(24, (24, 24, 24), 8) == (32, 32, 32)          # no pyramid: everything grows
    assert O.grown_schedule(24, (24, 24, 8), 8) == (32, 32, 8)            # only the last block prunes
    assert O.grown_schedule(24, (20, 20, 8), 8) == (20, 20, 8)            # block 1 prunes: nothing grows
    assert O.grown_schedule(100, (100, 60, 60, 30), 10) == (110, 60, 60, 30)


def test_append_recompute_equals_incremental_append_without_pyramid():
    """On an unpyramided cache the recomputation of the longer sequence equals the incremental
    append (new rows only, against the cached keys), cache rows and new final rows both."""
    w = synth.test_workload("tiny3_append")
    m, ws = w.model, synth.make_weights(w.model)
    old, new = synth.append_rows(w, 1)
    flat = (w.l_old,) * m.n_blocks
    rc_cache, rc_out = O.append_recompute(old, new, ws, m, flat)
    inc_cache, inc_out = O.append_events(O.prefill_user(old, ws, m, flat)[0], new, ws, m)
    for a, b in zip(rc_cache, inc_cache):
        assert _rel(a["k"], b["k"]) < 1e-12 and _rel(a["v"], b["v"]) < 1e-12
    assert _rel(rc_out, inc_out) < 1e-12


def _pyramid_route(old, new, ws, m, sched):
    """Append by the exact route, built from oracle pieces: blocks up to the first pruning block n*
    keep their cached rows and compute only the new rows; block n*'s kept outputs of the old
    sequence (its window) are extended by the new rows' outputs and cut to the block's kept count;
    the blocks after n* run as Stage I over that window."""
    L = old.shape[0]
    s, n_star = L, None
    for n, q in enumerate(sched):
        if q < s:
            n_star = n
            break
        s = q
    old_cache, _ = O.prefill_user(old, ws, m, sched)
    head = n_star + 1 if n_star is not None else m.n_blocks
    # blocks 0..n*: the cached rows of each are the whole sequence so far (no pruning before n*)
    head_cache, head_out = O.append_events(old_cache[:head], new, ws[:head], m)
    if n_star is None or n_star == m.n_blocks - 1:
        d_l = new.shape[0]
        q_last = sched[-1] if n_star is not None else L + d_l
        return head_cache, head_out[d_l - min(d_l, q_last):]
    # block n*'s kept outputs of the old sequence: Stage I of the first n* + 1 blocks
    _, window_old = O.prefill_user(old, ws[:head], m, sched[:head])
    q_star = sched[n_star]
    window = np.concatenate([window_old, head_out])[-q_star:]
    tail_cache, final = O.prefill_user(window, ws[head:], m, sched[head:])
    d_l = new.shape[0]
    return head_cache + tail_cache, final[final.shape[0] - min(d_l, sched[-1]):]


@pytest.mark.parametrize("sched_old,d_l", [((24, 20, 8), 8), ((24, 24, 8), 8), ((24, 20, 4), 8), ((24, 20, 8), 3),
                                           ((24, 24, 24), 8)])
def test_pyramided_append_route_equals_recompute(sched_old, d_l):
    """The route the device follows reaches exactly the recomputation of the longer sequence: the
    blocks up to the first pruning block keep every old row's keys/values (causal mask, window
    start 0), and the block after it sees old rows whose values did not change, so only the blocks
    from there on need their (slid) windows recomputed. Covers a first pruning block in the middle,
    only the last block pruning, more new rows than final rows, and no pyramid."""
    w = synth.test_workload("tiny3_append")
    m, ws = w.model, synth.make_weights(w.model)
    old = synth.user_sequence(w, 0)[:24]
    new = synth.append_rows(w, 1)[1][:d_l] + 0.5
    rc_cache, rc_out = O.append_recompute(old, new, ws, m, sched_old)
    rt_cache, rt_out = _pyramid_route(old, new, ws, m, sched_old)
    grown = O.grown_schedule(24, sched_old, d_l)
    s = 24 + d_l
    for n, (a, b) in enumerate(zip(rt_cache, rc_cache)):
        assert a["k"].shape[0] == b["k"].shape[0] == s, (n, a["k"].shape, s)
        assert _rel(a["k"], b["k"]) < 1e-12 and _rel(a["v"], b["v"]) < 1e-12, n
        s = grown[n]
    assert rt_out.shape == rc_out.shape == (min(d_l, grown[-1]), m.d_model)
    assert _rel(rt_out, rc_out) < 1e-12
    # the old rows of the blocks up to the first pruning block are untouched by the append
    old_cache, _ = O.prefill_user(old, ws, m, sched_old)
    assert _rel(rc_cache[0]["k"][:24], old_cache[0]["k"]) < 1e-12
    if sched_old[0] == 24 and sched_old[1] < 24:
        assert _rel(rc_cache[1]["k"][:24], old_cache[1]["k"]) < 1e-12
        # ...while the block after the first pruning block sees a slid window: its rows change
        assert rc_cache[2]["k"].shape == old_cache[2]["k"].shape
        assert _rel(rc_cache[2]["k"], old_cache[2]["k"]) > 1e-6


# --- P6 / P7: closed forms of the mask ---------------------------------------------------------

def test_equal_scores_give_mean_of_visible_values():
    """W^K = 0 makes every score equal, so each query returns the mean of the V rows it may see.
    This fixes the visible key count of every query: causal S, NS behind all S, pyramid tail."""
    m = T3.model
    ws = synth.make_weights(m)
    for p in ws:
        p.wk[:] = 0
    x0 = synth.forward_sample(T3, 2)
    traces = []
    O.forward(x0, ws, m, T3.s_queries, traces)
    s = T3.l_s
    for n, tr in enumerate(traces):
        q = T3.s_queries[n]
        csum = np.cumsum(tr.v, axis=0) / np.arange(1, tr.v.shape[0] + 1)[:, None]
        assert _rel(tr.o, csum[s - q:]) < 1e-13
        s = q


def test_single_token_attention_returns_value():
    m = replace(T3.model, l_ns=0, n_blocks=1)
    ws = synth.make_weights(m)
    x = np.random.default_rng(1).standard_normal((1, m.d_model)).astype(np.float32)
    traces = []
    O.forward(x, ws, m, (1,), traces)
    assert _rel(traces[0].o, traces[0].v) < 1e-15


# --- mixed-parameter indexing through the pyramid: closed form --------------------------------

def test_mixed_indexing_closed_form():
    """W^V = 0 and W^1 = 0: the attention adds nothing and the FFN adds W2_g phi(b1_g) + b2_g.

    So each output row equals its input row plus, for every block, the term of the
    parameter set it belongs to: set 0 for S rows, set 1 + j for NS token j. The
    expectation is computed with scalar erf, independent of the oracle's code.
    """
    m = T3.model
    ws = synth.make_weights(m)
    for p in ws:
        p.wv[:] = 0
        p.w1[:] = 0
    x0 = synth.forward_sample(T3, 3).astype(np.float64)
    out = O.forward(x0, ws, m, T3.s_queries)
    expect = x0[T3.l_s - T3.s_queries[-1]:].copy()
    for p in ws:
        for r in range(expect.shape[0]):
            g = 0 if r < T3.s_queries[-1] else 1 + (r - T3.s_queries[-1])
            ph = np.array([gelu_scalar(float(z)) for z in p.b1[g]])
            expect[r] += np.asarray(p.w2[g], np.float64) @ ph + p.b2[g]
    assert _rel(out, expect) < 1e-13


# --- P8: brute force with scalar loops on a tiny block ----------------------------------------

def _brute_block(x, s, q_keep, p, m):
    p = p.__class__(**{f: np.asarray(getattr(p, f), np.float64).tolist() for f in p.FIELDS})
    T, d = len(x), len(x[0])
    H = m.n_heads
    dh = d // H

    def grp(t):
        return 0 if t < s else 1 + t - s

    def nrm(row, g, b):
        ms = sum(v * v for v in row) / d
        return [row[i] / math.sqrt(ms + m.norm_eps) * g[i] for i in range(d)]

    def mv(W, vec, bias=None):
        return [sum(W[o][i] * vec[i] for i in range(len(vec))) + (bias[o] if bias is not None else 0.0)
                for o in range(len(W))]

    xh = [nrm(x[t], p.norm1_g, p.norm1_b) for t in range(T)]
    K = [mv(p.wk[grp(t)], xh[t]) for t in range(T)]
    V = [mv(p.wv[grp(t)], xh[t]) for t in range(T)]
    out = []
    for t in range(s - q_keep, T):
        qv = mv(p.wq[grp(t)], xh[t])
        o = [0.0] * d
        for h in range(H):
            sc = [sum(qv[h * dh + c] * K[u][h * dh + c] for c in range(dh)) / math.sqrt(dh)
                  for u in range(t + 1)]
            mx = max(sc)
            e = [math.exp(z - mx) for z in sc]
            z = sum(e)
            for c in range(dh):
                o[h * dh + c] = sum(e[u] * V[u][h * dh + c] for u in range(t + 1)) / z
        y = [x[t][i] + v for i, v in enumerate(mv(p.wo[grp(t)], o))]
        yh = nrm(y, p.norm2_g, p.norm2_b)
        hid = [gelu_scalar(v) for v in mv(p.w1[grp(t)], yh, p.b1[grp(t)])]
        out.append([y[i] + v for i, v in enumerate(mv(p.w2[grp(t)], hid, p.b2[grp(t)]))])
    return out


def test_brute_force_scalar_block():
    m = replace(T3.model, d_model=8, n_heads=2, d_ff=16, l_ns=2, n_blocks=1)
    ws = synth.make_weights(m)
    x = np.random.default_rng(3).standard_normal((6, 8))
    got = O.block_forward(x, 4, 2, ws[0], m)
    ref = _brute_block(x.tolist(), 4, 2, ws[0], m)
    assert _rel(got, ref) < 1e-13


# --- P9: samples are independent ---------------------------------------------------------------

def test_batch_independence_and_permutation():
    m = TINY.model
    ws = synth.make_weights(m)
    x = synth.forward_batch(TINY, [0, 1, 2, 3])
    out = O.forward_batch(x, ws, m, TINY.s_queries)
    perm = [2, 0, 3, 1]
    out_p = O.forward_batch(x[perm], ws, m, TINY.s_queries)
    np.testing.assert_array_equal(out_p, out[perm])


# --- generator sanity (inputs only) ------------------------------------------------------------

def test_generators_are_seeded_and_regenerable():
    w = synth.workload("onetrans_s")
    a = synth.forward_sample(w, 7)
    b = synth.forward_batch(w, [6, 7])[1]
    np.testing.assert_array_equal(a, b)
    # bf16 storage: every value is a bf16 number
    assert np.all((a.view(np.uint32) & 0xFFFF) == 0)
    # [SEP] rows are shared across samples
    c = synth.forward_sample(w, 8)
    for r in w.sep_rows:
        np.testing.assert_array_equal(a[r], c[r])
    assert w.sep_rows == (187, 388, 1189) and w.l_s == 1190


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3], np.float32)
    r = synth.round_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                       # halfway, even mantissa kept
    assert r[2] == 1.0 + 4 * 2 ** -8         # halfway, rounds up to even
    assert r[3] == 1.0
    assert r[4] == -2.5
    assert abs(r[5] - 3.0e-3) <= 3.0e-3 * 2 ** -8
