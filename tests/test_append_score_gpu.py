"""GPU parity of onetrans_append_score: a cross-request append followed by Stage II scoring of the
same users in one call, each block's attention for both query sets in one pass over the user's keys.

Two bars. Against the two separate calls it replaces (onetrans_append_events, then
onetrans_score_candidates on the extended cache) the results are bit-identical: the new rows, the
NS rows, every written cache row and the cache lengths. Against the oracle (the append, then Stage
II over the extended cache, per user) the bar is the parity suite's: max |gpu - oracle| /
rms(oracle) <= 1e-4 in fp32 mode, <= 2e-2 in bf16 mode.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import TOL, cache_to_host, dev, model, rel_err, say, weights
from unified_transformer_recommender_amd import binding as ob

pytestmark = pytest.mark.gpu


def _run(mdl, w, old, new, xn, lens, fused):
    cache = ob.KVCache(mdl, w.n_users, w.l_old + w.d_l, user_len=lens)
    ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
    x_new, x_ns = dev(new, mdl), dev(xn, mdl)
    if fused:
        out_new, out_ns = ob.onetrans_append_score(mdl, cache, x_new, x_ns)
    else:
        out_new = torch.empty((w.n_users, w.d_l, mdl.d_model), dtype=torch.float32, device=mdl.device)
        ob.onetrans_append_events(mdl, cache, x_new, out_new)
        out_ns = ob.onetrans_score_candidates(mdl, cache, x_ns)
    torch.cuda.synchronize()
    return out_new, out_ns, cache


def _case(w, lens, check_users):
    """Fused vs separate (bit-exact) and fused vs the oracle for `check_users`."""
    m, ws = w.model, weights(w.model)
    mdl = model(w, s_queries=(w.l_old,) * m.n_blocks)
    seq = synth.user_sequences(w)            # [U][l_old + d_l][d]; rows past a user's length pad
    old = np.ascontiguousarray(seq[:, : w.l_old])
    new = np.ascontiguousarray(seq[:, w.l_old:])
    xn = synth.candidate_batch(w)
    n1, s1, c1 = _run(mdl, w, old, new, xn, lens, fused=False)
    n2, s2, c2 = _run(mdl, w, old, new, xn, lens, fused=True)
    assert c1.lengths == c2.lengths and c1.user_lengths == c2.user_lengths and c1.q_last == c2.q_last
    assert torch.equal(n1, n2), "new rows differ from the separate calls"
    assert torch.equal(s1, s2), "NS rows differ from the separate calls"
    for u in range(w.n_users):   # each user's valid rows (rows past them are never written)
        rows = c1.user_lengths[u] if lens is not None else c1.lengths[0]
        assert torch.equal(c1.k[u, :, :, :rows], c2.k[u, :, :, :rows]), u
        assert torch.equal(c1.v[u, :, :, :rows], c2.v[u, :, :, :rows]), u
    dtype = m.dtype
    for u in check_users:
        n_old = lens[u] if lens is not None else w.l_old
        if n_old:
            oc, _ = O.prefill_user(old[u, :n_old], ws, m, (n_old,) * m.n_blocks)
            nc, ref_new = O.append_events(oc, new[u], ws, m)
        else:
            nc, ref_new = O.prefill_user(new[u], ws, m, (w.d_l,) * m.n_blocks)
        e_new = rel_err(n2[u].cpu().numpy(), ref_new)
        e_sc = max(rel_err(s2[u, c].cpu().numpy(), O.score_candidate(nc, xn[u, c], ws, m)) for c in range(w.n_cand))
        say(f"  user {u} (L_old {n_old}): new rows {e_new:.3e} scores {e_sc:.3e}")
        assert e_new <= TOL[dtype] and e_sc <= TOL[dtype], (u, e_new, e_sc)


@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_score_small(dtype, ragged):
    """3 blocks, d_head 16, 5 users x 3 candidates (12 NS rows per user); ragged: cached lengths
    24, 1, 17, 0, 9 (a user with no cached rows appends onto an empty cache)."""
    w = replace(synth.test_workload("tiny3_append", dtype), n_users=5, n_cand=3, input_seed=2119)
    lens = [24, 1, 17, 0, 9] if ragged else None
    say(f"[append+score] {w.key} dtype={dtype} lens={lens}")
    _case(w, lens, range(w.n_users))


@pytest.mark.parametrize("ragged", [False, True])
def test_append_score_split_over_streams(ragged):
    """33 users run as parts on several streams, each part's two workspaces at their own offsets;
    users on both sides of a part boundary (8, 9, 16, 17) match the oracle."""
    w = replace(synth.test_workload("tiny3_append", "bf16"), n_users=33, n_cand=2, input_seed=2120)
    lens = [(5 * u) % (w.l_old + 1) for u in range(w.n_users)] if ragged else None
    say(f"[append+score streams] users={w.n_users} ragged={ragged}")
    _case(w, lens, (8, 9, 16, 17))


@pytest.mark.parametrize("key", ["append", "append_ragged"])
def test_append_score_full(key):
    """The append workloads at full size (OneTransS shape, 128 users, 32 new rows, 1 candidate of 16
    NS rows), in the launch configuration the benchmark times."""
    w = synth.workload(key)
    lens = synth.user_cached_lengths(w) if key == "append_ragged" else None
    say(f"[append+score full] {key} U={w.n_users} dL={w.d_l}")
    _case(w, lens, (0, 127))


def test_append_score_two_candidates_full_width():
    """32 NS rows per user (2 candidates x 16 NS tokens) and 32 new rows: both query groups fill
    their 32 lanes; 20 users at the OneTransS shape with ragged lengths."""
    w = replace(synth.workload("append_ragged"), n_users=20, n_cand=2, input_seed=2121, parity_subset=(0, 19))
    lens = [int(x) for x in np.linspace(0, w.l_old, w.n_users)]
    say(f"[append+score 2 cand] U={w.n_users} lens {min(lens)}..{max(lens)}")
    _case(w, lens, (0, 19))
