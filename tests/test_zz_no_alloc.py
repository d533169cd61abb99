"""The allocation-free Stage II entry point (onetrans_score_candidates_noalloc, for callers that
cannot allocate): through the C ABI, its output equals that of onetrans_score_candidates with a
caller workspace, element by element, on two calls in a row (the second with a smaller input, so
the static scratch holds the first call's contents when the second starts), and matches the CPU
oracle at the bf16 bar. Sizes past the scratch are refused on the host."""

import ctypes
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import TOL, dev, model, rel_err, say, weights
from unified_transformer_recommender_amd import _lib as L
from unified_transformer_recommender_amd import binding as ob

pytestmark = pytest.mark.gpu


def _prefilled(w):
    mdl = model(w)
    cache = ob.KVCache(mdl, w.n_users, w.l_s)
    ob.onetrans_prefill_user(mdl, dev(synth.user_sequences(w), mdl), cache)
    return mdl, cache


def _pair(mdl, cache, xn):
    """(reference with a workspace, allocation-free) outputs of the same Stage II call."""
    ref = ob.onetrans_score_candidates(mdl, cache, xn)
    out = torch.full_like(ref, float("nan"))
    ob.onetrans_score_candidates_noalloc(mdl, cache, xn, out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_workspace_entry_two_calls():
    w = replace(synth.test_workload("tiny3_two_stage", "bf16"), n_users=20, n_cand=7, input_seed=2131)
    say(f"[noalloc] {w.key} users={w.n_users} cand={w.n_cand} then 3 x 2")
    mdl, cache = _prefilled(w)
    xn = synth.candidate_batch(w)
    ref, out = _pair(mdl, cache, dev(xn, mdl))
    assert torch.equal(ref, out)
    # second call, smaller: the first three users, two candidates each (scratch holds the first call)
    small = dev(np.ascontiguousarray(xn[:3, :2]), mdl)
    ref2, out2 = _pair(mdl, cache, small)
    assert torch.equal(ref2, out2)
    ws, m = weights(w.model), w.model
    for u in (0, 2):
        rc, _ = O.prefill_user(synth.user_sequences(w)[u], ws, m, w.s_queries)
        for c in range(2):
            e = rel_err(out2[u, c].cpu().numpy(), O.score_candidate(rc, xn[u, c], ws, m))
            say(f"  user {u} cand {c}: err {e:.3e}")
            assert e <= TOL["bf16"]


def test_noalloc_full_user_at_onetrans_s_shape_then_ragged():
    """One OneTransS-shaped user with 512 candidates (about 34 MB of scratch), then a smaller call
    on a ragged cache of three users."""
    w = replace(synth.workload("two_stage"), n_users=1)
    say(f"[noalloc] two_stage shape, 1 user x {w.n_cand} candidates")
    mdl, cache = _prefilled(w)
    xn = synth.candidate_batch(w)
    ref, out = _pair(mdl, cache, dev(xn, mdl))
    assert torch.equal(ref, out)
    ws, m = weights(w.model), w.model
    rc, _ = O.prefill_user(synth.user_sequences(w)[0], ws, m, w.s_queries)
    for c in (0, 311, 511):
        e = rel_err(out[0, c].cpu().numpy(), O.score_candidate(rc, xn[0, c], ws, m))
        say(f"  cand {c}: err {e:.3e}")
        assert e <= TOL["bf16"]
    # second, smaller call: ragged users on an unpyramided schedule of the tiny model
    t = replace(synth.test_workload("tiny3_two_stage", "bf16"), n_users=3, n_cand=2, input_seed=2132)
    lens = [32, 5, 0]
    mdl2 = model(t, s_queries=(t.l_s,) * t.model.n_blocks)
    cache2 = ob.KVCache(mdl2, t.n_users, t.l_s, user_len=lens)
    ob.onetrans_prefill_user(mdl2, dev(synth.user_sequences(t), mdl2), cache2)
    ref2, out2 = _pair(mdl2, cache2, dev(synth.candidate_batch(t), mdl2))
    assert torch.equal(ref2, out2)


def test_noalloc_refuses_calls_past_the_scratch():
    w = synth.workload("two_stage")
    mdl, cache = _prefilled(replace(w, n_users=1))
    n_cand = 2048                                  # about twice what fits (903 candidates at this shape)
    assert mdl.workspace_bytes(L.OP_SCORE, 1, n_cand=n_cand) > L.SCRATCH_BYTES
    xn = torch.zeros((1, n_cand, w.model.l_ns, w.model.d_model), dtype=mdl.torch_dtype, device=mdl.device)
    out = torch.empty((1, n_cand, w.model.l_ns, w.model.d_model), dtype=torch.float32, device=mdl.device)
    with pytest.raises(L.OneTransError) as e:
        ob.onetrans_score_candidates_noalloc(mdl, cache, xn, out)
    assert e.value.status == L.ERR_SCRATCH
