"""GPU parity of the four C-ABI entry points against the CPU oracle.

Every comparison is element by element on the same seeded inputs; the bar is
max |gpu - oracle| / rms(oracle) <= 1e-4 in fp32 mode and <= 2e-2 in bf16 mode. Full-size
workloads run in the launch configuration the benchmark times and compare a seeded subset of
samples / users / candidates (samples are independent).
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


def _forward_case(w, samples=None):
    say(f"[forward] {w.key} dtype={w.model.dtype} B={w.batch} L_S={w.l_s} q={w.s_queries}")
    mdl = model(w)
    x = synth.forward_batch(w)
    out = ob.onetrans_forward(mdl, dev(x, mdl))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    idx = range(w.batch) if samples is None else samples
    ws = weights(w.model)
    for b in idx:
        ref = O.forward(x[b], ws, w.model, w.s_queries)
        e = rel_err(got[b], ref)
        say(f"  sample {b}: err {e:.3e}")
        assert e <= TOL[w.model.dtype], (w.key, b, e)
    return got


# --- small shapes: several tiles, ragged tails, both precisions -------------------------------

def test_tiny_config_fp32_all_samples():
    _forward_case(synth.workload("tiny"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny3_pyramid_forward(dtype):
    _forward_case(synth.test_workload("tiny3_fwd", dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_layernorm_bf16_and_f32(dtype):
    _forward_case(synth.workload("tiny", dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mid_shape_ragged_tiles(dtype):
    """d=256 / 8 heads (d_head 32, 128x128 GEMM tiles) with lengths that leave ragged tiles."""
    m = replace(synth.workload("onetrans_s").model, n_blocks=3, dtype=dtype)
    w = replace(synth.workload("onetrans_s"), model=m, l_s=203, s_queries=(203, 131, 5), seq_lens=(60, 70, 70),
                batch=5, key="mid_ragged")
    _forward_case(w)


@pytest.mark.parametrize("norm", ["rms", "layer"])
def test_d128_shape_both_norms(norm):
    """d=128 / 4 heads in bf16 (the wave-pair post-attention kernel at its narrower width), with
    RMSNorm and LayerNorm, ragged tiles and a pyramid."""
    base = synth.workload("onetrans_s")
    m = replace(base.model, n_blocks=3, d_model=128, n_heads=4, d_ff=512, norm=norm,
                norm_eps=1e-6 if norm == "rms" else 1e-5, dtype="bf16")
    w = replace(base, model=m, l_s=181, s_queries=(181, 97, 3), seq_lens=(50, 60, 68), batch=5,
                key=f"d128_{norm}")
    _forward_case(w)


def _two_stage_case(w):
    dtype = w.model.dtype
    say(f"[two_stage] {w.key} dtype={dtype} d={w.model.d_model} norm={w.model.norm}")
    mdl = model(w)
    m, ws = w.model, weights(w.model)
    xs = synth.user_sequences(w)
    xn = synth.candidate_batch(w)
    cache = ob.KVCache(mdl, w.n_users, w.l_s)
    out_s = torch.empty((w.n_users, w.s_queries[-1], m.d_model), dtype=torch.float32, device=mdl.device)
    ob.onetrans_prefill_user(mdl, dev(xs, mdl), cache, out_s)
    out = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    expect_len, s = [], w.l_s
    for q in w.s_queries:
        expect_len.append(s)
        s = q
    assert cache.lengths == expect_len
    for u in range(w.n_users):
        rc, rs = O.prefill_user(xs[u], ws, m, w.s_queries)
        assert rel_err(out_s[u].cpu().numpy(), rs) <= TOL[dtype]
        for n, (k, v) in enumerate(cache_to_host(cache, u, m.n_blocks, cache.lengths)):
            assert rel_err(k, rc[n]["k"]) <= TOL[dtype] and rel_err(v, rc[n]["v"]) <= TOL[dtype], (u, n)
        for c in range(w.n_cand):
            e = rel_err(out[u, c].cpu().numpy(), O.score_candidate(rc, xn[u, c], ws, m))
            say(f"  user {u} cand {c}: err {e:.3e}")
            assert e <= TOL[dtype]


def _append_case(w):
    dtype = w.model.dtype
    say(f"[append] {w.key} dtype={dtype} d={w.model.d_model} norm={w.model.norm}")
    m, ws = w.model, weights(w.model)
    mdl = model(w, s_queries=(w.l_old,) * m.n_blocks)
    old, new = synth.append_batch(w)
    xn = np.stack([synth.candidate_tokens(w, u, 0) for u in range(w.n_users)])[:, None]
    cache = ob.KVCache(mdl, w.n_users, w.l_old + w.d_l)
    ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
    out_new = torch.empty((w.n_users, w.d_l, m.d_model), dtype=torch.float32, device=mdl.device)
    ob.onetrans_append_events(mdl, cache, dev(new, mdl), out_new)
    sc = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    assert cache.lengths == [w.l_old + w.d_l] * m.n_blocks
    for u in range(w.n_users):
        oc, _ = O.prefill_user(old[u], ws, m, (w.l_old,) * m.n_blocks)
        nc, ref_new = O.append_events(oc, new[u], ws, m)
        assert rel_err(out_new[u].cpu().numpy(), ref_new) <= TOL[dtype]
        for n, (k, v) in enumerate(cache_to_host(cache, u, m.n_blocks, cache.lengths)):
            assert rel_err(k, nc[n]["k"]) <= TOL[dtype] and rel_err(v, nc[n]["v"]) <= TOL[dtype]
        e = rel_err(sc[u, 0].cpu().numpy(), O.score_candidate(nc, xn[u, 0], ws, m))
        say(f"  user {u}: score err {e:.3e}")
        assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_two_stage_small(dtype):
    _two_stage_case(synth.test_workload("tiny3_two_stage", dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_small(dtype):
    _append_case(synth.test_workload("tiny3_append", dtype))


def _wide_layernorm_model(d):
    """The OneTransS-like widths at d (d_head 32, d_ff = 4 d) with LayerNorm, 3 blocks, bf16."""
    return replace(synth.workload("onetrans_s").model, name=f"ln{d}", n_blocks=3, d_model=d, n_heads=d // 32,
                   d_ff=4 * d, norm="layer", norm_eps=1e-5, dtype="bf16", weight_seed=1200 + d)


@pytest.mark.parametrize("d", [256, 512])
def test_layernorm_bf16_wide_forward(d):
    """bf16 LayerNorm at d >= 256: block 1's norm 1 takes the row statistics in the QKV kernel (one
    pass about the row's first element), blocks 2 and 3 read the (mean, rstd) that the previous
    block's post kernel wrote; pyramid with ragged tiles and a batch of 5."""
    base = synth.workload("onetrans_s")
    w = replace(base, model=_wide_layernorm_model(d), l_s=203, s_queries=(203, 131, 5), seq_lens=(60, 70, 70),
                batch=5, key=f"ln{d}_fwd")
    _forward_case(w)


def test_layernorm_bf16_d256_two_stage_and_append():
    """The same LayerNorm statistics handoff on Stage I / Stage II and on append (d = 256)."""
    m = _wide_layernorm_model(256)
    _two_stage_case(replace(synth.test_workload("tiny3_two_stage"), model=m, key="ln256_two_stage"))
    _append_case(replace(synth.test_workload("tiny3_append"), model=m, key="ln256_append"))


# Calls whose query rows exceed the split-post bound (rows * 8 * d * 4 bytes of partials > 32 MiB)
# run every post launch over the whole FFN, and each hands the next block its normalised input rows
# as bf16 fragments (the QKV kernel then neither reads the fp32 rows nor normalises). Odd batches
# leave partial 32-row groups in every parameter group; block 2 of the d = 256 case has enough tiles
# for two token groups per wave, block 3 runs one.
_HANDOFF_CASES = {
    "d256_layer": dict(d=256, norm="layer", batch=31, l_s=1099, sq=(1099, 1000, 9), seq=(400, 400, 296),
                       samples=(0, 17, 30)),
    "d256_rms": dict(d=256, norm="rms", batch=31, l_s=1099, sq=(1099, 1000, 9), seq=(400, 400, 296),
                     samples=(0, 30)),
    "d128_layer": dict(d=128, norm="layer", batch=19, l_s=500, sq=(500, 300, 4), seq=(160, 170, 167),
                       samples=(0, 9, 18)),
    "d128_rms": dict(d=128, norm="rms", batch=19, l_s=500, sq=(500, 300, 4), seq=(160, 170, 167),
                     samples=(0, 18)),
    "d64_layer": dict(d=64, norm="layer", batch=37, l_s=460, sq=(460, 250, 3), seq=(150, 150, 157),
                      samples=(0, 20, 36)),
    # d = 512: the wave-pair post kernel hands over, each half of a pair its own 16 k-chunks
    "d512_layer": dict(d=512, norm="layer", batch=11, l_s=211, sq=(211, 150, 7), seq=(69, 69, 70),
                       samples=(0, 10)),
    "d512_rms": dict(d=512, norm="rms", batch=11, l_s=211, sq=(211, 150, 7), seq=(69, 69, 70),
                     samples=(0, 10)),
}


@pytest.mark.parametrize("key", sorted(_HANDOFF_CASES))
def test_forward_normalised_row_handoff(key):
    c = _HANDOFF_CASES[key]
    d, lns = c["d"], 16
    rows = c["batch"] * (c["sq"][0] + lns)
    assert rows * 8 * d * 4 > 32 << 20, "the call must be too large for split post launches"
    base = synth.workload("onetrans_s")
    m = replace(base.model, name=f"handoff_{key}", n_blocks=len(c["sq"]), d_model=d, n_heads=d // 32, d_ff=4 * d,
                norm=c["norm"], norm_eps=1e-6 if c["norm"] == "rms" else 1e-5, dtype="bf16",
                weight_seed=1300 + d + (c["norm"] == "layer"))
    w = replace(base, model=m, l_s=c["l_s"], s_queries=c["sq"], seq_lens=c["seq"], batch=c["batch"],
                key=f"handoff_{key}")
    _forward_case(w, samples=c["samples"])


@pytest.mark.parametrize("d,n_users", [(128, 40), (256, 20)])
def test_two_stage_normalised_row_handoff(d, n_users):
    """Stage I (n_users x 220 rows) and Stage II (n_users x 13 candidates x 16 NS rows) calls above
    the split-post bound, so each block's post launch hands the next block its normalised rows in
    both stages; bf16 LayerNorm with a pyramid, every user's cache and candidate against the oracle."""
    lns, l_s, n_cand = 16, 220, 13
    for rows in (n_users * l_s, n_users * n_cand * lns):
        assert rows * 8 * d * 4 > 32 << 20, "the calls must be too large for split post launches"
    base = synth.workload("onetrans_s")
    m = replace(base.model, name=f"two_stage_handoff_{d}", n_blocks=3, d_model=d, n_heads=d // 32, d_ff=4 * d,
                norm="layer", norm_eps=1e-5, dtype="bf16", weight_seed=1400 + d)
    w = replace(synth.test_workload("tiny3_two_stage"), model=m, l_s=l_s, s_queries=(l_s, 130, 20),
                seq_lens=(72, 72, 73), n_users=n_users, n_cand=n_cand, input_seed=2140 + d,
                key=f"two_stage_handoff_{d}")
    _two_stage_case(w)


def test_ragged_score_normalised_row_handoff():
    """Stage II over ragged cached users (each user's keys end at its own length) in a call above
    the split-post bound (4 users x 130 candidates x 16 NS rows at d = 128), so the normalised NS
    rows are handed over between blocks; bf16 LayerNorm, every candidate against the oracle run on
    that user's own rows."""
    d, lns, n_cand, cap = 128, 16, 130, 150
    assert 4 * n_cand * lns * 8 * d * 4 > 32 << 20, "the call must be too large for split post launches"
    base = synth.workload("onetrans_s")
    m = replace(base.model, name="ragged_score_handoff", n_blocks=3, d_model=d, n_heads=d // 32, d_ff=4 * d,
                norm="layer", norm_eps=1e-5, dtype="bf16", weight_seed=1611)
    w = replace(synth.test_workload("tiny3_two_stage"), model=m, l_s=cap, s_queries=(cap,) * 3,
                seq_lens=(49, 49, 49), n_users=4, n_cand=n_cand, input_seed=2171, key="ragged_score_handoff")
    ws = weights(m)
    lens = [150, 3, 97, 41]
    say(f"[ragged score handoff] lens={lens} candidates={n_cand}")
    mdl = model(w)
    xs = synth.user_sequences(w)                # rows past a user's length pad
    xn = synth.candidate_batch(w)
    cache = ob.KVCache(mdl, w.n_users, cap, user_len=lens)
    ob.onetrans_prefill_user(mdl, dev(xs, mdl), cache)
    sc = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    for u, n in enumerate(lens):
        rc, _ = O.prefill_user(xs[u, :n], ws, m, (n,) * m.n_blocks)
        e = max(rel_err(sc[u, c].cpu().numpy(), O.score_candidate(rc, xn[u, c], ws, m)) for c in range(n_cand))
        say(f"  user {u} (L {n}): worst candidate {e:.3e}")
        assert e <= TOL["bf16"], (u, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_users_prefill_append_score(dtype):
    """Users with different cached lengths in one call (cache.user_len): padded prefill, append
    behind each user's own length, then Stage II scoring against each user's own keys. Each user
    is checked against the oracle run on that user's own rows alone; a user with no cached rows
    appends onto an empty cache (the oracle then is Stage I of the new rows by themselves)."""
    w = replace(synth.test_workload("tiny3_append", dtype), n_users=5, n_cand=2, input_seed=2117)
    m, ws = w.model, weights(w.model)
    lens = [24, 1, 17, 0, 9]                    # cached rows per user before the append
    say(f"[ragged] {w.key} dtype={dtype} lens={lens} d_l={w.d_l}")
    mdl = model(w, s_queries=(w.l_old,) * m.n_blocks)
    seq = synth.user_sequences(w)               # [U][l_old + d_l][d]; rows past a user's length pad
    old = np.ascontiguousarray(seq[:, : w.l_old])
    new = np.ascontiguousarray(seq[:, w.l_old:])
    xn = synth.candidate_batch(w)
    cache = ob.KVCache(mdl, w.n_users, w.l_old + w.d_l, user_len=lens)
    ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
    assert cache.user_lengths == lens
    out_new = torch.empty((w.n_users, w.d_l, m.d_model), dtype=torch.float32, device=mdl.device)
    ob.onetrans_append_events(mdl, cache, dev(new, mdl), out_new)
    sc = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    assert cache.user_lengths == [n + w.d_l for n in lens]
    for u, n_old in enumerate(lens):
        if n_old:
            oc, _ = O.prefill_user(old[u, :n_old], ws, m, (n_old,) * m.n_blocks)
            nc, ref_new = O.append_events(oc, new[u], ws, m)
        else:
            nc, ref_new = O.prefill_user(new[u], ws, m, (w.d_l,) * m.n_blocks)
        e_new = rel_err(out_new[u].cpu().numpy(), ref_new)
        n_all = n_old + w.d_l
        for n, (k, v) in enumerate(cache_to_host(cache, u, m.n_blocks, [n_all] * m.n_blocks)):
            assert rel_err(k, nc[n]["k"]) <= TOL[dtype] and rel_err(v, nc[n]["v"]) <= TOL[dtype], (u, n)
        e_sc = max(rel_err(sc[u, c].cpu().numpy(), O.score_candidate(nc, xn[u, c], ws, m)) for c in range(w.n_cand))
        say(f"  user {u} (L_old {n_old}): new rows {e_new:.3e} scores {e_sc:.3e}")
        assert e_new <= TOL[dtype] and e_sc <= TOL[dtype], (u, e_new, e_sc)


def test_edge_cases_forward():
    """batch 1, no NS tokens, pyramid down to one S query."""
    base = synth.test_workload("tiny3_fwd", "bf16")
    _forward_case(replace(base, batch=1, s_queries=(32, 7, 1), key="b1_q1"))
    m0 = replace(base.model, l_ns=0)
    _forward_case(replace(base, model=m0, batch=3, key="no_ns"))


# --- full workloads (the benchmark's launch configurations) -----------------------------------

def test_onetrans_s_forward_bf16_full_batch():
    w = synth.workload("onetrans_s")
    _forward_case(w, samples=w.parity_subset)


def test_onetrans_s_forward_f32_mode():
    w = replace(synth.workload("onetrans_s", "f32"), batch=12)
    _forward_case(w, samples=(0, 5, 11))


def test_two_stage_full():
    w = synth.workload("two_stage")
    say(f"[two_stage full] U={w.n_users} C={w.n_cand}")
    m, ws = w.model, weights(w.model)
    mdl = model(w)
    xs = synth.user_sequences(w)
    xn = synth.candidate_batch(w)
    cache = ob.KVCache(mdl, w.n_users, w.l_s)
    ob.onetrans_prefill_user(mdl, dev(xs, mdl), cache)
    out = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for u in w.parity_subset:
        rc, _ = O.prefill_user(xs[u], ws, m, w.s_queries)
        for c in sorted(rng.choice(w.n_cand, 16, replace=False)):
            e = rel_err(out[u, c].cpu().numpy(), O.score_candidate(rc, xn[u, c], ws, m))
            assert e <= TOL["bf16"], (u, c, e)
        say(f"  user {u}: 16 candidates ok")


def test_append_full():
    w = synth.workload("append")
    say(f"[append full] U={w.n_users} L_old={w.l_old} dL={w.d_l}")
    m, ws = w.model, weights(w.model)
    mdl = model(w, s_queries=(w.l_old,) * m.n_blocks)
    old, new = synth.append_batch(w)
    xn = np.stack([synth.candidate_tokens(w, u, 0) for u in range(w.n_users)])[:, None]
    cache = ob.KVCache(mdl, w.n_users, w.l_s)
    ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
    out_new = torch.empty((w.n_users, w.d_l, m.d_model), dtype=torch.float32, device=mdl.device)
    ob.onetrans_append_events(mdl, cache, dev(new, mdl), out_new)
    sc = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    for u in w.parity_subset:
        oc, _ = O.prefill_user(old[u], ws, m, (w.l_old,) * m.n_blocks)
        nc, ref_new = O.append_events(oc, new[u], ws, m)
        e1 = rel_err(out_new[u].cpu().numpy(), ref_new)
        e2 = rel_err(sc[u, 0].cpu().numpy(), O.score_candidate(nc, xn[u, 0], ws, m))
        say(f"  user {u}: new rows {e1:.3e} score {e2:.3e}")
        assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_append_ragged_full():
    """The ragged append workload in the launch configuration the benchmark times: 128 users
    with their own cached lengths, each checked user recomputed alone by the oracle."""
    w = synth.workload("append_ragged")
    lens = synth.user_cached_lengths(w)
    say(f"[append ragged full] U={w.n_users} L_old {min(lens)}..{max(lens)} dL={w.d_l}")
    m, ws = w.model, weights(w.model)
    mdl = model(w, s_queries=(w.l_old,) * m.n_blocks)
    old, new = synth.append_batch(w)
    xn = np.stack([synth.candidate_tokens(w, u, 0) for u in range(w.n_users)])[:, None]
    cache = ob.KVCache(mdl, w.n_users, w.l_s, user_len=lens)
    ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
    out_new = torch.empty((w.n_users, w.d_l, m.d_model), dtype=torch.float32, device=mdl.device)
    ob.onetrans_append_events(mdl, cache, dev(new, mdl), out_new)
    sc = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    assert cache.user_lengths == [n + w.d_l for n in lens]
    for u in w.parity_subset:
        oc, _ = O.prefill_user(old[u, : lens[u]], ws, m, (lens[u],) * m.n_blocks)
        nc, ref_new = O.append_events(oc, new[u], ws, m)
        e1 = rel_err(out_new[u].cpu().numpy(), ref_new)
        e2 = rel_err(sc[u, 0].cpu().numpy(), O.score_candidate(nc, xn[u, 0], ws, m))
        say(f"  user {u} (L_old {lens[u]}): new rows {e1:.3e} score {e2:.3e}")
        assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_onetrans_l_forward_bf16_full_batch():
    w = synth.workload("onetrans_l")
    _forward_case(w, samples=w.parity_subset)


def test_onetrans_l_forward_f32_mode():
    """fp32 mode of the OneTransL shape (d = 512): the fp32 QKV kernel with one workgroup per CU
    and the 16-token-tile fp32 post kernel, over the whole 8-block pyramid 2048 -> 32."""
    w = replace(synth.workload("onetrans_l", "f32"), batch=4)
    _forward_case(w, samples=(0, 3))


def _f32_wide_model(norm):
    return replace(synth.workload("onetrans_l").model, name=f"f32w_{norm}", n_blocks=3, norm=norm,
                   norm_eps=1e-6 if norm == "rms" else 1e-5, dtype="f32", weight_seed=1250)


@pytest.mark.parametrize("norm", ["rms", "layer"])
def test_f32_d512_ragged_tiles(norm):
    """fp32 at d = 512 with both norms: 3 blocks, a pyramid with ragged 64-token post tiles and 128-
    token QKV tiles (203 -> 131 -> 5 S rows, 16 NS rows), batch 5."""
    base = synth.workload("onetrans_l")
    w = replace(base, model=_f32_wide_model(norm), l_s=203, s_queries=(203, 131, 5), seq_lens=(60, 70, 70),
                batch=5, key=f"f32_d512_{norm}")
    _forward_case(w)


def test_f32_d512_two_stage_and_append():
    m = _f32_wide_model("rms")
    _two_stage_case(replace(synth.test_workload("tiny3_two_stage"), model=m, key="f32_d512_two_stage"))
    _append_case(replace(synth.test_workload("tiny3_append"), model=m, key="f32_d512_append"))


# --- GPU-side invariants ----------------------------------------------------------------------

def test_gpu_two_stage_matches_gpu_forward():
    w = synth.test_workload("tiny3_two_stage", "f32")
    mdl = model(w)
    xs = synth.user_sequences(w)
    xn = synth.candidate_batch(w)
    cache = ob.KVCache(mdl, w.n_users, w.l_s)
    ob.onetrans_prefill_user(mdl, dev(xs, mdl), cache)
    sc = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl)).cpu().numpy()
    x0 = np.concatenate([np.repeat(xs[:, None], w.n_cand, 1), xn], axis=2).reshape(-1, w.l_s + w.model.l_ns,
                                                                                   w.model.d_model)
    fw = ob.onetrans_forward(mdl, dev(x0, mdl)).cpu().numpy()
    ns = fw[:, -w.model.l_ns:].reshape(sc.shape)
    assert rel_err(sc, ns) <= 1e-5


def test_forward_two_streams_equal_one_stream():
    """A batch of 64+ (128+) runs as two (four) parts on as many streams: bit-identical to one
    stream, and correct on both sides of the part boundaries (33 samples per part of 130)."""
    w = replace(synth.test_workload("tiny3_fwd", "bf16"), batch=130)
    say(f"[forward two and four streams] {w.key} B={w.batch}")
    mdl = model(w)
    x = synth.forward_batch(w)
    xd = dev(x, mdl)
    outs = []
    try:
        for n_streams in (1, 2, 4):
            ob.set_streams(n_streams)
            outs.append(ob.onetrans_forward(mdl, xd))
            torch.cuda.synchronize()
    finally:
        ob.set_streams(2)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    got = outs[2].cpu().numpy()
    for b in (0, 32, 33, 64, 65, 129):
        e = rel_err(got[b], O.forward(x[b], weights(w.model), w.model, w.s_queries))
        say(f"  sample {b}: err {e:.3e}")
        assert e <= TOL["bf16"], (b, e)


@pytest.mark.parametrize("ragged", [False, True])
def test_append_two_streams_equal_one_stream(ragged):
    """An append over 16+ (32+) users runs as two (four) parts on as many streams: the new rows and
    every written cache row are bit-identical to one stream; users on both sides of a part boundary
    (8 and 9 of 33) match the oracle."""
    w = replace(synth.test_workload("tiny3_append", "bf16"), n_users=33, input_seed=2118)
    m, ws = w.model, weights(w.model)
    lens = [(5 * u) % (w.l_old + 1) for u in range(w.n_users)] if ragged else None
    say(f"[append two streams] {w.key} users={w.n_users} ragged={ragged}")
    mdl = model(w, s_queries=(w.l_old,) * m.n_blocks)
    seq = synth.user_sequences(w)
    old = np.ascontiguousarray(seq[:, : w.l_old])
    new = np.ascontiguousarray(seq[:, w.l_old:])
    res = []
    try:
        for n_streams in (1, 2, 4):
            ob.set_streams(n_streams)
            cache = ob.KVCache(mdl, w.n_users, w.l_old + w.d_l, user_len=lens)
            ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
            out_new = torch.empty((w.n_users, w.d_l, m.d_model), dtype=torch.float32, device=mdl.device)
            ob.onetrans_append_events(mdl, cache, dev(new, mdl), out_new)
            torch.cuda.synchronize()
            res.append((out_new.clone(), cache.k.clone(), cache.v.clone(), cache.lengths, cache.user_lengths))
    finally:
        ob.set_streams(2)
    (o1, k1, v1, l1, u1) = res[0]
    for (o2, k2, v2, l2, u2) in res[1:]:
        assert torch.equal(o1, o2) and l1 == l2 and u1 == u2
        for u in range(w.n_users):    # each user's valid rows (rows past them are never written)
            rows = u1[u] if ragged else l1[0]
            assert torch.equal(k1[u, :, :, :rows], k2[u, :, :, :rows])
            assert torch.equal(v1[u, :, :, :rows], v2[u, :, :, :rows])
    for u in (8, 9):
        n_old = lens[u] if ragged else w.l_old
        if n_old:
            oc, _ = O.prefill_user(old[u, :n_old], ws, m, (n_old,) * m.n_blocks)
            _, ref_new = O.append_events(oc, new[u], ws, m)
        else:
            _, ref_new = O.prefill_user(new[u], ws, m, (w.d_l,) * m.n_blocks)
        e = rel_err(o2[u].cpu().numpy(), ref_new)
        say(f"  user {u} (L_old {n_old}): {e:.3e}")
        assert e <= TOL["bf16"], (u, e)


@pytest.mark.parametrize("ragged", [False, True])
def test_score_two_streams_equal_one_stream(ragged):
    """Stage II over 16+ (32+) users runs as two (four) parts on as many streams: bit-identical to
    one stream, and users on both sides of a part boundary (8 and 9 of 33) match the oracle."""
    w = replace(synth.test_workload("tiny3_two_stage", "bf16"), n_users=33, n_cand=3, input_seed=2119)
    m, ws = w.model, weights(w.model)
    say(f"[score two streams] {w.key} users={w.n_users} ragged={ragged}")
    sched = (w.l_s,) * m.n_blocks if ragged else w.s_queries
    lens = [(7 * u) % (w.l_s + 1) for u in range(w.n_users)] if ragged else None
    mdl = model(w, s_queries=sched)
    xs = synth.user_sequences(w)
    xn = synth.candidate_batch(w)
    cache = ob.KVCache(mdl, w.n_users, w.l_s, user_len=lens)
    ob.onetrans_prefill_user(mdl, dev(xs, mdl), cache)
    res = []
    try:
        for n_streams in (1, 2, 4):
            ob.set_streams(n_streams)
            res.append(ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl)))
            torch.cuda.synchronize()
    finally:
        ob.set_streams(2)
    assert torch.equal(res[0], res[1]) and torch.equal(res[0], res[2])
    got = res[2].cpu().numpy()
    for u in (8, 9):
        n_old = lens[u] if ragged else w.l_s
        if ragged and n_old == 0:
            continue
        oc, _ = O.prefill_user(xs[u, :n_old], ws, m, (n_old,) * m.n_blocks if ragged else w.s_queries)
        for c in range(w.n_cand):
            e = rel_err(got[u, c], O.score_candidate(oc, xn[u, c], ws, m))
            say(f"  user {u} cand {c}: {e:.3e}")
            assert e <= TOL["bf16"], (u, c, e)


def test_prefill_two_streams_equal_one_stream():
    """Stage I over 16+ (32+) users runs as two (four) parts on as many streams: cache and final rows
    bit-identical to one stream (pyramided schedule)."""
    w = replace(synth.test_workload("tiny3_two_stage", "bf16"), n_users=33, input_seed=2120)
    m = w.model
    say(f"[prefill two streams] {w.key} users={w.n_users}")
    mdl = model(w)
    xs = dev(synth.user_sequences(w), mdl)
    res = []
    try:
        for n_streams in (1, 2, 4):
            ob.set_streams(n_streams)
            cache = ob.KVCache(mdl, w.n_users, w.l_s)
            out = torch.empty((w.n_users, w.s_queries[-1], m.d_model), dtype=torch.float32, device=mdl.device)
            ob.onetrans_prefill_user(mdl, xs, cache, out)
            torch.cuda.synchronize()
            res.append((out.clone(), cache.k.clone(), cache.v.clone(), cache.lengths))
    finally:
        ob.set_streams(2)
    (o1, k1, v1, l1) = res[0]
    for (o2, k2, v2, l2) in res[1:]:
        assert torch.equal(o1, o2) and l1 == l2
        for n, rows in enumerate(l1):   # rows past a block's length are never written
            assert torch.equal(k1[:, n, :, :rows], k2[:, n, :, :rows])
            assert torch.equal(v1[:, n, :, :rows], v2[:, n, :, :rows])


# --- cross-request append on a pyramided cache ------------------------------------------------

def _pyramid_append_case(w, sched_old, steps, users=None, check=None):
    """Prefill the old rows with `sched_old`, append the new rows in `steps` chunks, then score one
    candidate per user; every cache row, the final new-event rows of the last append and the scores
    are compared with the oracle's recomputation of the longer sequence."""
    m, ws = w.model, weights(w.model)
    dtype = m.dtype
    old, new = synth.append_batch(w, users)
    n_users = old.shape[0]
    l_old = old.shape[1]
    say(f"[pyramid append] {w.key} dtype={dtype} U={n_users} L_old={l_old} sched={sched_old} steps={steps}")
    mdl = model(w, s_queries=sched_old)
    cap = l_old + sum(steps)
    cache = ob.KVCache(mdl, n_users, cap, x_tail=True)
    ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
    done, sched = 0, tuple(sched_old)
    for dl in steps:
        grown = O.grown_schedule(l_old + done, sched, dl)
        out_new = torch.empty((n_users, min(dl, grown[-1]), m.d_model), dtype=torch.float32, device=mdl.device)
        ob.onetrans_append_events(mdl, cache, dev(np.ascontiguousarray(new[:, done:done + dl]), mdl), out_new)
        done += dl
        sched = grown
    xn = np.stack([synth.candidate_tokens(w, u, 0) for u in range(n_users)])[:, None]
    sc = ob.onetrans_score_candidates(mdl, cache, dev(xn, mdl))
    torch.cuda.synchronize()
    expect_len = [l_old + done] + list(sched[:-1])
    assert cache.lengths == expect_len and cache.q_last == sched[-1], (cache.lengths, cache.q_last, sched)
    last = steps[-1]
    for u in (range(n_users) if check is None else check):
        rc, _ = O.prefill_user(np.concatenate([old[u], new[u, :done]]), ws, m, sched)
        _, ref_out = O.append_recompute(np.concatenate([old[u], new[u, :done - last]]), new[u, done - last:done], ws,
                                        m, O.grown_schedule(l_old, sched_old, done - last) if done > last else sched_old)
        e_out = rel_err(out_new[u].cpu().numpy(), ref_out)
        e_kv = 0.0
        for n, (k, v) in enumerate(cache_to_host(cache, u, m.n_blocks, cache.lengths)):
            e_kv = max(e_kv, rel_err(k, rc[n]["k"]), rel_err(v, rc[n]["v"]))
        e_sc = rel_err(sc[u, 0].cpu().numpy(), O.score_candidate(rc, xn[u, 0], ws, m))
        say(f"  user {u}: new rows {e_out:.3e} cache {e_kv:.3e} score {e_sc:.3e}")
        assert max(e_out, e_kv, e_sc) <= TOL[dtype], (u, e_out, e_kv, e_sc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("sched_old,steps", [((24, 20, 8), (8,)),       # first pruning block 2 of 3
                                             ((24, 24, 8), (8,)),       # only the last block prunes
                                             ((24, 20, 4), (8,)),       # more new rows than final rows
                                             ((24, 6, 2), (8,)),        # window smaller than the append
                                             ((24, 20, 8), (4, 3, 1))]) # three appends in a row
def test_pyramid_append_small(dtype, sched_old, steps):
    _pyramid_append_case(replace(synth.test_workload("tiny3_append", dtype), n_users=3, input_seed=2140),
                         sched_old, steps)


def test_pyramid_append_onetrans_s_shape():
    """The OneTransS pyramid on 16 users: 1158 cached rows, 32 appended; blocks 3-6 recomputed."""
    w = synth.workload("append_pyramid")
    _pyramid_append_case(w, w.s_queries, (w.d_l,), users=range(16), check=(0, 15))


def test_pyramid_append_two_streams_equal_one_stream():
    w = replace(synth.test_workload("tiny3_append", "bf16"), n_users=33, input_seed=2141)
    m = w.model
    mdl = model(w, s_queries=(24, 20, 8))
    old, new = synth.append_batch(w)
    res = []
    try:
        for n_streams in (1, 2, 4):
            ob.set_streams(n_streams)
            cache = ob.KVCache(mdl, w.n_users, 32, x_tail=True)
            ob.onetrans_prefill_user(mdl, dev(old, mdl), cache)
            out_new = torch.empty((w.n_users, 8, m.d_model), dtype=torch.float32, device=mdl.device)
            ob.onetrans_append_events(mdl, cache, dev(new, mdl), out_new)
            torch.cuda.synchronize()
            res.append((out_new.clone(), cache.k.clone(), cache.v.clone(), cache.lengths))
    finally:
        ob.set_streams(2)
    (o1, k1, v1, l1) = res[0]
    for (o2, k2, v2, l2) in res[1:]:
        assert torch.equal(o1, o2) and l1 == l2
        for n, rows in enumerate(l1):
            assert torch.equal(k1[:, n, :, :rows], k2[:, n, :, :rows])
            assert torch.equal(v1[:, n, :, :rows], v2[:, n, :, :rows])
