"""GPU parity of onetrans_tokenize (the tokenizers ahead of block 1) against the CPU oracle.

Element by element on the same seeded inputs; bar max |gpu - oracle| / rms(oracle) <= 1e-4 in
fp32 mode and <= 2e-2 in bf16 mode (X(0) itself is stored in the storage dtype). The full-size
workload runs in the launch configuration the benchmark times and compares a seeded subset of
samples (samples are independent).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import TOL, rel_err, say
from unified_transformer_recommender_amd import binding as ob

pytestmark = pytest.mark.gpu


def _setup(w, device="cuda"):
    m = w.model
    host_w = synth.make_weights(replace(m, n_blocks=1))     # block weights only give the Model its config
    mdl = ob.Model.from_host(replace(m, n_blocks=1), (w.l_s,), host_w, device=device)
    tw = synth.tokenizer_weights(w)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device, dtype=mdl.torch_dtype)
    seq = [{k: t(v) for k, v in p.items()} for p in tw["seq"]]
    ns = {k: t(v) for k, v in tw["ns"].items()} if tw["ns"] is not None else None
    tok = ob.Tokenizer(mdl, w.seq_lens, seq, t(tw["sep"]), ns, merge=w.merge)
    return mdl, tok, tw, t


def _case(w, samples=None):
    say(f"[tokenize] {w.key} dtype={w.model.dtype} B={w.batch} L={w.seq_lens} D={w.seq_dims} "
        f"H={w.seq_hidden} F={w.ns_dim} l_ns={w.model.l_ns} merge={w.merge}")
    mdl, tok, tw, t = _setup(w)
    ev, ns = synth.tokenizer_batch(w)
    times = synth.tokenizer_times_batch(w) if w.merge == "time" else None
    x0 = ob.onetrans_tokenize(tok, [t(e) for e in ev], t(ns) if w.model.l_ns > 0 else None,
                              times=[torch.from_numpy(x).to("cuda") for x in times] if times else None)
    torch.cuda.synchronize()
    got = x0.float().cpu().numpy()
    assert got.shape == (w.batch, w.l_s + w.model.l_ns, w.model.d_model)
    for b in (range(w.batch) if samples is None else samples):
        tb = [x[b] for x in times] if times else None
        ref = O.tokenize([e[b] for e in ev], ns[b], tw, w.model.l_ns, times=tb)
        e = rel_err(got[b], ref)
        say(f"  sample {b}: err {e:.3e}")
        assert e <= TOL[w.model.dtype], (w.key, b, e)
        if times is None:
            # [SEP] rows are copies: bit-exact
            off = 0
            for i, L in enumerate(w.seq_lens):
                np.testing.assert_array_equal(got[b, off + L], tw["sep"][i])
                off += L + 1
        else:
            # the merge order is index work: every GPU row is nearest to the oracle row at its own
            # position, far ahead of any other row
            g, r = got[b, :w.l_s].astype(np.float64), ref[:w.l_s]
            d2 = (g * g).sum(1)[:, None] + (r * r).sum(1)[None, :] - 2.0 * g @ r.T
            np.testing.assert_array_equal(np.argmin(d2, axis=1), np.arange(w.l_s))
    return got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tokenize_tiny(dtype):
    _case(synth.tok_workload("tok_tiny", dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tokenize_ragged_tiles_and_empty_sequence(dtype):
    _case(synth.tok_workload("tok_mid", dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tokenize_without_ns_tokens(dtype):
    _case(synth.tok_workload("tok_mid", dtype).with_model(l_ns=0))


def test_tokenize_sep_rows_only():
    w = replace(synth.tok_workload("tok_mid", "bf16"), seq_lens=(0, 0, 0, 0))
    _case(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tokenize_time_merge(dtype):
    _case(synth.tok_workload("tok_mid_time", dtype))


def test_tokenize_time_merge_ties_everywhere():
    """All events of a sample at one time: the merge is the intent order without [SEP] rows."""
    w = synth.tok_workload("tok_mid_time", "f32")
    mdl, tok, tw, t = _setup(w)
    ev, ns = synth.tokenizer_batch(w)
    times = [np.full((w.batch, L), 42, dtype=np.int64) for L in w.seq_lens]
    x0 = ob.onetrans_tokenize(tok, [t(e) for e in ev], t(ns), times=[torch.from_numpy(x).to("cuda") for x in times])
    torch.cuda.synchronize()
    got = x0.float().cpu().numpy()
    for b in range(w.batch):
        ref = O.tokenize([e[b] for e in ev], ns[b], tw, w.model.l_ns, times=[x[b] for x in times])
        assert rel_err(got[b], ref) <= TOL["f32"]


def test_tokenize_time_merge_unsorted_timestamps():
    """Timestamps shuffled inside each type (not chronological): the exact all-pairs path."""
    w = synth.tok_workload("tok_mid_time", "bf16")
    mdl, tok, tw, t = _setup(w)
    ev, ns = synth.tokenizer_batch(w)
    rng = np.random.default_rng(11)
    times = [np.ascontiguousarray(rng.permuted(x, axis=1)) for x in synth.tokenizer_times_batch(w)]
    x0 = ob.onetrans_tokenize(tok, [t(e) for e in ev], t(ns), times=[torch.from_numpy(x).to("cuda") for x in times])
    torch.cuda.synchronize()
    got = x0.float().cpu().numpy()
    for b in range(w.batch):
        ref = O.tokenize([e[b] for e in ev], ns[b], tw, w.model.l_ns, times=[x[b] for x in times])
        assert rel_err(got[b], ref) <= TOL["bf16"]
        g, r = got[b, :w.l_s].astype(np.float64), ref[:w.l_s]
        d2 = (g * g).sum(1)[:, None] + (r * r).sum(1)[None, :] - 2.0 * g @ r.T
        np.testing.assert_array_equal(np.argmin(d2, axis=1), np.arange(w.l_s))


def test_tokenize_time_merge_full_size_sampled():
    w = synth.tok_workload("tokenize_s_time")
    _case(w, samples=w.parity_subset)


def test_tokenize_d512_model():
    """The OneTransL-shaped model (d = 512, 16 NS tokens): output tiles of 512-wide rows, hidden widths
    up to 512, a 2 x 8192-wide Auto-Split output per sample."""
    base = synth.tok_workload("tok_mid", "bf16")
    w = replace(base, key="tok_l", model=synth.workload("onetrans_l").model, seq_lens=(20, 33, 0),
                seq_dims=(128, 64, 64), seq_hidden=(256, 512, 64), ns_dim=256, ns_hidden=512, batch=3)
    _case(w)
    _case(replace(w, merge="time"))


def test_tokenize_full_size_sampled():
    w = synth.tok_workload("tokenize_s")
    _case(w, samples=w.parity_subset)


def test_tokenize_feeds_forward():
    """X(0) from the tokenizer goes straight into onetrans_forward: the forward of the GPU-built
    X(0) matches the oracle's forward of the oracle's X(0) (tiny model, fp32)."""
    w = synth.tok_workload("tok_tiny", "f32")
    fw = synth.test_workload("tiny3_fwd", "f32")
    mdl = ob.Model.from_host(fw.model, fw.s_queries, synth.make_weights(fw.model), device="cuda")
    tw = synth.tokenizer_weights(w)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=mdl.torch_dtype)
    tok = ob.Tokenizer(mdl, w.seq_lens, [{k: t(v) for k, v in p.items()} for p in tw["seq"]], t(tw["sep"]),
                       {k: t(v) for k, v in tw["ns"].items()})
    ev, ns = synth.tokenizer_batch(w)
    out = ob.onetrans_forward(mdl, ob.onetrans_tokenize(tok, [t(e) for e in ev], t(ns)))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    x_ref = O.tokenize_batch(ev, ns, tw, w.model.l_ns)
    for b in range(w.batch):
        ref = O.forward(x_ref[b], synth.make_weights(fw.model), fw.model, fw.s_queries)
        e = rel_err(got[b], ref)
        say(f"  sample {b}: err {e:.3e}")
        assert e <= TOL["f32"], (b, e)
