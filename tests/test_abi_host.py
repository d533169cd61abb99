"""C ABI checks that need no GPU: the library loads, exports every declared symbol, sizes its
buffers as documented, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from unified_transformer_recommender_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "onetrans.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libonetrans.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(onetrans_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "onetrans_forward" in names and "onetrans_tokenize" in names and len(names) == 17
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, f"binding lacks {n}"
    assert lib.onetrans_version().decode().startswith("onetrans-gfx950")


def _cfg(d=256, H=8, dff=1024, lns=16, N=2, sq=(100, 50), dtype=L.BF16, norm=L.RMSNORM):
    sqa = (ctypes.c_int * N)(*sq)
    c = L.Config(N, d, H, dff, lns, norm, 1e-6, dtype, sqa)
    c._keep = sqa
    return c


def _blocks(N, base=0x100000):
    b = (L.BlockWeights * N)()
    for i in range(N):
        for j, f in enumerate(L.WEIGHT_FIELDS):
            setattr(b[i], f, base + (i * 16 + j) * 4096)
    return b


FAKE = 0x7000000      # aligned, never dereferenced: every call below fails validation first


def test_workspace_and_cache_sizes():
    lib = L.lib()
    c = _cfg()
    B, l_s = 4, 120
    got = lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_FORWARD, B, l_s, 0, 0)
    d, T, R = 256, 136, 116
    al = lambda n: (n + 255) // 256 * 256
    part = al(B * R * 8 * d * 4)          # partial sums of split post launches (8 splits; at most 32 MiB)
    # bf16 rows normalised by each post launch for the next block's QKV launch, in 32-row groups of
    # each parameter group: at most one partial group per NS token and one for the S rows
    handoff = al((B * R + 32 * (16 + 1)) * d * 2)
    expect = (2 * al(B * R * d * 4) + 2 * al(B * R * 8) + al(B * R * d * 2) + 2 * al(B * T * d * 2) + al(B * R * d * 2)
              + al(16) + al(B * 4) + part + handoff)
    assert got == expect
    assert lib.onetrans_kv_cache_bytes(ctypes.byref(c), 3, 200) == 3 * 2 * 8 * 200 * 32 * 2
    assert lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_SCORE, 2, 0, 5, 0) > 0
    assert lib.onetrans_workspace_bytes(ctypes.byref(c), 9, 2, 10, 0, 0) == 0
    assert lib.onetrans_workspace_bytes(None, L.OP_FORWARD, 2, 10, 0, 0) == 0
    # pyramid longer than the sequence
    assert lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_FORWARD, 2, 60, 0, 0) == 0


def _fwd(c, blocks, x0=FAKE, B=2, l_s=120, out=FAKE, ws=FAKE, wsb=1 << 40):
    return L.lib().onetrans_forward(ctypes.byref(c) if c is not None else None, blocks, x0, B, l_s, out, ws, wsb,
                                    None)


def test_forward_validation_errors():
    c, b = _cfg(), _blocks(2)
    assert _fwd(None, b) == L.ERR_INVALID_ARG
    assert _fwd(c, None) == L.ERR_INVALID_ARG
    assert _fwd(c, b, x0=None) == L.ERR_INVALID_ARG
    assert _fwd(c, b, x0=FAKE + 2) == L.ERR_ALIGNMENT
    assert _fwd(c, b, out=FAKE + 8) == L.ERR_ALIGNMENT
    assert _fwd(c, b, wsb=1024) == L.ERR_WORKSPACE
    assert _fwd(c, b, ws=None) == L.ERR_INVALID_ARG
    assert _fwd(c, b, B=0) == L.ERR_SHAPE
    assert _fwd(c, b, l_s=60) == L.ERR_SHAPE                       # q_0 = 100 > s_0 = 60
    assert _fwd(_cfg(sq=(100, 120)), b) == L.ERR_SHAPE               # schedule must not grow
    assert _fwd(_cfg(sq=(100, 0)), b) == L.ERR_SHAPE
    assert _fwd(_cfg(d=256, H=4), b) == L.ERR_UNSUPPORTED            # d_head 64
    assert _fwd(_cfg(d=96, H=3), b) == L.ERR_UNSUPPORTED             # d not a multiple of 64
    assert _fwd(_cfg(d=192, H=6), b) == L.ERR_UNSUPPORTED            # d outside {64, 128, 256, 512}
    assert _fwd(_cfg(d=256, H=7), b) == L.ERR_SHAPE                  # d % H != 0
    assert _fwd(_cfg(lns=40), b) == L.ERR_UNSUPPORTED
    assert _fwd(_cfg(dtype=7), b) == L.ERR_INVALID_ARG
    assert _fwd(_cfg(norm=5), b) == L.ERR_INVALID_ARG
    nb = _blocks(2)
    nb[1].w2 = None
    assert _fwd(c, nb) == L.ERR_INVALID_ARG
    nb[1].w2 = FAKE + 4
    assert _fwd(c, nb) == L.ERR_ALIGNMENT
    # RMSNorm ignores the shift vectors, LayerNorm needs them
    nb = _blocks(2)
    nb[0].norm1_b = None
    assert _fwd(c, nb, wsb=1024) == L.ERR_WORKSPACE
    assert _fwd(_cfg(norm=L.LAYERNORM), nb) == L.ERR_INVALID_ARG


def test_launch_sizes_checked_before_enqueue():
    """Calls whose launch grids would not fit a 32-bit int fail validation (SHAPE) on the host, before
    the workspace check and before any HIP call, and advance no cache length."""
    lib = L.lib()
    c, b = _cfg(), _blocks(2)
    assert _fwd(c, b, B=1 << 21) == L.ERR_SHAPE                    # 2^21 x 136 rows x 8 heads > 2^31
    assert _fwd(c, b, B=1 << 20, wsb=1024) == L.ERR_WORKSPACE       # fits: 2^20 x 136 x 8 < 2^31
    kc = _cache(n_users=1 << 20, lens=(120, 120))
    assert lib.onetrans_score_candidates(ctypes.byref(c), b, ctypes.byref(kc), FAKE, 1 << 20, 64, FAKE, FAKE,
                                         1 << 40, None) == L.ERR_SHAPE
    flat = _cfg(sq=(120, 120))
    kc = _cache(n_users=1 << 22, cap=200, lens=(120, 120))
    assert lib.onetrans_append_events(ctypes.byref(flat), b, ctypes.byref(kc), FAKE, 1 << 22, 64, None, FAKE,
                                      1 << 40, None) == L.ERR_SHAPE
    assert list(kc._keep) == [120, 120]


def _cache(n_users=2, cap=200, lens=(120, 100)):
    ll = (ctypes.c_int * len(lens))(*lens)
    kc = L.KVCache(FAKE, FAKE, n_users, cap, ll)
    kc._keep = ll
    return kc


def test_serving_validation_errors():
    lib = L.lib()
    c, b = _cfg(), _blocks(2)
    kc = _cache()
    # prefill: capacity and user count
    assert lib.onetrans_prefill_user(ctypes.byref(c), b, FAKE, 2, 120, ctypes.byref(_cache(cap=100)), None, FAKE,
                                     1 << 40, None) == L.ERR_CACHE_CAPACITY
    assert lib.onetrans_prefill_user(ctypes.byref(c), b, FAKE, 3, 120, ctypes.byref(kc), None, FAKE, 1 << 40,
                                     None) == L.ERR_CACHE_CAPACITY
    assert lib.onetrans_prefill_user(ctypes.byref(c), b, FAKE, 2, 120, None, None, FAKE, 1 << 40,
                                     None) == L.ERR_INVALID_ARG
    assert lib.onetrans_prefill_user(ctypes.byref(c), b, FAKE, 2, 120, ctypes.byref(kc), None, FAKE, 16,
                                     None) == L.ERR_WORKSPACE
    # score: users beyond the cache, bad layer length, NS-free model
    assert lib.onetrans_score_candidates(ctypes.byref(c), b, ctypes.byref(kc), FAKE, 3, 4, FAKE, FAKE, 1 << 40,
                                         None) == L.ERR_SHAPE
    assert lib.onetrans_score_candidates(ctypes.byref(c), b, ctypes.byref(_cache(lens=(120, 300))), FAKE, 2, 4,
                                         FAKE, FAKE, 1 << 40, None) == L.ERR_SHAPE
    assert lib.onetrans_score_candidates(ctypes.byref(_cfg(lns=0)), b, ctypes.byref(kc), FAKE, 2, 4, FAKE, FAKE,
                                         1 << 40, None) == L.ERR_SHAPE
    assert lib.onetrans_score_candidates(ctypes.byref(c), b, ctypes.byref(kc), FAKE, 2, 4, FAKE, FAKE, 64,
                                         None) == L.ERR_WORKSPACE
    # append: a cache that prunes before its last block needs x_tail; a pyramid that grows is no state
    # prefill produces; the workspace must cover the recomputed window (100 rows here, not d_l = 8)
    assert lib.onetrans_append_events(ctypes.byref(c), b, ctypes.byref(kc), FAKE, 2, 8, None, FAKE, 1 << 40,
                                      None) == L.ERR_INVALID_ARG
    kt = _cache()
    kt.x_tail = FAKE
    small = lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_APPEND, 2, 0, 0, 8)
    need = lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_APPEND, 2, 100, 0, 8)
    assert 0 < small < need
    assert lib.onetrans_append_events(ctypes.byref(c), b, ctypes.byref(kt), FAKE, 2, 8, None, FAKE, small,
                                      None) == L.ERR_WORKSPACE
    kt.x_tail = FAKE + 8
    assert lib.onetrans_append_events(ctypes.byref(c), b, ctypes.byref(kt), FAKE, 2, 8, None, FAKE, need,
                                      None) == L.ERR_ALIGNMENT
    grows = _cache(lens=(100, 120))
    assert lib.onetrans_append_events(ctypes.byref(c), b, ctypes.byref(grows), FAKE, 2, 8, None, FAKE, 1 << 40,
                                      None) == L.ERR_SHAPE
    grows = _cache(lens=(100, 100))
    grows.q_last = 150
    assert lib.onetrans_append_events(ctypes.byref(c), b, ctypes.byref(grows), FAKE, 2, 8, None, FAKE, 1 << 40,
                                      None) == L.ERR_SHAPE
    assert list(kt._keep) == [120, 100]              # nothing advanced on error
    full = _cache(cap=128, lens=(124, 124))
    assert lib.onetrans_append_events(ctypes.byref(c), b, ctypes.byref(full), FAKE, 2, 8, None, FAKE, 1 << 40,
                                      None) == L.ERR_CACHE_CAPACITY
    assert list(full._keep) == [124, 124]            # nothing advanced on error
    assert lib.onetrans_append_events(ctypes.byref(c), b, ctypes.byref(full), FAKE, 2, 0, None, FAKE, 1 << 40,
                                      None) == L.ERR_SHAPE



def test_append_score_validation_errors():
    """The fused append + Stage II call: its own limits (d_l <= 32, n_cand * l_ns <= 32, an unpyramided
    cache, out_new required) and the checks of the two calls it replaces, all before any HIP call;
    no cache length advances on an error."""
    lib = L.lib()
    flat = _cfg(sq=(120, 120))
    b = _blocks(2)

    def call(kc, U=2, dl=8, C=2, out_new=FAKE, wsb=1 << 40, cfg=flat):
        return lib.onetrans_append_score(ctypes.byref(cfg), b, ctypes.byref(kc), FAKE, U, dl, out_new, FAKE, C,
                                         FAKE, FAKE, wsb, None)

    kc = _cache(lens=(120, 120))
    assert call(kc, dl=33) == L.ERR_UNSUPPORTED
    assert call(kc, C=3) == L.ERR_UNSUPPORTED                 # 3 x 16 NS rows > 32
    assert call(_cache(lens=(120, 100))) == L.ERR_UNSUPPORTED  # pyramided
    pruned = _cache(lens=(120, 120))
    pruned.q_last = 50
    assert call(pruned) == L.ERR_UNSUPPORTED
    assert call(kc, out_new=None) == L.ERR_INVALID_ARG
    assert call(kc, out_new=FAKE + 4) == L.ERR_ALIGNMENT
    assert call(kc, dl=0) == L.ERR_SHAPE
    assert call(kc, U=3) == L.ERR_SHAPE                       # more users than the cache holds
    assert call(_cache(cap=124, lens=(120, 120))) == L.ERR_CACHE_CAPACITY
    need = lib.onetrans_workspace_bytes(ctypes.byref(flat), L.OP_APPEND_SCORE, 2, 0, 2, 8)
    parts = (lib.onetrans_workspace_bytes(ctypes.byref(flat), L.OP_APPEND, 2, 0, 0, 8)
             + lib.onetrans_workspace_bytes(ctypes.byref(flat), L.OP_SCORE, 2, 0, 2, 0))
    assert parts <= need < parts + 256
    assert call(kc, wsb=need - 1) == L.ERR_WORKSPACE
    assert list(kc._keep) == [120, 120]
    rk = _ragged_cache((100, 195))
    assert call(rk) == L.ERR_CACHE_CAPACITY                   # 195 + 8 > 200
    assert list(rk._keep_ul) == [100, 195]

def _ragged_cache(user_len, n_users=2, cap=200, lens=(120, 120)):
    kc = _cache(n_users, cap, lens)
    ul = (ctypes.c_int * len(user_len))(*user_len)
    kc.user_len = ul
    kc._keep_ul = ul
    return kc


def test_ragged_user_validation_errors():
    """Ragged users (per-user cached lengths): every check returns before any HIP call."""
    lib = L.lib()
    flat = _cfg(sq=(120, 120))
    b = _blocks(2)
    # prefill: padding rows are only harmless without pruning; lengths within [0, l_s]
    assert lib.onetrans_prefill_user(ctypes.byref(_cfg()), b, FAKE, 2, 120, ctypes.byref(_ragged_cache((50, 120))),
                                     None, FAKE, 1 << 40, None) == L.ERR_UNSUPPORTED
    assert lib.onetrans_prefill_user(ctypes.byref(flat), b, FAKE, 2, 120, ctypes.byref(_ragged_cache((50, 121))),
                                     None, FAKE, 1 << 40, None) == L.ERR_SHAPE
    assert lib.onetrans_prefill_user(ctypes.byref(flat), b, FAKE, 2, 120, ctypes.byref(_ragged_cache((-1, 7))),
                                     None, FAKE, 1 << 40, None) == L.ERR_SHAPE
    # append: each user's own capacity, lengths within the cache; nothing advanced on error
    kc = _ragged_cache((100, 125), cap=128)
    assert lib.onetrans_append_events(ctypes.byref(flat), b, ctypes.byref(kc), FAKE, 2, 8, None, FAKE, 1 << 40,
                                      None) == L.ERR_CACHE_CAPACITY
    assert list(kc._keep_ul) == [100, 125] and list(kc._keep) == [120, 120]
    assert lib.onetrans_append_events(ctypes.byref(flat), b, ctypes.byref(_ragged_cache((100, 201))), FAKE, 2, 8,
                                      None, FAKE, 1 << 40, None) == L.ERR_SHAPE
    # score: lengths within the cache
    assert lib.onetrans_score_candidates(ctypes.byref(flat), b, ctypes.byref(_ragged_cache((10, 201))), FAKE, 2, 4,
                                         FAKE, FAKE, 1 << 40, None) == L.ERR_SHAPE
    # ragged users need an unpyramided cache (also when only the last block prunes)
    kr = _ragged_cache((100, 110))
    kr.q_last = 60
    assert lib.onetrans_append_events(ctypes.byref(flat), b, ctypes.byref(kr), FAKE, 2, 8, None, FAKE, 1 << 40,
                                      None) == L.ERR_UNSUPPORTED


def _tok_cfg(lens=(15, 15), dims=(64, 128), hid=(128, 64), ns_dim=192, ns_hidden=128, merge=L.MERGE_INTENT):
    n = len(lens)
    arrs = [(ctypes.c_int * n)(*v) for v in (lens, dims, hid)]
    tc = L.TokenizerConfig(n, *arrs, ns_dim, ns_hidden, merge)
    tc._keep = arrs
    return tc


def _mlps(n, base=0x200000):
    m = (L.MlpWeights * n)()
    for i in range(n):
        for j, f in enumerate(L.MLP_FIELDS):
            setattr(m[i], f, base + (i * 4 + j) * 4096)
    return m


def test_tokenize_workspace_bytes():
    lib = L.lib()
    c = _cfg(d=64, H=4, dff=256, lns=4, N=1, sq=(32,), dtype=L.F32)
    al = lambda n: (n + 255) // 256 * 256
    B = 8
    got = lib.onetrans_tokenize_workspace_bytes(ctypes.byref(c), ctypes.byref(_tok_cfg()), B)
    assert got == al(B * 15 * 128 * 4) + al(B * 15 * 64 * 4) + al(B * 128 * 4)
    assert lib.onetrans_tokenize_workspace_bytes(ctypes.byref(c), ctypes.byref(_tok_cfg(dims=(64, 96))), B) == 0
    assert lib.onetrans_tokenize_workspace_bytes(ctypes.byref(c), None, B) == 0
    # timestamp-aware merge: plus one int32 row index per event
    got = lib.onetrans_tokenize_workspace_bytes(ctypes.byref(c), ctypes.byref(_tok_cfg(merge=L.MERGE_TIME)), B)
    assert got == (al(B * 15 * 128 * 4) + al(B * 15 * 64 * 4) + al(B * 128 * 4) + 2 * al(B * 15 * 4))
    assert lib.onetrans_tokenize_workspace_bytes(ctypes.byref(c), ctypes.byref(_tok_cfg(merge=2)), B) == 0
    assert lib.onetrans_tokenize_workspace_bytes(ctypes.byref(c), ctypes.byref(
        _tok_cfg(lens=(4096, 4097), merge=L.MERGE_TIME)), B) == 0      # more than 8192 events per sample
    assert lib.onetrans_tokenize_workspace_bytes(ctypes.byref(c), ctypes.byref(
        _tok_cfg(lens=(0, 0), merge=L.MERGE_TIME)), B) == 0            # no S rows at all


def test_tokenize_validation_errors():
    """Every check returns before any HIP call."""
    lib = L.lib()
    c = _cfg(d=64, H=4, dff=256, lns=4, N=1, sq=(32,), dtype=L.BF16)
    ev = (ctypes.c_void_p * 2)(FAKE, FAKE)

    def call(tc=None, seq=None, sep=FAKE, ns=True, events=ev, ns_feat=FAKE, B=8, x0=FAKE, ws=FAKE, wsb=1 << 40,
             cfg=c, times=None):
        tc = tc or _tok_cfg()
        seq = seq if seq is not None else _mlps(tc.n_seq)
        nsm = _mlps(1, 0x400000) if ns else None
        return lib.onetrans_tokenize(ctypes.byref(cfg), ctypes.byref(tc), seq, sep, nsm, events, times, ns_feat, B,
                                     x0, ws, wsb, None)

    assert call(sep=None) == L.ERR_INVALID_ARG
    assert call(x0=None) == L.ERR_INVALID_ARG
    assert call(ns=False) == L.ERR_INVALID_ARG                       # l_ns > 0 needs the Auto-Split MLP
    assert call(ns_feat=None) == L.ERR_INVALID_ARG
    assert call(events=(ctypes.c_void_p * 2)(FAKE, None)) == L.ERR_INVALID_ARG
    assert call(x0=FAKE + 8) == L.ERR_ALIGNMENT
    assert call(events=(ctypes.c_void_p * 2)(FAKE, FAKE + 4)) == L.ERR_ALIGNMENT
    bad = _mlps(2)
    bad[1].b2 = FAKE + 2
    assert call(seq=bad) == L.ERR_ALIGNMENT
    bad[1].b2 = None
    assert call(seq=bad) == L.ERR_INVALID_ARG
    assert call(B=0) == L.ERR_SHAPE
    assert call(tc=_tok_cfg(lens=(15, -1))) == L.ERR_SHAPE
    assert call(tc=_tok_cfg(dims=(64, 100))) == L.ERR_UNSUPPORTED    # widths are multiples of 64
    assert call(tc=_tok_cfg(hid=(32, 64))) == L.ERR_UNSUPPORTED
    assert call(tc=_tok_cfg(ns_hidden=130)) == L.ERR_UNSUPPORTED
    assert call(tc=_tok_cfg(lens=(1,) * 8, dims=(64,) * 8, hid=(64,) * 8),
                events=(ctypes.c_void_p * 8)(*[FAKE] * 8)) == L.ERR_UNSUPPORTED   # at most 7 types
    assert call(wsb=64) == L.ERR_WORKSPACE
    assert call(cfg=_cfg(d=64, H=4, dff=256, lns=4, N=1, sq=(32,), dtype=5)) == L.ERR_INVALID_ARG
    # timestamp-aware merge: timestamps required (8-byte aligned) for every non-empty type
    tt = _tok_cfg(merge=L.MERGE_TIME)
    assert call(tc=tt) == L.ERR_INVALID_ARG
    assert call(tc=tt, times=(ctypes.c_void_p * 2)(FAKE, None)) == L.ERR_INVALID_ARG
    assert call(tc=tt, times=(ctypes.c_void_p * 2)(FAKE, FAKE + 4)) == L.ERR_ALIGNMENT
    assert call(tc=tt, times=(ctypes.c_void_p * 2)(FAKE, FAKE), wsb=64) == L.ERR_WORKSPACE
    assert call(tc=_tok_cfg(merge=3)) == L.ERR_INVALID_ARG
    # an empty sequence needs no event buffer
    assert call(tc=_tok_cfg(lens=(15, 0)), events=(ctypes.c_void_p * 2)(FAKE, None), wsb=64) == L.ERR_WORKSPACE


def test_forward_workspace_covers_the_split():
    """Batches of 64+ run as two halves: the workspace holds two half-batch layouts, which also covers
    the single-stream layout of the whole batch."""
    lib = L.lib()
    # 416 query rows per sample: no call of 10+ samples is small enough for split post launches, so
    # every layout below is the same per-sample layout
    c = _cfg(sq=(400, 200))
    one = lambda B: lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_FORWARD, B, 400, 0, 0)
    assert one(64) == 2 * one(32)
    assert one(65) == 2 * one(33)
    assert one(65) >= one(63)
    assert one(128) == 4 * one(32) and one(130) == 4 * one(33)     # four parts from 128 samples
    assert lib.onetrans_set_streams(3) == L.ERR_INVALID_ARG
    assert lib.onetrans_set_streams(4) == L.OK
    assert lib.onetrans_set_streams(0) == L.ERR_INVALID_ARG
    assert lib.onetrans_set_streams(2) == L.OK


def test_status_strings():
    for s in range(-7, 1):
        assert L.status_string(s) not in ("", "unknown status")
    assert L.status_string(-99) == "unknown status"


def test_noalloc_score_validation():
    """The allocation-free Stage II validates like onetrans_score_candidates and refuses a call past
    its static scratch (SCRATCH) on the host, before any HIP call."""
    lib = L.lib()
    c, b = _cfg(), _blocks(2)
    kc = _cache()
    f = lib.onetrans_score_candidates_noalloc
    assert f(ctypes.byref(c), b, ctypes.byref(kc), FAKE, 3, 4, FAKE, None) == L.ERR_SHAPE       # users > cache
    assert f(ctypes.byref(c), b, ctypes.byref(kc), None, 2, 4, FAKE, None) == L.ERR_INVALID_ARG
    assert f(ctypes.byref(c), b, ctypes.byref(kc), FAKE, 2, 4, FAKE + 4, None) == L.ERR_ALIGNMENT
    assert f(ctypes.byref(_cfg(lns=0)), b, ctypes.byref(kc), FAKE, 2, 4, FAKE, None) == L.ERR_SHAPE
    # the scratch holds about 900 candidates of this shape (d = 256, 16 NS tokens): 2 users x 600 do not fit
    assert lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_SCORE, 1, 0, 900, 0) <= L.SCRATCH_BYTES
    assert f(ctypes.byref(c), b, ctypes.byref(kc), FAKE, 2, 600, FAKE, None) == L.ERR_SCRATCH
    # ...and the candidates that fit form one range (the split post launches' partials buffer only
    # exists for small calls and never pushes a smaller call past the scratch)
    need = [lib.onetrans_workspace_bytes(ctypes.byref(c), L.OP_SCORE, 1, 0, n, 0) for n in range(1, 1100, 7)]
    fits = [x <= L.SCRATCH_BYTES for x in need]
    assert fits == sorted(fits, reverse=True)
    assert "scratch" in L.status_string(L.ERR_SCRATCH)


def _grads(N, base=0x200000):
    g = (L.BlockGrads * N)()
    for i in range(N):
        for j, f in enumerate(L.WEIGHT_FIELDS):
            setattr(g[i], f, base + (i * 16 + j) * 4096)
    return g


def _bwd(c, blocks, grads, x0=FAKE, B=2, l_s=120, d_out=FAKE, out=None, dx0=FAKE, ws=FAKE, wsb=1 << 40):
    return L.lib().onetrans_backward(ctypes.byref(c) if c is not None else None, blocks, x0, B, l_s, d_out, out, dx0,
                                     grads, ws, wsb, None)


def test_backward_validation_errors():
    """The training step validates like the forward, plus its gradient pointers, before enqueueing anything."""
    lib = L.lib()
    c, b, g = _cfg(), _blocks(2), _grads(2)
    need = lib.onetrans_backward_workspace_bytes(ctypes.byref(c), 2, 120)
    assert need > 0
    assert lib.onetrans_backward_workspace_bytes(ctypes.byref(c), 2, 60) == 0      # schedule longer than l_s
    assert lib.onetrans_backward_workspace_bytes(None, 2, 120) == 0
    assert _bwd(c, b, g, wsb=need - 1) == L.ERR_WORKSPACE
    assert _bwd(None, b, g) == L.ERR_INVALID_ARG
    assert _bwd(c, None, g) == L.ERR_INVALID_ARG
    assert _bwd(c, b, None) == L.ERR_INVALID_ARG
    assert _bwd(c, b, g, x0=None) == L.ERR_INVALID_ARG
    assert _bwd(c, b, g, d_out=None) == L.ERR_INVALID_ARG
    assert _bwd(c, b, g, ws=None) == L.ERR_INVALID_ARG
    assert _bwd(c, b, g, d_out=FAKE + 4) == L.ERR_ALIGNMENT
    assert _bwd(c, b, g, out=FAKE + 4) == L.ERR_ALIGNMENT
    assert _bwd(c, b, g, dx0=FAKE + 4) == L.ERR_ALIGNMENT
    assert _bwd(c, b, g, B=0) == L.ERR_SHAPE
    assert _bwd(c, b, g, l_s=60) == L.ERR_SHAPE
    assert _bwd(_cfg(d=256, H=4), b, g) == L.ERR_UNSUPPORTED
    ng = _grads(2)
    ng[1].wq = None
    assert _bwd(c, b, ng) == L.ERR_INVALID_ARG
    ng = _grads(2)
    ng[0].b1 = FAKE + 8
    assert _bwd(c, b, ng) == L.ERR_ALIGNMENT
    ng = _grads(2)
    ng[0].norm1_b = None                                                            # optional under RMSNorm
    assert _bwd(c, b, ng, wsb=need - 1) == L.ERR_WORKSPACE
    # launch sizes: rows x heads beyond 2^31, and feature-major tiles beyond 32-bit offsets
    assert _bwd(c, b, g, B=1 << 21) == L.ERR_SHAPE
    assert _bwd(c, b, g, B=1 << 17, wsb=1024) == L.ERR_SHAPE
    assert _bwd(c, b, g, B=1 << 15, wsb=1024) == L.ERR_WORKSPACE


def test_backward_workspace_grows_with_batch():
    lib = L.lib()
    c = _cfg()
    sizes = [lib.onetrans_backward_workspace_bytes(ctypes.byref(c), B, 120) for B in (1, 2, 8, 64)]
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    # the checkpoints alone: block 1's input rows, fp32
    assert sizes[1] - sizes[0] >= (100 + 16) * 256 * 4
