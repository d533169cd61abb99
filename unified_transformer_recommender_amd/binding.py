"""Python binding of the C ABI: the same entry points, torch tensors in and out.

Only argument marshalling happens here. torch provides device memory and the current stream;
every step of the computation runs in the HIP library (libonetrans.so). If the library is
missing, every call raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib as L

DTYPES = {"f32": (L.F32, torch.float32, 4), "bf16": (L.BF16, torch.bfloat16, 2)}
NORMS = {"rms": L.RMSNORM, "layer": L.LAYERNORM}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return s.cuda_stream


class Model:
    """Configuration plus per-block device weights of a OneTrans stack.

    ``blocks`` is a sequence (one per block) of mappings or objects providing the twelve
    parameter tensors named in ``_lib.WEIGHT_FIELDS`` on the device, in the storage dtype,
    contiguous, shaped as documented in include/onetrans.h.
    """

    def __init__(self, *, n_blocks: int, d_model: int, n_heads: int, d_ff: int, l_ns: int, norm: str,
                 norm_eps: float, dtype: str, s_queries: Sequence[int], blocks):
        self.n_blocks, self.d_model, self.n_heads, self.d_ff, self.l_ns = n_blocks, d_model, n_heads, d_ff, l_ns
        self.dtype = dtype
        self.dt_code, self.torch_dtype, self.esz = DTYPES[dtype]
        self.s_queries = tuple(int(q) for q in s_queries)
        self._sq = (ctypes.c_int * n_blocks)(*self.s_queries)
        self.cfg = L.Config(n_blocks, d_model, n_heads, d_ff, l_ns, NORMS[norm], float(norm_eps), self.dt_code,
                            self._sq)
        self._tensors = []
        self.blocks = (L.BlockWeights * n_blocks)()
        for i, b in enumerate(blocks):
            for f in L.WEIGHT_FIELDS:
                t = b[f] if isinstance(b, dict) else getattr(b, f)
                if not (t.is_contiguous() and t.dtype == self.torch_dtype):
                    raise ValueError(f"block {i} {f}: need a contiguous {self.torch_dtype} tensor")
                self._tensors.append(t)
                setattr(self.blocks[i], f, t.data_ptr())
        self.device = self._tensors[0].device

    @classmethod
    def from_host(cls, shape, s_queries: Sequence[int], host_blocks, device="cuda") -> "Model":
        """Upload host weights (numpy float32 arrays, already representable in the storage dtype)."""
        _, tdt, _ = DTYPES[shape.dtype]
        blocks = [{f: torch.from_numpy(getattr(b, f)).to(device=device, dtype=tdt).contiguous()
                   for f in L.WEIGHT_FIELDS} for b in host_blocks]
        return cls(n_blocks=shape.n_blocks, d_model=shape.d_model, n_heads=shape.n_heads, d_ff=shape.d_ff,
                   l_ns=shape.l_ns, norm=shape.norm, norm_eps=shape.norm_eps, dtype=shape.dtype,
                   s_queries=s_queries, blocks=blocks)

    def with_schedule(self, s_queries: Sequence[int]) -> "Model":
        """Same weights, another pyramid schedule."""
        m = Model.__new__(Model)
        m.__dict__.update(self.__dict__)
        m.s_queries = tuple(int(q) for q in s_queries)
        m._sq = (ctypes.c_int * self.n_blocks)(*m.s_queries)
        m.cfg = L.Config(self.cfg.n_blocks, self.cfg.d_model, self.cfg.n_heads, self.cfg.d_ff, self.cfg.l_ns,
                         self.cfg.norm, self.cfg.norm_eps, self.cfg.dtype, m._sq)
        return m

    def workspace_bytes(self, op: int, n_seq: int, l_s: int = 0, n_cand: int = 0, d_l: int = 0) -> int:
        return int(L.lib().onetrans_workspace_bytes(ctypes.byref(self.cfg), op, n_seq, l_s, n_cand, d_l))

    def workspace(self, op: int, n_seq: int, l_s: int = 0, n_cand: int = 0, d_l: int = 0) -> torch.Tensor:
        n = self.workspace_bytes(op, n_seq, l_s, n_cand, d_l)
        if n == 0:
            raise ValueError("invalid configuration for a workspace")
        return torch.empty(n, dtype=torch.uint8, device=self.device)


class KVCache:
    """Caller-owned K/V cache [user][block][head][capacity][d_head] in the storage dtype.

    `user_len` (one int per user) makes the users ragged: user u's valid rows are its first
    user_len[u] rows of every block, and prefill / append / score read (and append advances) these
    per-user lengths. `x_tail=True` allocates the fp32 rows [user][capacity][d] that an append to a
    cache whose pyramid prunes before its last block recomputes from (prefill writes them)."""

    def __init__(self, model: Model, n_users: int, capacity: int, user_len=None, x_tail: bool = False):
        nbytes = int(L.lib().onetrans_kv_cache_bytes(ctypes.byref(model.cfg), n_users, capacity))
        if nbytes == 0:
            raise ValueError("invalid cache shape")
        shape = (n_users, model.n_blocks, model.n_heads, capacity, model.d_model // model.n_heads)
        self.k = torch.empty(shape, dtype=model.torch_dtype, device=model.device)
        self.v = torch.empty(shape, dtype=model.torch_dtype, device=model.device)
        assert self.k.numel() * model.esz == nbytes
        self.layer_len = (ctypes.c_int * model.n_blocks)()
        self.user_len = None
        if user_len is not None:
            if len(user_len) != n_users:
                raise ValueError("user_len needs one length per user")
            self.user_len = (ctypes.c_int * n_users)(*[int(x) for x in user_len])
        self.x_tail = (torch.empty((n_users, capacity, model.d_model), dtype=torch.float32, device=model.device)
                       if x_tail else None)
        self.c = L.KVCache(self.k.data_ptr(), self.v.data_ptr(), n_users, capacity, self.layer_len,
                           self.user_len, 0, _ptr(self.x_tail))

    @property
    def lengths(self):
        return list(self.layer_len)

    @property
    def user_lengths(self):
        return None if self.user_len is None else list(self.user_len)

    @property
    def q_last(self) -> int:
        """S rows the last block keeps (its final rows), as the library maintains it."""
        return int(self.c.q_last) or self.layer_len[len(self.layer_len) - 1]

    def append_window(self) -> int:
        """Rows of the block after the first pruning block (recomputed by an append), or 0."""
        lens = self.lengths + [self.q_last]
        for n in range(len(lens) - 2):
            if lens[n + 1] < lens[n]:
                return lens[n + 1]
        return 0

    def copy_(self, other: "KVCache") -> "KVCache":
        self.k.copy_(other.k)
        self.v.copy_(other.v)
        if self.x_tail is not None and other.x_tail is not None:
            self.x_tail.copy_(other.x_tail)
        for i, n in enumerate(other.layer_len):
            self.layer_len[i] = n
        self.c.q_last = other.c.q_last
        if self.user_len is not None and other.user_len is not None:
            for i, n in enumerate(other.user_len):
                self.user_len[i] = n
        return self


def _check_input(model: Model, x: torch.Tensor, ndim: int, name: str):
    if x.dtype != model.torch_dtype or not x.is_contiguous() or x.dim() != ndim or x.shape[-1] != model.d_model:
        raise ValueError(f"{name}: need a contiguous {model.torch_dtype} tensor of rank {ndim} and width d_model")


def onetrans_forward(model: Model, x0: torch.Tensor, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """x0 [B][L_S + l_ns][d] (storage dtype) -> out [B][q_last + l_ns][d] fp32."""
    _check_input(model, x0, 3, "x0")
    B, T, d = x0.shape
    l_s = T - model.l_ns
    if out is None:
        out = torch.empty((B, model.s_queries[-1] + model.l_ns, d), dtype=torch.float32, device=x0.device)
    if ws is None:
        ws = model.workspace(L.OP_FORWARD, B, l_s)
    st = L.lib().onetrans_forward(ctypes.byref(model.cfg), model.blocks, x0.data_ptr(), B, l_s, out.data_ptr(),
                                  ws.data_ptr(), ws.numel(), _stream(x0.device, stream))
    L.check(st, "onetrans_forward")
    return out


def weight_shapes(model: Model) -> dict:
    """Shape of every per-block parameter (and of its fp32 gradient)."""
    d, f, G = model.d_model, model.d_ff, 1 + model.l_ns
    return {"norm1_g": (d,), "norm1_b": (d,), "norm2_g": (d,), "norm2_b": (d,), "wq": (G, d, d), "wk": (G, d, d),
            "wv": (G, d, d), "wo": (G, d, d), "w1": (G, f, d), "b1": (G, f), "w2": (G, d, f), "b2": (G, d)}


def backward_workspace(model: Model, batch: int, l_s: int) -> torch.Tensor:
    n = int(L.lib().onetrans_backward_workspace_bytes(ctypes.byref(model.cfg), batch, l_s))
    if n == 0:
        raise ValueError("invalid configuration for a backward workspace")
    return torch.empty(n, dtype=torch.uint8, device=model.device)


def grad_buffers(model: Model) -> list:
    """One {field: fp32 tensor} per block, shaped like the parameters."""
    return [{f: torch.empty(s, dtype=torch.float32, device=model.device) for f, s in weight_shapes(model).items()}
            for _ in range(model.n_blocks)]


def onetrans_backward(model: Model, x0: torch.Tensor, d_out: torch.Tensor, want_out: bool = False,
                      want_dx0: bool = True, grads=None, ws: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, dx0: Optional[torch.Tensor] = None, stream=None):
    """One training step's gradients: x0 [B][L_S + l_ns][d] (storage dtype) and d_out [B][q_last + l_ns][d]
    fp32 -> (out or None, dx0 or None, grads), grads a list (one per block) of {field: fp32 tensor}
    summed over the batch. Preallocated `grads` (grad_buffers), `out`, `dx0` and `ws` are overwritten."""
    _check_input(model, x0, 3, "x0")
    B, T, d = x0.shape
    l_s = T - model.l_ns
    R = model.s_queries[-1] + model.l_ns
    if d_out.dtype != torch.float32 or not d_out.is_contiguous() or tuple(d_out.shape) != (B, R, d):
        raise ValueError("d_out: need a contiguous fp32 tensor [B][q_last + l_ns][d]")
    dev = x0.device
    if out is None and want_out:
        out = torch.empty((B, R, d), dtype=torch.float32, device=dev)
    if dx0 is None and want_dx0:
        dx0 = torch.empty((B, T, d), dtype=torch.float32, device=dev)
    if grads is None:
        grads = grad_buffers(model)
    gs = (L.BlockGrads * model.n_blocks)()
    for i, g in enumerate(grads):
        for f in L.WEIGHT_FIELDS:
            setattr(gs[i], f, _ptr(g.get(f)))
    if ws is None:
        ws = backward_workspace(model, B, l_s)
    st = L.lib().onetrans_backward(ctypes.byref(model.cfg), model.blocks, x0.data_ptr(), B, l_s, d_out.data_ptr(),
                                   _ptr(out), _ptr(dx0), gs, ws.data_ptr(), ws.numel(), _stream(dev, stream))
    L.check(st, "onetrans_backward")
    return out, dx0, grads


def onetrans_prefill_user(model: Model, x_s: torch.Tensor, cache: KVCache, out_s: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """Stage I: x_s [U][L_S][d] -> cache K/V per block (and optionally out_s [U][q_last][d] fp32)."""
    _check_input(model, x_s, 3, "x_s")
    U, l_s, _ = x_s.shape
    if ws is None:
        ws = model.workspace(L.OP_PREFILL, U, l_s)
    st = L.lib().onetrans_prefill_user(ctypes.byref(model.cfg), model.blocks, x_s.data_ptr(), U, l_s,
                                       ctypes.byref(cache.c), _ptr(out_s), ws.data_ptr(), ws.numel(),
                                       _stream(x_s.device, stream))
    L.check(st, "onetrans_prefill_user")
    return out_s


def onetrans_score_candidates(model: Model, cache: KVCache, x_ns: torch.Tensor,
                              out_ns: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                              stream=None) -> torch.Tensor:
    """Stage II: x_ns [U][C][l_ns][d] -> out_ns [U][C][l_ns][d] fp32."""
    _check_input(model, x_ns, 4, "x_ns")
    U, C, _, d = x_ns.shape
    if out_ns is None:
        out_ns = torch.empty((U, C, model.l_ns, d), dtype=torch.float32, device=x_ns.device)
    if ws is None:
        ws = model.workspace(L.OP_SCORE, U, n_cand=C)
    st = L.lib().onetrans_score_candidates(ctypes.byref(model.cfg), model.blocks, ctypes.byref(cache.c),
                                           x_ns.data_ptr(), U, C, out_ns.data_ptr(), ws.data_ptr(), ws.numel(),
                                           _stream(x_ns.device, stream))
    L.check(st, "onetrans_score_candidates")
    return out_ns


def onetrans_score_candidates_noalloc(model: Model, cache: KVCache, x_ns: torch.Tensor, out_ns: torch.Tensor,
                                      stream=None) -> torch.Tensor:
    """Stage II without a workspace argument (the library's static device scratch): x_ns [U][C][l_ns][d]
    -> out_ns [U][C][l_ns][d] fp32, both given by the caller; nothing is allocated here either."""
    _check_input(model, x_ns, 4, "x_ns")
    U, C, _, d = x_ns.shape
    st = L.lib().onetrans_score_candidates_noalloc(ctypes.byref(model.cfg), model.blocks, ctypes.byref(cache.c),
                                                   x_ns.data_ptr(), U, C, out_ns.data_ptr(),
                                                   _stream(x_ns.device, stream))
    L.check(st, "onetrans_score_candidates_noalloc")
    return out_ns


def onetrans_append_events(model: Model, cache: KVCache, x_new: torch.Tensor,
                           out_new: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                           stream=None) -> Optional[torch.Tensor]:
    """Cross-request append: x_new [U][dL][d] -> cache extended by dL rows per block (+ out_new fp32,
    [U][min(dL, q_last after the append)][d]: the final rows of the new events)."""
    _check_input(model, x_new, 3, "x_new")
    U, dl, _ = x_new.shape
    if ws is None:
        ws = model.workspace(L.OP_APPEND, U, l_s=cache.append_window(), d_l=dl)
    st = L.lib().onetrans_append_events(ctypes.byref(model.cfg), model.blocks, ctypes.byref(cache.c),
                                        x_new.data_ptr(), U, dl, _ptr(out_new), ws.data_ptr(), ws.numel(),
                                        _stream(x_new.device, stream))
    L.check(st, "onetrans_append_events")
    return out_new



def onetrans_append_score(model: Model, cache: KVCache, x_new: torch.Tensor, x_ns: torch.Tensor,
                          out_new: Optional[torch.Tensor] = None, out_ns: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None, stream=None):
    """A cross-request append then Stage II for the same users in one call: x_new [U][dL][d] and
    x_ns [U][C][l_ns][d] -> (out_new [U][dL][d], out_ns [U][C][l_ns][d]) fp32; the cache is extended
    by dL rows per block as onetrans_append_events does."""
    _check_input(model, x_new, 3, "x_new")
    _check_input(model, x_ns, 4, "x_ns")
    U, dl, d = x_new.shape
    C = x_ns.shape[1]
    if out_new is None:
        out_new = torch.empty((U, dl, d), dtype=torch.float32, device=x_new.device)
    if out_ns is None:
        out_ns = torch.empty((U, C, model.l_ns, d), dtype=torch.float32, device=x_ns.device)
    if ws is None:
        ws = model.workspace(L.OP_APPEND_SCORE, U, n_cand=C, d_l=dl)
    st = L.lib().onetrans_append_score(ctypes.byref(model.cfg), model.blocks, ctypes.byref(cache.c),
                                       x_new.data_ptr(), U, dl, out_new.data_ptr(), x_ns.data_ptr(), C,
                                       out_ns.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x_new.device, stream))
    L.check(st, "onetrans_append_score")
    return out_new, out_ns

class Tokenizer:
    """Device weights of the tokenizers ahead of block 1 for one model (see onetrans_tokenize).

    ``seq_mlps``: one mapping per behaviour type (intent order) with w1 [hidden][D_i], b1 [hidden],
    w2 [d][hidden], b2 [d]; ``seq_vec`` [n_seq][d]: the [SEP] rows (merge "intent") or the
    behaviour-type embeddings (merge "time"); ``ns_mlp``: the Auto-Split MLP (w1 [hidden][ns_dim],
    b1, w2 [l_ns * d][hidden], b2) or None when l_ns = 0. All contiguous, storage dtype, on device.
    """

    def __init__(self, model: Model, seq_lens: Sequence[int], seq_mlps, seq_vec: torch.Tensor, ns_mlp=None,
                 merge: str = "intent"):
        self.model = model
        self.seq_lens = tuple(int(v) for v in seq_lens)
        n = len(self.seq_lens)
        if len(seq_mlps) != n:
            raise ValueError("one MLP per behaviour type")
        self.merge = merge
        merge_code = {"intent": L.MERGE_INTENT, "time": L.MERGE_TIME}[merge]
        self._tensors = [seq_vec]
        self._mlps = (L.MlpWeights * n)()
        dims, hidden = [], []
        for i, p in enumerate(seq_mlps):
            self._fill(self._mlps[i], p)
            hidden.append(int(p["w1"].shape[0]))
            dims.append(int(p["w1"].shape[1]))
        self._ns = None
        ns_dim = ns_hidden = 0
        if ns_mlp is not None:
            self._ns = L.MlpWeights()
            self._fill(self._ns, ns_mlp)
            ns_hidden, ns_dim = int(ns_mlp["w1"].shape[0]), int(ns_mlp["w1"].shape[1])
        self.seq_dims, self.seq_hidden, self.ns_dim = tuple(dims), tuple(hidden), ns_dim
        self._len = (ctypes.c_int * n)(*self.seq_lens)
        self._dim = (ctypes.c_int * n)(*dims)
        self._hid = (ctypes.c_int * n)(*hidden)
        self.tc = L.TokenizerConfig(n, self._len, self._dim, self._hid, ns_dim, ns_hidden, merge_code)
        self.seq_vec = seq_vec
        self.l_s = sum(self.seq_lens) + (n if merge == "intent" else 0)

    def _fill(self, c, p):
        for f in L.MLP_FIELDS:
            t = p[f]
            if not (t.is_contiguous() and t.dtype == self.model.torch_dtype):
                raise ValueError(f"tokenizer {f}: need a contiguous {self.model.torch_dtype} tensor")
            self._tensors.append(t)
            setattr(c, f, t.data_ptr())

    def workspace(self, batch: int) -> torch.Tensor:
        n = int(L.lib().onetrans_tokenize_workspace_bytes(ctypes.byref(self.model.cfg), ctypes.byref(self.tc), batch))
        if n == 0:
            raise ValueError("invalid tokenizer configuration")
        return torch.empty(n, dtype=torch.uint8, device=self.model.device)


def onetrans_tokenize(tok: Tokenizer, events: Sequence[torch.Tensor], ns_feat: Optional[torch.Tensor],
                      x0: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                      stream=None, times: Optional[Sequence[torch.Tensor]] = None) -> torch.Tensor:
    """events[i] [B][L_i][D_i], ns_feat [B][ns_dim] (times[i] int64 [B][L_i] for the time merge)
    -> X(0) [B][L_S + l_ns][d] (storage dtype)."""
    m = tok.model
    B = int(ns_feat.shape[0]) if ns_feat is not None else int(events[0].shape[0])
    for i, e in enumerate(events):
        if e.dtype != m.torch_dtype or not e.is_contiguous() or tuple(e.shape) != (B, tok.seq_lens[i], tok.seq_dims[i]):
            raise ValueError(f"events[{i}]: need a contiguous {m.torch_dtype} tensor [B][L_i][D_i]")
    if ns_feat is not None and (ns_feat.dtype != m.torch_dtype or not ns_feat.is_contiguous()):
        raise ValueError(f"ns_feat: need a contiguous {m.torch_dtype} tensor")
    dev = m.device
    if x0 is None:
        x0 = torch.empty((B, tok.l_s + m.l_ns, m.d_model), dtype=m.torch_dtype, device=dev)
    if ws is None:
        ws = tok.workspace(B)
    ev = (ctypes.c_void_p * len(events))(*[e.data_ptr() for e in events])
    tm = None
    if tok.merge == "time":
        if times is None or len(times) != len(events):
            raise ValueError("the time merge needs one int64 [B][L_i] timestamp tensor per behaviour type")
        for i, t in enumerate(times):
            if t.dtype != torch.int64 or not t.is_contiguous() or tuple(t.shape) != (B, tok.seq_lens[i]):
                raise ValueError(f"times[{i}]: need a contiguous int64 tensor [B][L_i]")
        tm = (ctypes.c_void_p * len(times))(*[t.data_ptr() for t in times])
    st = L.lib().onetrans_tokenize(ctypes.byref(m.cfg), ctypes.byref(tok.tc), tok._mlps, tok.seq_vec.data_ptr(),
                                   ctypes.byref(tok._ns) if tok._ns is not None else None, ev, tm, _ptr(ns_feat), B,
                                   x0.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev, stream))
    L.check(st, "onetrans_tokenize")
    return x0


def set_streams(n: int) -> None:
    """Streams of the batched calls: 2 (default) splits a forward of 64+ samples and an append over 16+
    users into two halves on two streams; 1 does not."""
    L.check(L.lib().onetrans_set_streams(int(n)), "onetrans_set_streams")


def timing_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with hipEvents on its stream (tracing aid)."""
    L.check(L.lib().onetrans_timing_enable(1 if on else 0), "onetrans_timing_enable")


def timing_read() -> dict:
    """{class: (total device ms, launches)} accumulated since the last read."""
    n = len(L.KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_longlong * n)()
    L.check(L.lib().onetrans_timing_read(ms, cnt), "onetrans_timing_read")
    return {k: (ms[i], int(cnt[i])) for i, k in enumerate(L.KERNEL_CLASSES)}
