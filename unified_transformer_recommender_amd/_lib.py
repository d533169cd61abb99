"""ctypes declarations of the C ABI in include/onetrans.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_size_t, c_void_p

# The in-tree build; ONETRANS_LIB names another build of the same sources (the host-sanitized
# library of the CPU tests).
LIB_PATH = os.environ.get("ONETRANS_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libonetrans.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_SHAPE = -2
ERR_UNSUPPORTED = -3
ERR_WORKSPACE = -4
ERR_CACHE_CAPACITY = -5
ERR_ALIGNMENT = -6
ERR_HIP = -7
ERR_SCRATCH = -8
SCRATCH_BYTES = 64 << 20     # ONETRANS_SCRATCH_BYTES

F32, BF16 = 0, 1
RMSNORM, LAYERNORM = 0, 1
OP_FORWARD, OP_PREFILL, OP_SCORE, OP_APPEND, OP_APPEND_SCORE = 0, 1, 2, 3, 4
KERNEL_CLASSES = ("qkv", "attn", "post", "lin", "merge", "bwd_gemm", "bwd_attn", "bwd_rows")
MERGE_INTENT, MERGE_TIME = 0, 1

WEIGHT_FIELDS = ("norm1_g", "norm1_b", "norm2_g", "norm2_b", "wq", "wk", "wv", "wo", "w1", "b1", "w2", "b2")


class Config(ctypes.Structure):
    _fields_ = [("n_blocks", c_int), ("d_model", c_int), ("n_heads", c_int), ("d_ff", c_int), ("l_ns", c_int),
                ("norm", c_int), ("norm_eps", c_float), ("dtype", c_int), ("s_queries", POINTER(c_int))]


class BlockWeights(ctypes.Structure):
    _fields_ = [(f, c_void_p) for f in WEIGHT_FIELDS]


class BlockGrads(ctypes.Structure):
    _fields_ = [(f, c_void_p) for f in WEIGHT_FIELDS]


class KVCache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("n_users", c_int), ("capacity", c_int),
                ("layer_len", POINTER(c_int)), ("user_len", POINTER(c_int)), ("q_last", c_int),
                ("x_tail", c_void_p)]


class TokenizerConfig(ctypes.Structure):
    _fields_ = [("n_seq", c_int), ("seq_len", POINTER(c_int)), ("seq_dim", POINTER(c_int)),
                ("seq_hidden", POINTER(c_int)), ("ns_dim", c_int), ("ns_hidden", c_int), ("merge", c_int)]


MLP_FIELDS = ("w1", "b1", "w2", "b2")


class MlpWeights(ctypes.Structure):
    _fields_ = [(f, c_void_p) for f in MLP_FIELDS]


SIGNATURES = {
    "onetrans_workspace_bytes": (c_size_t, [POINTER(Config), c_int, c_int, c_int, c_int, c_int]),
    "onetrans_kv_cache_bytes": (c_size_t, [POINTER(Config), c_int, c_int]),
    "onetrans_forward": (c_int, [POINTER(Config), POINTER(BlockWeights), c_void_p, c_int, c_int, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "onetrans_prefill_user": (c_int, [POINTER(Config), POINTER(BlockWeights), c_void_p, c_int, c_int,
                                      POINTER(KVCache), c_void_p, c_void_p, c_size_t, c_void_p]),
    "onetrans_score_candidates": (c_int, [POINTER(Config), POINTER(BlockWeights), POINTER(KVCache), c_void_p,
                                          c_int, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "onetrans_score_candidates_noalloc": (c_int, [POINTER(Config), POINTER(BlockWeights), POINTER(KVCache),
                                                  c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "onetrans_append_events": (c_int, [POINTER(Config), POINTER(BlockWeights), POINTER(KVCache), c_void_p,
                                       c_int, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "onetrans_append_score": (c_int, [POINTER(Config), POINTER(BlockWeights), POINTER(KVCache), c_void_p, c_int,
                                      c_int, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "onetrans_tokenize_workspace_bytes": (c_size_t, [POINTER(Config), POINTER(TokenizerConfig), c_int]),
    "onetrans_tokenize": (c_int, [POINTER(Config), POINTER(TokenizerConfig), POINTER(MlpWeights), c_void_p,
                                  POINTER(MlpWeights), POINTER(c_void_p), POINTER(c_void_p), c_void_p, c_int,
                                  c_void_p, c_void_p, c_size_t, c_void_p]),
    "onetrans_backward_workspace_bytes": (c_size_t, [POINTER(Config), c_int, c_int]),
    "onetrans_backward": (c_int, [POINTER(Config), POINTER(BlockWeights), c_void_p, c_int, c_int, c_void_p,
                                  c_void_p, c_void_p, POINTER(BlockGrads), c_void_p, c_size_t, c_void_p]),
    "onetrans_set_streams": (c_int, [c_int]),
    "onetrans_timing_enable": (c_int, [c_int]),
    "onetrans_timing_read": (c_int, [POINTER(ctypes.c_double), POINTER(ctypes.c_longlong)]),
    "onetrans_status_string": (c_char_p, [c_int]),
    "onetrans_version": (c_char_p, []),
}

_LIB = None


class OneTransError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """The loaded HIP library. Raises if it has not been built: there is no other code path."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library missing: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().onetrans_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != OK:
        raise OneTransError(status, where)
