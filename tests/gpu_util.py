"""Shared helpers of the GPU parity tests (inputs from synth, expectations from the oracle)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from unified_transformer_recommender_amd import binding as ob

TOL = {"f32": 1e-4, "bf16": 2e-2}     # max |gpu - oracle| / rms(oracle), per compared tensor

_WEIGHTS = {}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref * ref)))


def weights(m):
    key = (m.name, m.dtype, m.n_blocks, m.d_model, m.l_ns, m.norm, m.weight_seed)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        _WEIGHTS[key] = synth.make_weights(m)
    return _WEIGHTS[key]


def model(w, s_queries=None, device="cuda"):
    return ob.Model.from_host(w.model, s_queries or w.s_queries, weights(w.model), device=device)


def dev(x, mdl):
    return torch.from_numpy(np.ascontiguousarray(x)).to(mdl.device, dtype=mdl.torch_dtype)


def cache_to_host(cache, user, n_blocks, lens):
    """[(k [s_n][d], v [s_n][d]) per block] of one user from the device cache (head-major)."""
    out = []
    k = cache.k[user].float().cpu().numpy()     # [N][H][cap][dh]
    v = cache.v[user].float().cpu().numpy()
    for n in range(n_blocks):
        s = lens[n]
        out.append((k[n, :, :s].transpose(1, 0, 2).reshape(s, -1), v[n, :, :s].transpose(1, 0, 2).reshape(s, -1)))
    return out
