"""Independent references used to pin the oracle (test helpers, CPU only).

Nothing here calls the oracle. Each helper builds the same quantity from library
routines (PyTorch's own layers) or from a closed form, so that a slip in the
oracle (a dropped term, a wrong index or mask) shows up as a mismatch.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(np.asarray(a, np.float64))


def torch_encoder_layer_stack(x0: np.ndarray, weights, m) -> np.ndarray:
    """Textbook pre-LayerNorm causal Transformer from ``torch.nn.TransformerEncoderLayer``.

    Uses group-0 (shared) parameters for every row: the OneTrans block reduces to
    this when every W_NS,j equals W_S and no pyramid is applied.
    """
    assert m.norm == "layer"
    T = x0.shape[-2]
    x = _t(x0)[None]
    mask = torch.nn.Transformer.generate_square_subsequent_mask(T, dtype=torch.float64)
    for p in weights:
        layer = torch.nn.TransformerEncoderLayer(
            m.d_model, m.n_heads, m.d_ff, dropout=0.0, activation="gelu", layer_norm_eps=m.norm_eps,
            batch_first=True, norm_first=True, dtype=torch.float64)
        with torch.no_grad():
            layer.self_attn.in_proj_weight.copy_(_t(np.concatenate([p.wq[0], p.wk[0], p.wv[0]])))
            layer.self_attn.in_proj_bias.zero_()
            layer.self_attn.out_proj.weight.copy_(_t(p.wo[0]))
            layer.self_attn.out_proj.bias.zero_()
            layer.linear1.weight.copy_(_t(p.w1[0]))
            layer.linear1.bias.copy_(_t(p.b1[0]))
            layer.linear2.weight.copy_(_t(p.w2[0]))
            layer.linear2.bias.copy_(_t(p.b2[0]))
            layer.norm1.weight.copy_(_t(p.norm1_g))
            layer.norm1.bias.copy_(_t(p.norm1_b))
            layer.norm2.weight.copy_(_t(p.norm2_g))
            layer.norm2.bias.copy_(_t(p.norm2_b))
        layer.train(False)
        with torch.no_grad():
            x = layer(x, src_mask=mask, is_causal=True)
    return x[0].numpy()


def _functional_stack(x, params, m, s_queries):
    """The mixed-parameter stack in torch over tensors (x [L_S + l_ns][d], params[n][field])."""
    d, H = m.d_model, m.n_heads
    dh = d // H
    s = x.shape[0] - m.l_ns

    def nrm(z, g, b):
        if m.norm == "rms":
            return F.rms_norm(z, (d,), weight=g, eps=m.norm_eps)
        return F.layer_norm(z, (d,), weight=g, bias=b, eps=m.norm_eps)

    def lin(z, W, rows, b=None):
        out = []
        for i, t in enumerate(rows):
            gi = 0 if t < s else 1 + (t - s)
            out.append(F.linear(z[i:i + 1], W[gi], None if b is None else b[gi]))
        return torch.cat(out)

    for n, p in enumerate(params):
        T = x.shape[0]
        q_keep = s_queries[n]
        rows = list(range(T))
        tail = list(range(s - q_keep, T))
        xh = nrm(x, p["norm1_g"], p["norm1_b"])
        k = lin(xh, p["wk"], rows)
        v = lin(xh, p["wv"], rows)
        q = lin(xh[tail], p["wq"], tail)
        R = len(tail)
        mask = torch.arange(T)[None, :] <= torch.tensor(tail)[:, None]
        o = F.scaled_dot_product_attention(q.view(R, H, dh).transpose(0, 1), k.view(T, H, dh).transpose(0, 1),
                                           v.view(T, H, dh).transpose(0, 1), attn_mask=mask)
        o = o.transpose(0, 1).reshape(R, d)
        y = x[tail] + lin(o, p["wo"], tail)
        hid = F.gelu(lin(nrm(y, p["norm2_g"], p["norm2_b"]), p["w1"], tail, p["b1"]), approximate="none")
        x = y + lin(hid, p["w2"], tail, p["b2"])
        s = q_keep
    return x


_FIELDS = ("norm1_g", "norm1_b", "norm2_g", "norm2_b", "wq", "wk", "wv", "wo", "w1", "b1", "w2", "b2")


def torch_functional_forward(x0: np.ndarray, weights, m, s_queries) -> np.ndarray:
    """Mixed-parameter stack written with torch library calls (F.rms_norm / F.layer_norm,
    F.linear, F.scaled_dot_product_attention with an explicit bottom-right causal mask, F.gelu).

    Row t of a block with s S rows uses parameter set 0 if t < s, else 1 + (t - s).
    """
    params = [{f: _t(getattr(p, f)) for f in _FIELDS} for p in weights]
    with torch.no_grad():
        return _functional_stack(_t(x0), params, m, s_queries).numpy()


def torch_functional_grads(x0: np.ndarray, weights, m, s_queries, d_out: np.ndarray):
    """torch.autograd (fp64) gradients of L = sum(d_out * stack(x0)) through the same torch-functional
    stack: (dL/dx0, [{field: dL/dparam} per block])."""
    x = _t(x0).requires_grad_(True)
    params = [{f: _t(getattr(p, f)).requires_grad_(True) for f in _FIELDS} for p in weights]
    out = _functional_stack(x, params, m, s_queries)
    (out * _t(d_out)).sum().backward()
    grads = [{f: (p[f].grad.numpy() if p[f].grad is not None else np.zeros(p[f].shape)) for f in _FIELDS}
             for p in params]
    return x.grad.numpy(), grads


def gelu_scalar(z: float) -> float:
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))
