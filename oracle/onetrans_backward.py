"""Plain, slow fp64 CPU backward of the OneTrans block stack (gradients of a training step).

TEST INFRASTRUCTURE. Only tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the HIP product path shares no code with it.

Sources: fun-rec-mdbook (English), chapter 7.5 "OneTrans", section 7.5.1 (the block: pre-norm,
mixed Q/K/V, causal attention, mixed FFN) and 7.5.2 (Pyramid Stack); the closing paragraph of
7.5.3 and the paper-daily deep reading's system-efficiency table name the training recipe this
backward serves: mixed precision with activation recomputation.

What is computed, per sample: for a loss L whose gradient with respect to the stack's final rows
is d_out, the gradients dL/dX(0) and dL/dtheta for every parameter of every block, each weight set
(the shared S set 0 and NS set 1 + j) separately. The forward of each block is recomputed from its
input rows (activation recomputation: only block inputs are kept), then the chain rule runs
backwards through it:

  X' = Y + W2[w] phi(W1[w] Yh + b1[w]) + b2[w],  Yh = Norm2(Y)     Mixed FFN + pre-norm
  Y  = X[tail] + Wo[w] O                                            attention residual
  O  = softmax_{u <= t}(Q_t . K_u / sqrt(dh)) V_u  per head          causal attention
  Q, K, V = Wq/Wk/Wv[w] Xh,  Xh = Norm1(X)                          mixed Q/K/V + pre-norm

with w = w(t) the row's weight set, and the pyramid keeping only the tail rows as queries
(their gradients flow back to the block's input rows; rows outside the tail only receive
gradient through the keys and values).
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erf

from .onetrans_oracle import block_forward, causal_attention, gelu, mixed_linear, norm, weight_group

F64 = np.float64
FIELDS = ("norm1_g", "norm1_b", "norm2_g", "norm2_b", "wq", "wk", "wv", "wo", "w1", "b1", "w2", "b2")


def zero_grads(p) -> Dict[str, np.ndarray]:
    """A gradient per parameter of one block, shaped like the parameter (fp64 zeros)."""
    return {f: np.zeros(np.shape(getattr(p, f)), F64) for f in FIELDS}


def norm_backward(x: np.ndarray, g: np.ndarray, kind: str, eps: float, dy: np.ndarray
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Rows of y = Norm(x) (RMSNorm x r g, r = 1/sqrt(mean x^2 + eps); LayerNorm (x - mu) r g + b with the
    population variance): returns (dx, dg, db) for the upstream gradient dy. dg and db sum over rows."""
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    g = np.asarray(g, F64)
    d = x.shape[-1]
    if kind == "rms":
        r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
        xhat = x * r
        gy = dy * g
        # d(x_i r)/dx_j = r delta_ij - x_i x_j r^3 / d = r (delta_ij - xhat_i xhat_j / d)
        dx = r * (gy - xhat * np.mean(gy * xhat, axis=-1, keepdims=True))
        return dx, np.sum(dy * xhat, axis=0), np.zeros(d, F64)
    mu = np.mean(x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(np.mean((x - mu) ** 2, axis=-1, keepdims=True) + eps)
    xhat = (x - mu) * r
    gy = dy * g
    dx = r * (gy - np.mean(gy, axis=-1, keepdims=True) - xhat * np.mean(gy * xhat, axis=-1, keepdims=True))
    return dx, np.sum(dy * xhat, axis=0), np.sum(dy, axis=0)


def gelu_derivative(x: np.ndarray) -> np.ndarray:
    """d/dx of 0.5 x (1 + erf(x / sqrt 2)) = Phi(x) + x phi(x)."""
    x = np.asarray(x, F64)
    return 0.5 * (1.0 + erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def mixed_linear_backward(x: np.ndarray, w: np.ndarray, rows: Sequence[int], s: int, dy: np.ndarray,
                          dw: np.ndarray, db: np.ndarray = None) -> np.ndarray:
    """Backward of y_t = W[w(t)] x_t (+ b[w(t)]): returns dx and adds dW[w] (and db[w]) in place."""
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    dx = np.empty_like(x)
    for i, t in enumerate(rows):
        gset = weight_group(t, s)
        W = np.asarray(w[gset], F64)
        dx[i] = W.T @ dy[i]
        dw[gset] += np.outer(dy[i], x[i])
        if db is not None:
            db[gset] += dy[i]
    return dx


def causal_attention_backward(q, k, v, q_pos, k_pos, n_heads, do):
    """Backward of causal_attention: (dq, dk, dv). Per head with scale c = 1/sqrt(dh):
    P = softmax(c Q K^T) over visible keys, dV = P^T dO, dP = dO V^T,
    dS = P (dP - rowsum(dP P)), dQ = c dS K, dK = c dS^T Q."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    do = np.asarray(do, F64)
    d = q.shape[1]
    dh = d // n_heads
    c = 1.0 / math.sqrt(dh)
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        sc = np.where(visible, c * (q[:, sl] @ k[:, sl].T), -np.inf)
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        dv[:, sl] = p.T @ do[:, sl]
        dp = do[:, sl] @ v[:, sl].T
        ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
        dq[:, sl] = c * ds @ k[:, sl]
        dk[:, sl] = c * ds.T @ q[:, sl]
    return dq, dk, dv


def block_backward(x: np.ndarray, s: int, q_keep: int, p, m, d_out: np.ndarray, gr: Dict[str, np.ndarray]
                   ) -> np.ndarray:
    """One block over x = [s S rows; l_ns NS rows] whose output is its tail q_keep S rows + NS rows:
    recompute the block's forward from x, then return dL/dx for the gradient d_out of its output
    rows and add the parameter gradients into gr."""
    x = np.asarray(x, F64)
    T = x.shape[0]
    rows = list(range(T))
    tail = list(range(s - q_keep, T))
    # forward recompute
    xh = norm(x, p.norm1_g, p.norm1_b, m.norm, m.norm_eps)
    k = mixed_linear(xh, p.wk, rows, s)
    v = mixed_linear(xh, p.wv, rows, s)
    q = mixed_linear(xh[tail], p.wq, tail, s)
    o = causal_attention(q, k, v, tail, rows, m.n_heads)
    y = x[tail] + mixed_linear(o, p.wo, tail, s)
    yh = norm(y, p.norm2_g, p.norm2_b, m.norm, m.norm_eps)
    hpre = mixed_linear(yh, p.w1, tail, s, p.b1)
    hid = gelu(hpre)
    # FFN
    d_out = np.asarray(d_out, F64)
    d_hid = mixed_linear_backward(hid, p.w2, tail, s, d_out, gr["w2"], gr["b2"])
    d_hpre = d_hid * gelu_derivative(hpre)
    d_yh = mixed_linear_backward(yh, p.w1, tail, s, d_hpre, gr["w1"], gr["b1"])
    d_y, dg2, db2 = norm_backward(y, p.norm2_g, m.norm, m.norm_eps, d_yh)
    gr["norm2_g"] += dg2
    if m.norm == "layer":
        gr["norm2_b"] += db2
    d_y = d_y + d_out                                          # X' = Y + FFN(Y)
    # attention
    d_o = mixed_linear_backward(o, p.wo, tail, s, d_y, gr["wo"])
    d_q, d_k, d_v = causal_attention_backward(q, k, v, tail, rows, m.n_heads, d_o)
    d_xh = mixed_linear_backward(xh, p.wk, rows, s, d_k, gr["wk"])
    d_xh = d_xh + mixed_linear_backward(xh, p.wv, rows, s, d_v, gr["wv"])
    d_xh[s - q_keep:] += mixed_linear_backward(xh[tail], p.wq, tail, s, d_q, gr["wq"])
    d_x, dg1, db1 = norm_backward(x, p.norm1_g, m.norm, m.norm_eps, d_xh)
    gr["norm1_g"] += dg1
    if m.norm == "layer":
        gr["norm1_b"] += db1
    d_x[s - q_keep:] += d_y                                    # Y = X[tail] + ...
    return d_x


def backward(x0: np.ndarray, weights, m, s_queries: Sequence[int], d_out: np.ndarray
             ) -> Tuple[np.ndarray, List[Dict[str, np.ndarray]]]:
    """Gradients of one sample: (dL/dX(0) [L_S + l_ns][d], per-block parameter gradients) for the
    gradient d_out [q_last + l_ns][d] of the stack's final rows. Only the block inputs are kept from
    the forward pass; each block's internals are recomputed in its backward step."""
    x = np.asarray(x0, F64)
    s = x.shape[0] - m.l_ns
    inputs, ss = [], []
    for n, p in enumerate(weights):
        inputs.append(x)
        ss.append(s)
        x = block_forward(x, s, s_queries[n], p, m)
        s = s_queries[n]
    grads = [zero_grads(p) for p in weights]
    d = np.asarray(d_out, F64)
    for n in range(len(weights) - 1, -1, -1):
        d = block_backward(inputs[n], ss[n], s_queries[n], weights[n], m, d, grads[n])
    return d, grads


def backward_batch(x0: np.ndarray, weights, m, s_queries: Sequence[int], d_out: np.ndarray
                   ) -> Tuple[np.ndarray, List[Dict[str, np.ndarray]]]:
    """Over a batch [B][L_S + l_ns][d]: dX(0) per sample and the parameter gradients summed over samples."""
    dxs, total = [], None
    for b in range(x0.shape[0]):
        dx, g = backward(x0[b], weights, m, s_queries, d_out[b])
        dxs.append(dx)
        total = g if total is None else [{f: a[f] + bb[f] for f in FIELDS} for a, bb in zip(total, g)]
    return np.stack(dxs), total
