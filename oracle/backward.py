"""fp64 gradients of the attention forward, for the backward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The backward pass is not on the pages: they stop at the forward of the aiml.sh
page "Speed up long contexts with FlashAttention" (lab.py, standard_attention
and tiled_flash_attention).  What is differentiated here is exactly that
forward, per (batch, head):

    S = scale * Q K^T, with S_ij = -inf where the key is hidden (causal: j > i)
    P = softmax of each row of S
    O = P V

and the gradients, for an upstream gradient dO of O, are the chain rule
written out in plain matrix form:

    dV = P^T dO
    dP = dO V^T
    delta_i = sum_j P_ij dP_ij  (= dO_i . O_i)
    dS = P * (dP - delta)       (the softmax Jacobian applied row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

Nothing is blocked, fused or reordered: each line is one numpy expression.
The tests pin this module to central finite differences of the C forward
oracle (``dense``), which shares none of these formulas, and to invariants
that a dropped term, a wrong sign or a transposed operand would break.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x: np.ndarray, dtype: str | None) -> np.ndarray:
    """Storage -> float64: bf16 bit patterns (uint16, dtype="bf16") or a float array."""
    x = np.asarray(x)
    if dtype == "bf16" or x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _head_probabilities(qh: np.ndarray, kh: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    """P of one head: softmax rows of scale * Q K^T with hidden keys at -inf."""
    s = scale * (qh @ kh.T)
    if causal:
        n = s.shape[0]
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_backward(q, k, v, do, causal: bool = True, scale: float | None = None,
                       dtype: str | None = None, bh_idx=None):
    """fp64 (dq, dk, dv) of the forward above, each ``[n_bh, S, D]``.

    ``q, k, v, do``: ``[B, H, S, D]`` arrays (float, or uint16 bfloat16 bit
    patterns with ``dtype="bf16"``).  ``scale`` defaults to ``1/sqrt(D)``.
    ``bh_idx`` selects flattened ``b*H+h`` heads (default: all).
    """
    q, k, v, do = (_as_f64(t, dtype) for t in (q, k, v, do))
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    flat = [t.reshape(B * H, S, D) for t in (q, k, v, do)]
    heads = range(B * H) if bh_idx is None else list(bh_idx)
    dq = np.empty((len(heads), S, D)); dk = np.empty_like(dq); dv = np.empty_like(dq)
    for n, bh in enumerate(heads):
        qh, kh, vh, doh = (t[bh] for t in flat)
        p = _head_probabilities(qh, kh, causal, scale)
        dv[n] = p.T @ doh
        dp = doh @ vh.T
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[n] = scale * (ds @ kh)
        dk[n] = scale * (ds.T @ qh)
    return dq, dk, dv


def row_deltas(o, do, dtype: str | None = None):
    """delta_i = dO_i . O_i per row, ``[B*H, S]`` fp64, from the given O and dO."""
    o, do = _as_f64(o, dtype), _as_f64(do, dtype)
    B, H, S, D = o.shape
    return (o * do).sum(axis=-1).reshape(B * H, S)
