"""The tiled online-softmax method as a plain fp64 loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the method of the aiml.sh page "Speed up long contexts with
FlashAttention" (lab.py, tiled_flash_attention), written from its description
rather than from its listing.  Its steps, in the page's order:

1. Split the queries into row blocks of ``block_q``.  Each block keeps, per
   row, a running maximum (starting at -inf), a running sum (starting at 0) and
   an output accumulator (starting at 0).
2. Stream key/value blocks of ``block_kv`` in increasing order.  Under the
   causal rule a key block that starts at or after the end of the query block
   lies wholly above the diagonal and ends the stream for that query block.
   The last blocks of either kind may be short (``min`` with the length).
3. For every row of the query block, keep only the keys of the current block
   that the row may see (key index <= row index when causal).  A row with none
   is left untouched.  Otherwise:
   score = (q . k) * scale for the kept keys; new max = max(running max, block
   max); alpha = exp(old max - new max), taken as 0 while the old max is still
   -inf; p = exp(score - new max); running sum = running sum * alpha + sum(p);
   accumulator = accumulator * alpha + sum_j p_j v_j.
4. After the last key block, divide each accumulator row by its running sum.

The log-sum-exp (running max + log(running sum)) is not on the pages; it is
returned because the GPU kernel writes it and the merge of partial results
across sequence shards needs it.

``rescale_previous_acc=False`` leaves the accumulator unscaled by alpha, as the
page's switch of that name does: a deliberately wrong variant, used only as a
negative control that the parity checks must reject.
"""
from __future__ import annotations

import math

import numpy as np


def _one_head(q, k, v, block_q, block_kv, causal, scale, rescale_previous_acc):
    n, d = q.shape
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    tiles_visited = 0
    for q_start in range(0, n, block_q):
        q_end = min(q_start + block_q, n)
        rows = q_end - q_start
        run_max = np.full(rows, -math.inf)
        run_sum = np.zeros(rows)
        acc = np.zeros((rows, d))
        for kv_start in range(0, n, block_kv):
            if causal and kv_start >= q_end:
                break
            kv_end = min(kv_start + block_kv, n)
            tiles_visited += 1
            for r in range(rows):
                i = q_start + r
                last = min(kv_end, i + 1) if causal else kv_end
                if last <= kv_start:
                    continue  # no key of this block is visible to row i
                keys = slice(kv_start, last)
                s = (k[keys] @ q[i]) * scale
                new_max = max(run_max[r], float(s.max()))
                alpha = math.exp(run_max[r] - new_max) if run_max[r] > -math.inf else 0.0
                p = np.exp(s - new_max)
                run_sum[r] = run_sum[r] * alpha + p.sum()
                carry = alpha if rescale_previous_acc else 1.0
                acc[r] = acc[r] * carry + p @ v[keys]
                run_max[r] = new_max
        out[q_start:q_end] = acc / run_sum[:, None]
        lse[q_start:q_end] = run_max + np.log(run_sum)
    meta = {
        "materialized_nxn_elements": 0,
        "max_sram_score_tile_elements": block_q * block_kv,
        "tiles_visited": tiles_visited,
    }
    return out, lse, meta


def tiled_attention(q, k, v, block_q: int = 16, block_kv: int = 16, causal: bool = True,
                    scale: float | None = None, rescale_previous_acc: bool = True):
    """fp64 tiled online-softmax attention.

    ``q, k, v``: float arrays ``[S, D]`` or ``[B, H, S, D]`` (widened to float64).
    Returns ``(o, lse, meta)``; ``meta["tiles_visited"]`` sums over heads.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if block_q < 1 or block_kv < 1:
        raise ValueError("block sizes must be positive")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if q.ndim == 2:
        return _one_head(q, k, v, block_q, block_kv, causal, scale, rescale_previous_acc)
    B, H, S, D = q.shape
    o = np.empty((B, H, S, D))
    lse = np.empty((B, H, S))
    tiles = 0
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], meta = _one_head(q[b, h], k[b, h], v[b, h], block_q, block_kv,
                                                 causal, scale, rescale_previous_acc)
            tiles += meta["tiles_visited"]
    meta = dict(meta, tiles_visited=tiles)
    return o, lse, meta
