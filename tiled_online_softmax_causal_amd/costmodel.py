"""Work, traffic and roofline arithmetic for the attention forward pass (host logic).

Three groups of closed forms live here:

* The algorithmic work used for every reported rate: FLOPs count the two
  matrix products only, 4*B*H*S^2*D, halved under the causal rule -- the
  convention of the chipfoundryservices.com "FlashAttention" reduced-order
  model (outputs.flops_gflop).  Bytes count Q, K, V read once, O written once
  and the fp32 log-sum-exp written once.
* The logical-access model of the aiml.sh page "Speed up long contexts with
  FlashAttention" (lab.py, estimate_hbm_bytes; printed as hbm_traffic_sweep in
  run-output.txt): the dense path moves Q, K, V, O plus a write and a read of
  both N x N matrices per head; the tiled causal path reads Q and writes O
  once and re-reads the K/V prefix once per query block, with no cache reuse.
* The roofline of the chipfoundryservices.com reduced-order model: time is the
  larger of compute time and memory time, the naive path moving the causal
  half of the score matrix twice on top of Q, K, V, O.

The MI355X figures are AMD's published peaks: 2.5 PFLOP/s dense bf16 MFMA and
8 TB/s HBM3E.
"""
from __future__ import annotations

import math

MI355X_BF16_DENSE_PEAK = 2.5e15   # FLOP/s, dense (no structured sparsity)
MI355X_FP32_VECTOR_PEAK = 157.3e12
MI355X_HBM_BW = 8.0e12            # B/s


def attention_flops(B: int, H: int, S: int, D: int, causal: bool = True) -> float:
    """FLOPs of QK^T and PV: 2 products x 2*S*S*D per head, halved when causal."""
    f = 4.0 * B * H * S * S * D
    return f / 2 if causal else f


def algorithmic_bytes(B: int, H: int, S: int, D: int, elem_bytes: int, with_lse: bool = True) -> int:
    """Compulsory HBM bytes: Q, K, V read once, O written once (+ fp32 LSE)."""
    return 4 * B * H * S * D * elem_bytes + (4 * B * H * S if with_lse else 0)


def causal_kv_tiles(S: int, block_q: int, block_kv: int, causal: bool = True) -> int:
    """Key/value tiles visited by one head.

    A query block [q0, q1) visits key blocks starting below q1 when causal
    (all of them otherwise), the rule of lab.py's tiled_flash_attention.
    """
    n_kv = -(-S // block_kv)
    total = 0
    for q0 in range(0, S, block_q):
        q1 = min(q0 + block_q, S)
        total += min(n_kv, -(-q1 // block_kv)) if causal else n_kv
    return total


def executed_mfma_flops(B: int, H: int, S: int, D: int, block_q: int, block_kv: int,
                        causal: bool = True) -> float:
    """FLOPs the matrix cores execute when whole tiles are computed, masked or not."""
    return 4.0 * B * H * causal_kv_tiles(S, block_q, block_kv, causal) * block_q * block_kv * D


# --- the aiml.sh logical-access model -------------------------------------------------

def page_logical_traffic(seq_len: int, num_heads: int = 32, head_dim: int = 128,
                         bytes_per_elem: int = 2, block_q: int = 128) -> dict:
    """Logical bytes of dense vs causal-tiled attention for one layer (no cache reuse)."""
    qkvo = 4 * num_heads * seq_len * head_dim * bytes_per_elem
    nxn = 4 * num_heads * seq_len * seq_len * bytes_per_elem  # write + read of S and of P
    kv_rows = sum(min(seq_len, start + block_q) for start in range(0, seq_len, block_q))
    tiled = (2 * num_heads * seq_len * head_dim + 2 * num_heads * kv_rows * head_dim) * bytes_per_elem
    return {
        "qkvo_bytes": qkvo,
        "nxn_bytes": nxn,
        "standard_total_bytes": qkvo + nxn,
        "tiled_logical_bytes": tiled,
        "num_q_blocks": math.ceil(seq_len / block_q),
    }


# --- the chipfoundryservices.com reduced-order roofline ---------------------------------

def page_roofline(batch: int, heads: int, seq: float, head_dim: int, elem_bytes: float,
                  peak_flops: float, hbm_bw: float, causal: bool = True, sram_bytes: float = None,
                  block: int = None) -> dict:
    """Roofline of naive (score matrix through HBM) vs tiled attention."""
    half = 0.5 if causal else 1.0
    flops = 4.0 * batch * heads * seq * seq * head_dim * half
    fa_bytes = 4.0 * batch * heads * seq * head_dim * elem_bytes
    scores_bytes = batch * heads * seq * seq * elem_bytes * half
    naive_bytes = fa_bytes + 2.0 * scores_bytes
    t_compute = flops / peak_flops
    fa_time = max(t_compute, fa_bytes / hbm_bw)
    naive_time = max(t_compute, naive_bytes / hbm_bw)
    out = {
        "flops": flops,
        "scores_bytes": scores_bytes,
        "fa_bytes": fa_bytes,
        "naive_bytes": naive_bytes,
        "hbm_reduction": naive_bytes / fa_bytes,
        "machine_balance": peak_flops / hbm_bw,
        "ai_fa": flops / fa_bytes,
        "ai_naive": flops / naive_bytes,
        "fa_bound": "compute" if t_compute >= fa_bytes / hbm_bw else "memory bandwidth",
        "naive_bound": "compute" if t_compute >= naive_bytes / hbm_bw else "memory bandwidth",
        "fa_time_s": fa_time,
        "naive_time_s": naive_time,
        "speedup": naive_time / fa_time,
        "fa_flops_per_s": flops / fa_time,
    }
    if sram_bytes is not None and block is not None:
        per_row = 4.0 * head_dim * elem_bytes  # one row each of the Q, K, V and O tiles
        out["sram_needed_bytes"] = block * per_row
        out["max_block_sram"] = int(sram_bytes // per_row)
        out["sram_fit"] = block * per_row <= sram_bytes
        out["q_blocks"] = math.ceil(seq / block)
    return out


def page_profile_seqs(first: float = 512.0, last: float = 131072.0, n: int = 48) -> list:
    """Geometric sequence-length grid of the reduced-order model's profile curves."""
    r = (last / first) ** (1.0 / (n - 1))
    return [first * r ** i for i in range(n)]
