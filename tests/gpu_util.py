"""Shared helpers of the GPU parity tests: seeded device inputs, the oracle on the
same rounded values, and the tolerance checks.

Tolerances (bf16 inputs, fp32 softmax state and accumulation):
  O    max |gpu - oracle| <= 1e-2 and mean <= 1e-3, the oracle run in fp64 on the
       very bf16 values the kernel read.  The kernel rounds P to bf16 before the
       P.V product (relative error 2^-9 per probability, so at most
       2^-9 * max|v| = 1.6e-3 on O for |v| <= 0.8) and rounds O to bf16 (another
       2^-9 relative); the bound leaves room for fp32 summation order.
  lse  max |gpu - oracle| <= 1e-3: scores are exact bf16 products summed in
       fp32 and the denominator is an fp32 sum of fp32 exponentials, so the
       error is a few fp32 ulps of ln(S) plus summation growth.
fp32 inputs: O and lse within 1e-5 (max abs).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import tiled_online_softmax_causal_amd as fa
from oracle import attention_dense
from workloads import uniform_qkv_device

BF16_MAX, BF16_MEAN, LSE_TOL = 1e-2, 1e-3, 1e-3
FP32_MAX = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU device")


def case(msg: str):
    print(f"[case] {msg}", flush=True)


def device_inputs(B, H, S, D, dtype=torch.bfloat16, seed=42, low=-0.8, high=0.8):
    return uniform_qkv_device(B, H, S, D, seed=seed, low=low, high=high, dtype=dtype, device="cuda")


def scale_of(D: int) -> float:
    """fp32(1/sqrt(D)), the value the kernel receives; the oracle gets the same number."""
    return float(np.float32(1.0 / math.sqrt(D)))


def host_view(t: torch.Tensor) -> np.ndarray:
    """Storage of a device tensor as numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).cpu().numpy()
    return t.cpu().numpy()


def oracle_on(q, k, v, causal, scale, bh_idx=None, row_idx=None):
    """Run the fp64 oracle on exactly the device inputs (only the selected heads are copied)."""
    B, H, S, D = q.shape
    dtype = "bf16" if q.dtype == torch.bfloat16 else "f32"
    if bh_idx is not None:
        idx = torch.as_tensor(np.asarray(bh_idx), device=q.device)
        sel = [t.reshape(B * H, S, D).index_select(0, idx).reshape(1, len(bh_idx), S, D) for t in (q, k, v)]
        return attention_dense(*(host_view(t) for t in sel), dtype=dtype, causal=causal, scale=scale,
                               row_idx=row_idx)
    return attention_dense(*(host_view(t) for t in (q, k, v)), dtype=dtype, causal=causal, scale=scale,
                           row_idx=row_idx)


def gather(o, lse, bh_idx, row_idx):
    """Pick [len(bh), len(rows), D] / [len(bh), len(rows)] from device outputs."""
    B, H, S, D = o.shape
    bh = torch.as_tensor(np.asarray(bh_idx), device=o.device)
    rows = torch.as_tensor(np.asarray(row_idx), device=o.device)
    og = o.reshape(B * H, S, D).index_select(0, bh).index_select(1, rows).float().cpu().numpy()
    lg = lse.reshape(B * H, S).index_select(0, bh).index_select(1, rows).cpu().numpy()
    return og.astype(np.float64), lg.astype(np.float64)


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64).reshape(o_ref.shape)
    err = np.abs(o_gpu - o_ref)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    msg = f"{what}: O max {err.max():.3e} mean {err.mean():.3e}"
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64).reshape(lse_ref.shape)
        lerr = np.abs(lse_gpu - lse_ref).max()
        msg += f" lse max {lerr:.3e}"
    print(msg, flush=True)
    if dtype == torch.bfloat16:
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, msg
        if lse_gpu is not None:
            assert lerr <= LSE_TOL, msg
    else:
        assert err.max() <= FP32_MAX, msg
        if lse_gpu is not None:
            assert lerr <= FP32_MAX, msg
    return err.max()


def run_fwd(q, k, v, causal=True, scale=None, variant="auto"):
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale, variant=variant)
    torch.cuda.synchronize()
    return o, lse
