"""Parity of the GPU backward (fa_bwd) with the fp64 backward oracle.

The GPU path gets the forward's own outputs (fa_fwd: O in bf16, the fp32 LSE)
and a seeded dO; the oracle differentiates the exact forward on the very bf16
values the kernels read.

Tolerance, per gradient tensor and head, relative to the largest oracle value
m = max(max |g_ref|, 1e-3):  max |g_gpu - g_ref| <= 2e-2 m and mean <= 2e-3 m.
  - the outputs are rounded to bf16: 2^-9 relative, at most 2e-3 m;
  - P and dS are rounded to bf16 as MFMA operands: 2^-9 times the sum of
    |terms| of each dot product, which for these inputs is a few times the
    largest result (cancellation), hence the 2e-2 bound on the maximum;
  - delta comes from the bf16 O of the forward and P from its fp32 LSE, both
    within the forward's own tolerance, which adds far less than the above;
  - the floor of m: a gradient the oracle gives as exactly zero (one visible
    key: dS = P (dP - delta) with dP and delta the same dot product) comes out
    at fp32 rounding size (1e-8), since the kernel sums dP and delta in
    different orders.
Invariants at full size (no oracle): the key gradients of every head sum to
zero over keys and the value gradients to the sum of dO rows, within 1e-3 of
the sums of absolute values.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tiled_online_softmax_causal_amd as fa
from gpu_util import case, device_inputs, host_view, require_gpu, scale_of
from oracle.backward import attention_backward

pytestmark = pytest.mark.gpu
REL_MAX, REL_MEAN, M_FLOOR = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    fa.load_library()
    yield
    torch.cuda.synchronize()


def _run(B, H, S, D, causal=True, scale=None, seed=42, low=-0.8, high=0.8):
    q, k, v = device_inputs(B, H, S, D, seed=seed, low=low, high=high)
    do, _, _ = device_inputs(B, H, S, D, seed=seed + 1000, low=-1.0, high=1.0)
    scale = scale_of(D) if scale is None else scale
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv), scale


def _check(inputs, grads, causal, scale, heads=None, what=""):
    q, k, v, do = inputs
    B, H, S, D = q.shape
    bh = list(range(B * H)) if heads is None else heads
    idx = torch.as_tensor(bh, device=q.device)
    sel = lambda t: t.reshape(B * H, S, D).index_select(0, idx).reshape(1, len(bh), S, D)
    refs = attention_backward(*(host_view(sel(t)) for t in (q, k, v, do)), causal=causal, scale=scale,
                              dtype="bf16")
    for name, g, ref in zip(("dq", "dk", "dv"), grads, refs):
        gg = sel(g).float().cpu().numpy().astype(np.float64).reshape(ref.shape)
        assert np.isfinite(gg).all(), f"{what} {name}: non-finite"
        for n in range(len(bh)):
            m = max(np.abs(ref[n]).max(), M_FLOOR)
            err = np.abs(gg[n] - ref[n])
            msg = f"{what} {name} head {bh[n]}: max {err.max() / m:.2e} mean {err.mean() / m:.2e} of max|ref| {m:.3e}"
            assert err.max() <= REL_MAX * m and err.mean() <= REL_MEAN * m, msg
        worst = max(np.abs(gg[n] - ref[n]).max() / max(np.abs(ref[n]).max(), M_FLOOR) for n in range(len(bh)))
        print(f"{what} {name}: worst max/m {worst:.2e}", flush=True)


@pytest.mark.parametrize("S", [1, 7, 64, 65, 127, 128, 129, 200, 333])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_small_full(S, D, causal):
    case(f"bwd bf16 1x2x{S}x{D} causal={causal}, full oracle")
    inputs, grads, scale = _run(1, 2, S, D, causal=causal, seed=S + D)
    _check(inputs, grads, causal, scale, what=f"S{S} D{D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_b1_h4_s1024_full(D):
    case(f"bwd bf16 1x4x1024x{D} causal, full oracle")
    inputs, grads, scale = _run(1, 4, 1024, D)
    _check(inputs, grads, True, scale, what=f"1x4x1024x{D}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.0])
def test_bwd_scale_values(scale):
    case(f"bwd bf16 1x2x300x128 scale={scale}")
    inputs, grads, scale = _run(1, 2, 300, 128, scale=scale, seed=7)
    _check(inputs, grads, True, scale, what=f"scale {scale}")


def test_bwd_wide_score_range():
    case("bwd bf16 1x2x500x128 Q,K uniform(-4,4)")
    inputs, grads, scale = _run(1, 2, 500, 128, seed=13, low=-4.0, high=4.0)
    _check(inputs, grads, True, scale, what="wide range")


def test_bwd_b1_h32_s4096_two_heads():
    case("bwd bf16 1x32x4096x128 causal, heads 0 and 31 against the oracle")
    inputs, grads, scale = _run(1, 32, 4096, 128)
    _check(inputs, grads, True, scale, heads=[0, 31], what="1x32x4096")


def test_bwd_b8_h32_s8192_one_head_and_invariants():
    """The benchmark shape: one head against the oracle; every head through the
    key-shift and value-sum invariants."""
    case("bwd bf16 8x32x8192x128 causal, head 117 against the oracle, invariants on all")
    inputs, grads, scale = _run(8, 32, 8192, 128)
    q, k, v, do = inputs
    dq, dk, dv = grads
    sk = dk.float().sum(dim=2)
    assert (sk.abs() <= 1e-3 * dk.float().abs().sum(dim=2) + 1e-6).all(), "key gradients do not sum to zero"
    sv = dv.float().sum(dim=2) - do.float().sum(dim=2)
    assert (sv.abs() <= 1e-3 * dv.float().abs().sum(dim=2) + 1e-3).all(), "value gradients do not sum to sum dO"
    _check(inputs, grads, True, scale, heads=[117], what="8x32x8192")
    del inputs, grads, q, k, v, do, dq, dk, dv
    torch.cuda.empty_cache()


def test_bwd_deterministic():
    """One writer per output row and no atomics: two runs agree bit for bit."""
    case("bwd bf16 2x8x1000x128 twice")
    inputs, g1, scale = _run(2, 8, 1000, 128, seed=5)
    q, k, v, do = inputs
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bwd_rejects_bad_workspace():
    q, k, v = device_inputs(1, 1, 64, 128)
    o, lse = fa.fwd(q, k, v)
    ws = torch.empty(63, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, q, workspace=ws)
