"""fa_fwd_ws (the forward with a scheduling workspace) through the C ABI.

Where its balanced schedule applies (a resident grid over whole XCDs, at least
8 heads per XCD) the last work items of every XCD are claimed at run time, and
any workgroup may compute any of them.  Which workgroup computes an item does
not change its arithmetic, so the outputs must equal fa_fwd's bit for bit, at
every shape, whether the balanced schedule applies or not.  fa_fwd itself is
checked against the fp64 oracle in test_gpu_parity.py; one balanced shape is
checked against the oracle here as well.  The workspace must be zero before a
call and is left zero after it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tiled_online_softmax_causal_amd as fa
from gpu_util import assert_close, case, device_inputs, gather, oracle_on, require_gpu, scale_of
from workloads import sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    fa.load_library()
    yield
    torch.cuda.synchronize()


def _ws():
    return torch.zeros(fa.fwd_workspace_bytes(), dtype=torch.uint8, device="cuda")


# (B, H, S, D, causal): balanced where B*H >= 64 and the items outnumber the CUs
SHAPES = [
    (8, 32, 8192, 128, True),    # the benchmark shape
    (2, 32, 4096, 128, True),    # 64 heads, 1024 items
    (1, 64, 2048, 64, True),     # d = 64
    (4, 16, 3000, 128, True),    # ragged S (tail tiles), 768 items
    (2, 32, 2048, 128, False),   # non-causal
    (1, 64, 1000, 128, True),    # 256 items: one per CU, not resident -> static
    (1, 32, 4096, 128, True),    # 32 heads -> static
]


@pytest.mark.parametrize("B,H,S,D,causal", SHAPES)
def test_ws_equals_fwd_bitwise(B, H, S, D, causal):
    case(f"fa_fwd_ws vs fa_fwd bf16 {B}x{H}x{S}x{D} causal={causal}, bitwise")
    q, k, v = device_inputs(B, H, S, D, seed=S + D)
    ws = _ws()
    o1, l1 = fa.fwd(q, k, v, causal=causal)
    o2, l2 = fa.fwd(q, k, v, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "O differs from fa_fwd"
    assert torch.equal(l1, l2), "LSE differs from fa_fwd"
    assert int(ws.count_nonzero()) == 0, "workspace not left zero"


def test_ws_reused_across_calls():
    """One workspace, calls of different shapes in a row: each equals fa_fwd and leaves it zero."""
    case("fa_fwd_ws, one workspace over 4 calls (2x32x4096, 1x64x2048, 2x32x4096 again, 8x8x1024)")
    ws = _ws()
    for i, (B, H, S) in enumerate([(2, 32, 4096), (1, 64, 2048), (2, 32, 4096), (8, 8, 1024)]):
        q, k, v = device_inputs(B, H, S, 128, seed=100 + i)
        o1, l1 = fa.fwd(q, k, v)
        o2, l2 = fa.fwd(q, k, v, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"call {i}"
        assert int(ws.count_nonzero()) == 0, f"workspace not zero after call {i}"


def test_ws_against_oracle_sampled():
    """A balanced shape against the fp64 oracle on sampled heads and rows (tile edges included)."""
    case("fa_fwd_ws bf16 2x32x4096x128 causal vs oracle, 4 heads x sampled rows")
    B, H, S, D = 2, 32, 4096, 128
    q, k, v = device_inputs(B, H, S, D)
    o, lse = fa.fwd(q, k, v, workspace=_ws())
    torch.cuda.synchronize()
    bh = [0, 21, 40, 63]
    rows = sample_rows(S, 96, seed=3)
    ref_o, ref_l = oracle_on(q, k, v, True, scale_of(D), bh_idx=bh, row_idx=rows)
    og, lg = gather(o, lse, bh, rows)
    assert_close(og, lg, ref_o, ref_l, torch.bfloat16, "fa_fwd_ws 2x32x4096 sampled")


def test_ws_rejects_small_workspace():
    q, k, v = device_inputs(1, 1, 64, 128)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, workspace=torch.zeros(100, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, workspace=_ws(), variant="mfma_b128")
