"""Parity of the dense, materialising GPU forward (fa_dense_fwd) with the fp64 oracle.

The dense path is the standard attention of the aiml.sh page "Speed up long
contexts with FlashAttention" (lab.py, standard_attention) run on the GPU with
its score and probability matrices in HBM; it must give the tiled path's
results.  Same tolerances as the tiled path (tests/gpu_util.py): it too rounds
the probabilities to bf16 before the P.V product.  Cases: full oracle checks at
S = 1024, ragged and tiny lengths, both head dims, non-causal, scale edge
cases, wide score ranges, chunked workspaces (bit-identical to one chunk), and
the benchmark shape b8 h32 S8192 d128 on sampled heads and rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tiled_online_softmax_causal_amd as fa
from gpu_util import assert_close, case, device_inputs, gather, oracle_on, require_gpu, run_fwd, scale_of
from workloads import sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    fa.load_library()
    yield
    torch.cuda.synchronize()


def _dense(q, k, v, causal=True, scale=None, **kw):
    o, lse = fa.dense_fwd(q, k, v, causal=causal, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [64, 128])
def test_dense_b1_h4_s1024_full(causal, D):
    case(f"dense bf16 1x4x1024x{D} causal={causal}, full oracle")
    q, k, v = device_inputs(1, 4, 1024, D)
    o, lse = _dense(q, k, v, causal=causal)
    ref_o, ref_l = oracle_on(q, k, v, causal, scale_of(D))
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16, f"dense D{D}")


@pytest.mark.parametrize("S", [1, 2, 7, 63, 64, 127, 129, 255, 333, 1000])
@pytest.mark.parametrize("D", [64, 128])
def test_dense_ragged_lengths(S, D):
    case(f"dense bf16 2x3x{S}x{D}, causal and not")
    q, k, v = device_inputs(2, 3, S, D, seed=S + 1)
    for causal in (True, False):
        o, lse = _dense(q, k, v, causal=causal)
        ref_o, ref_l = oracle_on(q, k, v, causal, scale_of(D))
        assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16,
                     f"dense S{S} D{D} causal={causal}")


def test_dense_chunked_workspace_is_bit_identical():
    """A workspace for one head at a time gives exactly the one-chunk result."""
    case("dense bf16 2x3x333x128, workspace of 1 and 2 heads vs 6")
    q, k, v = device_inputs(2, 3, 333, 128, seed=11)
    o_all, l_all = _dense(q, k, v)
    per_head = fa.dense_workspace_bytes(333)
    for heads in (1, 2):
        o, lse = _dense(q, k, v, max_workspace_bytes=heads * per_head)
        assert torch.equal(o, o_all) and torch.equal(lse, l_all)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.0])
def test_dense_scale_values(scale):
    case(f"dense bf16 1x2x300x128 scale={scale}")
    q, k, v = device_inputs(1, 2, 300, 128, seed=7)
    o, lse = _dense(q, k, v, scale=scale)
    ref_o, ref_l = oracle_on(q, k, v, True, scale)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16, f"dense scale {scale}")


def test_dense_wide_score_range():
    case("dense bf16 1x4x1000x128 Q,K uniform(-4,4)")
    q, k, _ = device_inputs(1, 4, 1000, 128, seed=13, low=-4.0, high=4.0)
    _, _, v = device_inputs(1, 4, 1000, 128, seed=14)
    o, lse = _dense(q, k, v)
    ref_o, ref_l = oracle_on(q, k, v, True, scale_of(128))
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16, "dense wide range")


def test_dense_agrees_with_tiled_s4096():
    """The two GPU paths on b1 h32 S4096: both within tolerance of each other."""
    case("dense vs tiled bf16 1x32x4096x128 causal")
    q, k, v = device_inputs(1, 32, 4096, 128)
    od, ld = _dense(q, k, v)
    ot, lt = run_fwd(q, k, v)
    err = (od.float() - ot.float()).abs()
    assert err.max().item() <= 1e-2 and err.mean().item() <= 1e-3
    assert (ld - lt).abs().max().item() <= 1e-3
    rows = sample_rows(4096, 32, tile_edges=(128,))
    ref_o, ref_l = oracle_on(q, k, v, True, scale_of(128), bh_idx=[0, 31], row_idx=rows)
    og, lg = gather(od, ld, [0, 31], rows)
    assert_close(og, lg, ref_o, ref_l, torch.bfloat16, "dense S4096 sampled")


def test_dense_b8_h32_s8192_sampled():
    """The benchmark shape through a 16-head workspace (16 chunks), sampled heads x rows."""
    case("dense bf16 8x32x8192x128 causal, 16-head workspace, 4 heads x 128 rows")
    q, k, v = device_inputs(8, 32, 8192, 128)
    o, lse = _dense(q, k, v, max_workspace_bytes=16 * fa.dense_workspace_bytes(8192))
    bh = [0, 3 * 32 + 17, 5 * 32 + 4, 7 * 32 + 31]
    rows = sample_rows(8192, 128, tile_edges=(128, 256))
    ref_o, ref_l = oracle_on(q, k, v, True, scale_of(128), bh_idx=bh, row_idx=rows)
    og, lg = gather(o, lse, bh, rows)
    assert_close(og, lg, ref_o, ref_l, torch.bfloat16, "dense b8 S8192 sampled")
    assert torch.equal(o[:, :, 0], v[:, :, 0])  # causal row 0 is V row 0
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_dense_small_workspace_rejected():
    q, k, v = device_inputs(1, 1, 64, 128)
    ws = torch.empty(fa.dense_workspace_bytes(64) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fa.dense_fwd(q, k, v, workspace=ws)
