"""The library's main entry point, fa_fwd(q, k, v, o, lse, B, H, S, D, causal,
scale, dtype, stream), called through the C ABI at the five workload shapes and
at two shapes between the short-sequence and the full-grid choices.

fa_fwd runs the automatic variant on the automatic schedule.  At each shape its
outputs must equal fa_fwd_variant(FA_VARIANT_AUTO)'s bit for bit (the same
kernels) and match the fp64 oracle: in full where the oracle is quick, else on
sampled heads and rows (first and last rows and the tile edges included).  The
outputs start as NaN, so a row the kernels skipped cannot pass.  The operation
is the forward pass of the aiml.sh page "Speed up long contexts with
FlashAttention" (lab.py, tiled_flash_attention, whose dense counterpart
standard_attention the oracle follows).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import tiled_online_softmax_causal_amd as fa
from gpu_util import assert_close, case, device_inputs, gather, oracle_on, require_gpu, scale_of
from workloads import page_qkv, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    fa.load_library()
    yield
    torch.cuda.synchronize()


def _call(q, k, v, causal, scale, variant=None):
    """One C-ABI call on NaN-filled outputs: fa_fwd (variant None) or fa_fwd_variant."""
    B, H, S, D = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=q.device)
    dt = fa.FA_DTYPE_BF16 if q.dtype == torch.bfloat16 else fa.FA_DTYPE_FP32
    st = torch.cuda.current_stream().cuda_stream
    status = fa.fa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, S, D,
                           causal, scale, dt, st, variant)
    assert status == fa.FA_OK, fa.status_str(status)
    torch.cuda.synchronize()
    return o, lse


# (name, B, H, S, D, causal, oracle heads or None for all, rows per head or None for all)
SHAPES = [
    ("b1 h32 S1024 d128 causal", 1, 32, 1024, 128, True, None, None),
    ("b1 h32 S4096 d128 causal", 1, 32, 4096, 128, True, list(range(32)), 48),
    ("b1 h32 S4096 d128 non-causal", 1, 32, 4096, 128, False, list(range(0, 32, 3)), 48),
    ("b8 h32 S8192 d128 causal", 8, 32, 8192, 128, True, [0, 3 * 32 + 17, 5 * 32 + 4, 7 * 32 + 31], 128),
    ("b1 h32 S32768 d128 causal", 1, 32, 32768, 128, True, [0, 31], 256),
    # between one round of split units and a full grid of 256-row items: the
    # 256-row kernel with idle CUs below 2048 keys, the split kernel in two
    # rounds of units from there
    ("b1 h32 S1792 d128 causal", 1, 32, 1792, 128, True, list(range(0, 32, 5)), 96),
    ("b1 h16 S3000 d128 causal", 1, 16, 3000, 128, True, list(range(16)), 96),
    ("b1 h32 S1792 d64 causal", 1, 32, 1792, 64, True, list(range(0, 32, 5)), 96),
]


@pytest.mark.parametrize("name,B,H,S,D,causal,heads,rows", SHAPES, ids=[s[0] for s in SHAPES])
def test_fa_fwd_workloads(name, B, H, S, D, causal, heads, rows):
    case(f"fa_fwd {name}: bitwise vs fa_fwd_variant(AUTO), oracle parity")
    q, k, v = device_inputs(B, H, S, D)
    scale = scale_of(D)
    o, lse = _call(q, k, v, causal, scale)
    o2, lse2 = _call(q, k, v, causal, scale, fa.FA_VARIANT_AUTO)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "fa_fwd differs from fa_fwd_variant(AUTO)"
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "rows left unwritten"
    del o2, lse2
    if heads is None:
        ref_o, ref_l = oracle_on(q, k, v, causal, scale)
        assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16, name)
    else:
        r = sample_rows(S, rows, tile_edges=(64, 128, 256))
        ref_o, ref_l = oracle_on(q, k, v, causal, scale, bh_idx=heads, row_idx=r)
        og, lg = gather(o, lse, heads, r)
        assert_close(og, lg, ref_o, ref_l, torch.bfloat16, name)
    if causal:
        assert torch.equal(o[:, :, 0], v[:, :, 0]), "causal row 0 must be V row 0"
    del q, k, v, o, lse
    torch.cuda.empty_cache()


def test_fa_fwd_page_example_fp32():
    """The page's worked example (one head, S = 64, d = 16, fp32, Random(42) inputs) through fa_fwd."""
    case("fa_fwd fp32 1x1x64x16 causal, page inputs")
    qp, kp, vp = page_qkv(64, 16, seed=42)
    q, k, v = (torch.tensor(x, dtype=torch.float32, device="cuda")[None, None].contiguous() for x in (qp, kp, vp))
    o, lse = _call(q, k, v, True, 0.25)
    o2, lse2 = _call(q, k, v, True, 0.25, fa.FA_VARIANT_AUTO)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    ref_o, ref_l = oracle_on(q, k, v, True, 0.25)
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.float32, "page example via fa_fwd")
    assert np.array_equal(o[0, 0, 0].cpu().numpy(), v[0, 0, 0].cpu().numpy())
