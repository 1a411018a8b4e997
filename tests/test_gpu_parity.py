"""Parity of the HIP forward pass with the fp64 oracle, through the C ABI.

Workloads: the worked example of the aiml.sh page "Speed up long contexts with
FlashAttention" (one head, S=64, d=16, fp32, Random(42) inputs), then bf16
[B, H, S, D] workloads with i.i.d. uniform(-0.8, 0.8) Q/K/V from a seeded
generator, scale fp32(1/sqrt(D)): b1 h32 S1024 d128 (full check), b1 h32 S4096
(causal and non-causal, sampled rows of every head), b8 h32 S8192 (the
benchmark's launch, sampled heads x rows) and b1 h32 S32768 (2 heads x 256
rows).  Sampled rows always include the first and last rows and the tile
edges.  Edge cases: ragged and tiny S, every kernel variant, non-causal,
negative and zero scale, wide score ranges, and closed forms that hold at any
size (Q = 0 gives the causal prefix mean of V and lse_i = ln(i+1)).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import tiled_online_softmax_causal_amd as fa
from gpu_util import (assert_close, case, device_inputs, gather, oracle_on, require_gpu, run_fwd,
                      scale_of)
from workloads import page_qkv, sample_rows

pytestmark = pytest.mark.gpu

# the matrix-core kernels: 256-query ping-pong with 64- and 128-key tiles, the
# 128-query four-wave kernel with 64- and 128-key tiles, and the short-sequence
# kernel (pairs of 64-row blocks, four key streams merged on chip)
MFMA = ["mfma_b256", "mfma_b256_k128", "mfma_b128", "mfma_b128_k128", "split"]
# the ping-pong kernels copy whole key tiles (a last tile cut short is copied as
# the sequence's last BK rows), so they take S >= BK
PINGPONG_MIN_S = {"mfma_b256": 64, "mfma_b256_k128": 128}

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    fa.load_library()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- the page's worked example, fp32

def test_page_worked_example_fp32():
    case("fp32 1x1x64x16 causal, page inputs Random(42), VALU variant")
    with open(os.path.join(GOLDEN, "page_equivalence_check.json")) as f:
        g = json.load(f)
    qp, kp, vp = page_qkv(64, 16, seed=42)
    q, k, v = (torch.tensor(x, dtype=torch.float32, device="cuda")[None, None].contiguous() for x in (qp, kp, vp))
    o, lse = run_fwd(q, k, v, causal=True, scale=0.25)
    ref_o, ref_l = oracle_on(q, k, v, True, 0.25)
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.float32, "page example")
    on = o.cpu().numpy()[0, 0].astype(np.float64)
    # the page prints 6 decimals: the kernel's values must round-trip within the fp32 bound
    assert np.abs(on[0, :4] - g["sample_row0_first4"]).max() <= 5e-7 + 1e-5
    assert np.abs(on[-1, :4] - g["sample_last_row_first4"]).max() <= 5e-7 + 1e-5
    # causal row 0 sees only key 0: O[0] is V[0] exactly
    assert np.array_equal(o[0, 0, 0].cpu().numpy(), v[0, 0, 0].cpu().numpy())


# ---------------------------------------------------------------- full checks at oracle-sized shapes

@pytest.mark.parametrize("variant", ["auto", *MFMA, "valu"])
@pytest.mark.parametrize("causal", [True, False])
def test_b1_h32_s1024_d128(variant, causal):
    case(f"bf16 1x32x1024x128 causal={causal} variant={variant}, full oracle")
    q, k, v = device_inputs(1, 32, 1024, 128)
    o, lse = run_fwd(q, k, v, causal=causal, variant=variant)
    ref_o, ref_l = oracle_on(q, k, v, causal, scale_of(128))
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16,
                 f"S1024 {variant} causal={causal}")


@pytest.mark.parametrize("S", [1, 2, 31, 63, 64, 65, 127, 129, 255, 257, 333, 1000])
@pytest.mark.parametrize("variant", [*MFMA, "valu"])
@pytest.mark.parametrize("D", [64, 128])
def test_ragged_lengths_bf16(S, variant, D):
    if S < PINGPONG_MIN_S.get(variant, 1):
        pytest.skip(f"{variant} takes whole key tiles: S >= {PINGPONG_MIN_S[variant]} (FA_ERR_UNSUPPORTED below)")
    case(f"bf16 2x3x{S}x{D} causal variant={variant}")
    q, k, v = device_inputs(2, 3, S, D, seed=S)
    for causal in (True, False):
        o, lse = run_fwd(q, k, v, causal=causal, variant=variant)
        ref_o, ref_l = oracle_on(q, k, v, causal, scale_of(D))
        assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16,
                     f"S{S} D{D} {variant} causal={causal}")


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("S", [1, 33, 64, 200])
def test_fp32_valu(S, D):
    case(f"fp32 1x2x{S}x{D} VALU")
    q, k, v = device_inputs(1, 2, S, D, dtype=torch.float32, seed=100 + S)
    for causal in (True, False):
        o, lse = run_fwd(q, k, v, causal=causal)
        ref_o, ref_l = oracle_on(q, k, v, causal, scale_of(D))
        assert_close(o.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.float32,
                     f"fp32 S{S} D{D} causal={causal}")


@pytest.mark.parametrize("D", [16, 32])
def test_bf16_small_head_dims(D):
    case(f"bf16 1x4x300x{D} (VALU path)")
    q, k, v = device_inputs(1, 4, 300, D, seed=D)
    o, lse = run_fwd(q, k, v, causal=True)
    ref_o, ref_l = oracle_on(q, k, v, True, scale_of(D))
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16, f"bf16 D{D}")


# ---------------------------------------------------------------- scale and score-range edge cases

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("variant", [*MFMA, "valu"])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.0])
def test_scale_values(variant, scale, causal):
    """S = 300 is not a multiple of any key tile: the last tile is cut short.  With
    scale 0 every visible key weighs the same, so a key counted twice (the
    ping-pong kernels copy a cut-short tile as the sequence's last BK rows and mask
    the keys it repeats) would show in the mean."""
    case(f"bf16 1x2x300x128 scale={scale} causal={causal} variant={variant}")
    q, k, v = device_inputs(1, 2, 300, 128, seed=7)
    o, lse = run_fwd(q, k, v, causal=causal, scale=scale, variant=variant)
    ref_o, ref_l = oracle_on(q, k, v, causal, scale)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16,
                 f"scale {scale} causal={causal} {variant}")


@pytest.mark.parametrize("variant", MFMA)
def test_wide_score_range(variant):
    """Q, K ~ uniform(-4, 4): score std ~5, so the running max jumps and alpha rescales often."""
    case(f"bf16 1x4x1000x128 Q,K uniform(-4,4) variant={variant}")
    q, k, _ = device_inputs(1, 4, 1000, 128, seed=13, low=-4.0, high=4.0)
    _, _, v = device_inputs(1, 4, 1000, 128, seed=14)
    o, lse = run_fwd(q, k, v, causal=True, variant=variant)
    ref_o, ref_l = oracle_on(q, k, v, True, scale_of(128))
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16, "wide range")


def test_increasing_scores_force_rescale():
    """Scores that grow with the key index make every key tile raise the running max."""
    case("bf16 1x1x700x128 growing scores")
    S, D = 700, 128
    q = torch.full((1, 1, S, D), 0.25, device="cuda")
    k = (torch.arange(S, device="cuda", dtype=torch.float32) / S * 3.0)[None, None, :, None].expand(1, 1, S, D)
    _, _, v = device_inputs(1, 1, S, D, seed=5)
    q, k = q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous()
    for variant in (*MFMA, "valu"):
        o, lse = run_fwd(q, k, v, causal=True, variant=variant)
        ref_o, ref_l = oracle_on(q, k, v, True, scale_of(D))
        assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16,
                     f"growing {variant}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("variant", [*MFMA, "valu"])
def test_scores_outgrow_fp32_range(variant, causal):
    """Scores that rise by ~1.85 (base 2) per key: within one 64-key tile they grow
    by ~118, so exponentiating against the previous tile's maximum would overflow
    fp32.  Kernels that keep a stale maximum must detect that and rescale.  Non-
    causal, the largest scores sit in the cut-short last tile (S = 700), next to the
    keys it repeats from the tile before, which must stay masked through the redo."""
    case(f"bf16 1x2x700x128 scale=1 growing scores, causal={causal} variant={variant}")
    S, D = 700, 128
    q = torch.full((1, 2, S, D), 0.5, device="cuda")
    k = (torch.arange(S, device="cuda", dtype=torch.float32) * 0.02)[None, None, :, None].expand(1, 2, S, D)
    _, _, v = device_inputs(1, 2, S, D, seed=6)
    q, k = q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous()
    o, lse = run_fwd(q, k, v, causal=causal, scale=1.0, variant=variant)
    ref_o, ref_l = oracle_on(q, k, v, causal, 1.0)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16,
                 f"outgrow causal={causal} {variant}")


@pytest.mark.parametrize("variant", MFMA)
def test_scores_outgrow_fp32_range_masked(variant):
    """As above but decreasing keys: the largest scores sit in the first tile and
    the causal mask hides the end of each diagonal tile, so rows whose visible
    keys are all far below the running maximum must still come out right."""
    case(f"bf16 1x1x333x128 scale=1 shrinking scores, variant={variant}")
    S, D = 333, 128
    q = torch.full((1, 1, S, D), 0.5, device="cuda")
    k = ((S - torch.arange(S, device="cuda", dtype=torch.float32)) * 0.02)[None, None, :, None].expand(1, 1, S, D)
    _, _, v = device_inputs(1, 1, S, D, seed=8)
    q, k = q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous()
    o, lse = run_fwd(q, k, v, causal=True, scale=1.0, variant=variant)
    ref_o, ref_l = oracle_on(q, k, v, True, 1.0)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, torch.bfloat16,
                 f"shrink {variant}")


# ---------------------------------------------------------------- the benchmark's workloads, sampled

def _sampled_check(B, H, S, D, causal, bh_idx, n_rows, variant="auto"):
    q, k, v = device_inputs(B, H, S, D)
    o, lse = run_fwd(q, k, v, causal=causal, variant=variant)
    rows = sample_rows(S, n_rows, tile_edges=(32, 64, 128, 256))
    ref_o, ref_l = oracle_on(q, k, v, causal, scale_of(D), bh_idx=bh_idx, row_idx=rows)
    og, lg = gather(o, lse, bh_idx, rows)
    assert_close(og, lg, ref_o, ref_l, torch.bfloat16, f"{B}x{H}x{S}x{D} causal={causal} sampled")
    # causal row 0 is V row 0 for every head
    if causal:
        assert torch.equal(o[:, :, 0], v[:, :, 0])
    return q, k, v, o, lse


@pytest.mark.parametrize("causal", [True, False])
def test_b1_h32_s4096_sampled(causal):
    case(f"bf16 1x32x4096x128 causal={causal}, all heads x 48 rows")
    _sampled_check(1, 32, 4096, 128, causal, list(range(32)), 48)


@pytest.mark.parametrize("variant", ["auto", "mfma_b256", "mfma_b256_k128"])
def test_b8_h32_s8192_sampled(variant):
    case(f"bf16 8x32x8192x128 causal (benchmark launch) variant={variant}, 4 heads x 256 rows")
    bh = [0 * 32 + 0, 3 * 32 + 17, 5 * 32 + 4, 7 * 32 + 31]
    _sampled_check(8, 32, 8192, 128, True, bh, 256, variant=variant)
    torch.cuda.empty_cache()


def test_b1_h32_s32768_sampled():
    case("bf16 1x32x32768x128 causal, 2 heads x 256 rows")
    _sampled_check(1, 32, 32768, 128, True, [0, 31], 256)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,H,S,n_rows", [(1, 2, 131072, 48), (1, 1, 1 << 20, 24)])
def test_long_sequences_sampled(B, H, S, n_rows):
    """The end of the measured sweep (S = 131072) and S = 2^20, where row offsets
    reach 2^27 elements; sampled rows always include the last ones."""
    case(f"bf16 {B}x{H}x{S}x128 causal, {n_rows} rows per head")
    _sampled_check(B, H, S, 128, True, list(range(B * H)), n_rows)
    torch.cuda.empty_cache()


def _run_poisoned(q, k, v, causal, scale, variant="auto"):
    """The forward into NaN-filled outputs; every element must come out finite (no
    work item skipped, none written twice with a stale value)."""
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse, variant=variant)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "rows left unwritten"
    return o, lse


@pytest.mark.parametrize("B,H,S", [(1, 5, 16384), (2, 8, 5000), (1, 32, 7723), (1, 32, 2373), (1, 12, 8192),
                                   (1, 20, 4096), (2, 32, 7723)])
def test_resident_grid_sequences(B, H, S):
    """More work items than CUs, so one resident workgroup per CU walks a sequence of
    items: h5 (heads not grouped per XCD, items taken in strides of the grid),
    b2 h8 S5000 (grouped per XCD, 40 items per XCD for 32 workgroups: a partial
    second round), b1 h32 at S = 7723 and 2373 (31 and 10 query blocks per head,
    not a multiple of the 32 workgroups of an XCD, where the cost model may deal an
    XCD's heads block by block), b1 h12 and h20 (flat lists, heads not a multiple of
    8) and b2 h32 S7723.  Items of odd rounds walk their keys from the diagonal
    down.  Outputs start as NaN and must all come out finite; sampled rows of every
    head against the oracle."""
    case(f"bf16 {B}x{H}x{S}x128 causal, resident grid")
    q, k, v = device_inputs(B, H, S, 128, seed=S)
    o, lse = _run_poisoned(q, k, v, True, scale_of(128))
    rows = sample_rows(S, 24, tile_edges=(128, 256))
    bh = list(range(B * H))
    ref_o, ref_l = oracle_on(q, k, v, True, scale_of(128), bh_idx=bh, row_idx=rows)
    og, lg = gather(o, lse, bh, rows)
    assert_close(og, lg, ref_o, ref_l, torch.bfloat16, f"resident {B}x{H}x{S}")


@pytest.mark.parametrize("B,H,S,D,causal,scale", [
    (4, 80, 128, 128, True, None),     # one-tile items: a K copy runs two items ahead
    (4, 80, 200, 128, True, None),     # two-tile items, the second cut short (copied as keys 72..199)
    (4, 80, 129, 64, True, None),      # two-tile items, the second one key wide
    (1, 10, 8000, 128, False, None),   # non-causal: every item sees all 63 tiles
    (1, 5, 16384, 128, True, -0.05),   # negative scale across item boundaries
    (2, 8, 5000, 64, True, None),      # d = 64
])
def test_resident_grid_edge_items(B, H, S, D, causal, scale):
    """Resident grids (more items than CUs) at the edges of the item chaining: the tile
    sequence of a workgroup runs across item boundaries, where one matrix phase
    finishes an item and starts the next.  Sampled rows of every head (all rows for
    the short sequences).  The ping-pong kernel is named explicitly: for the shortest
    of these shapes the automatic choice is the 128-row kernel."""
    scale = scale_of(D) if scale is None else scale
    case(f"bf16 {B}x{H}x{S}x{D} causal={causal} scale={scale}, resident grid")
    q, k, v = device_inputs(B, H, S, D, seed=S + D)
    o, lse = _run_poisoned(q, k, v, causal, scale, variant="mfma_b256_k128")
    rows = np.arange(S) if S <= 256 else sample_rows(S, 16, tile_edges=(128, 256))
    bh = list(range(B * H))
    ref_o, ref_l = oracle_on(q, k, v, causal, scale, bh_idx=bh, row_idx=rows)
    og, lg = gather(o, lse, bh, rows)
    assert_close(og, lg, ref_o, ref_l, torch.bfloat16, f"resident edge {B}x{H}x{S}x{D}")


# ---------------------------------------------------------------- closed forms at full size

@pytest.mark.parametrize("shape", [(8, 32, 8192, 128), (1, 32, 32768, 128), (2, 3, 1000, 64)])
def test_zero_query_prefix_mean(shape):
    """Q = 0: every score is 0, so O_i is the mean of V_0..V_i and lse_i = ln(i+1), at any size."""
    B, H, S, D = shape
    case(f"bf16 {B}x{H}x{S}x{D} Q=0 closed form")
    _, k, v = device_inputs(B, H, S, D, seed=21)
    q = torch.zeros_like(v)
    o, lse = run_fwd(q, k, v, causal=True)
    n = torch.arange(1, S + 1, device="cuda", dtype=torch.float64)
    want = v.double().cumsum(dim=2) / n[None, None, :, None]
    err = (o.double() - want).abs()
    lerr = (lse.double() - torch.log(n)[None, None]).abs().max().item()
    print(f"Q=0 {shape}: O max {err.max().item():.3e} mean {err.mean().item():.3e} lse {lerr:.3e}", flush=True)
    assert err.max().item() <= 1e-2 and err.mean().item() <= 1e-3 and lerr <= 1e-3
    del q, k, v, o, want, err
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- invariants of the implementation

def test_deterministic_and_stream_independent():
    case("bf16 1x32x1024x128 repeat x3 and on a side stream")
    q, k, v = device_inputs(1, 32, 1024, 128)
    o0, l0 = run_fwd(q, k, v)
    for _ in range(2):
        o1, l1 = run_fwd(q, k, v)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        o2, l2 = fa.fwd(q, k, v, causal=True)
    side.synchronize()
    assert torch.equal(o0, o2) and torch.equal(l0, l2)


@pytest.mark.parametrize("other", ["mfma_b128", "mfma_b128_k128", "mfma_b256_k128", "split"])
def test_variants_agree(other):
    """Different tilings and schedules give the same result within rounding."""
    case(f"bf16 2x4x777x128 mfma_b256 vs {other}")
    q, k, v = device_inputs(2, 4, 777, 128, seed=3)
    oa, la = run_fwd(q, k, v, variant="mfma_b256")
    ob, lb = run_fwd(q, k, v, variant=other)
    assert (oa.float() - ob.float()).abs().max().item() <= 1e-2
    assert (la - lb).abs().max().item() <= 1e-5


def test_causality_on_gpu():
    """Changing K/V rows after i leaves O rows 0..i bit-identical."""
    case("bf16 1x2x512x128 causality")
    q, k, v = device_inputs(1, 2, 512, 128, seed=9)
    o1, l1 = run_fwd(q, k, v)
    i = 300
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i + 1:] = -k2[:, :, i + 1:] * 3
    v2[:, :, i + 1:] = v2[:, :, i + 1:] * 2
    o2, l2 = run_fwd(q, k2, v2)
    assert torch.equal(o1[:, :, : i + 1], o2[:, :, : i + 1])
    assert torch.equal(l1[:, :, : i + 1], l2[:, :, : i + 1])


def test_lse_optional_and_output_buffer():
    case("bf16 1x2x256x128 lse=NULL, caller-provided out")
    q, k, v = device_inputs(1, 2, 256, 128, seed=4)
    o_ref, _ = run_fwd(q, k, v)
    out = torch.full_like(q, float("nan"))
    o = fa.fwd(q, k, v, causal=True, out=out, return_lse=False)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and torch.equal(o, o_ref)


def test_invalid_calls_enqueue_nothing():
    case("error paths on the GPU")
    q, k, v = device_inputs(1, 1, 64, 128)
    o = torch.zeros_like(q)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v[..., :64].contiguous())
    with pytest.raises(ValueError):
        fa.fwd(q.float(), k, v)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, scale=float("nan"))
    st = fa.fa_fwd_raw(q.data_ptr() + 2, k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, 1, 1, 64, 128, True, 0.1,
                       fa.FA_DTYPE_BF16)
    assert st == fa.FA_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
