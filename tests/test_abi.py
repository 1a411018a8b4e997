"""The C-ABI library without a GPU: it loads, exports every declared symbol, and
its host-side logic (argument checks, variant choice, tile scheduler counts) is
right.  No call here reaches a kernel launch: every fa_fwd call below fails
validation on the host, before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

import tiled_online_softmax_causal_amd as fa
from tiled_online_softmax_causal_amd.costmodel import causal_kv_tiles

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    declared = _declared_functions()
    assert declared, "no declarations found in include/fa.h"
    assert sorted(fa.EXPORTS) == declared
    raw = ctypes.CDLL(fa.LIBRARY_PATH)
    for name in declared:
        assert hasattr(raw, name), name
    assert fa.version().startswith("fa_mi355x")
    assert "gfx950" in fa.version()
    assert lib.fa_last_hip_error() == 0


def test_status_strings():
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARGUMENT, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP, 99):
        assert isinstance(fa.status_str(code), str) and fa.status_str(code)


# Fake, 256-byte-aligned, never-dereferenced addresses: every call below is
# rejected before the library touches them.
P = 1 << 20


@pytest.mark.parametrize("ptrs", [(0, P, P, P), (P, 0, P, P), (P, P, 0, P), (P, P, P, 0)])
def test_null_pointer_rejected(ptrs):
    assert fa.fa_fwd_raw(*ptrs, 0, 1, 1, 64, 128, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("B,H,S,D", [(0, 1, 64, 128), (1, 0, 64, 128), (1, 1, 0, 128), (1, 1, 64, 0),
                                     (-1, 1, 64, 128)])
def test_bad_sizes_rejected(B, H, S, D):
    assert fa.fa_fwd_raw(P, P, P, P, 0, B, H, S, D, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), -float("inf")])
def test_non_finite_scale_rejected(scale):
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 64, 128, True, scale, fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT


def test_misaligned_pointers_rejected():
    for i in range(4):
        ptrs = [P, P, P, P]
        ptrs[i] += 2
        assert fa.fa_fwd_raw(*ptrs, 0, 1, 1, 64, 128, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_fwd_raw(P, P, P, P, P + 2, 1, 1, 64, 128, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("D", [8, 48, 96, 256])
def test_unsupported_head_dim(D):
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 64, D, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_UNSUPPORTED


def test_unsupported_dtype_and_variant():
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 64, 128, True, 0.1, 7) == fa.FA_ERR_UNSUPPORTED
    # the matrix-core variants are bf16-only and D in {64, 128}
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 64, 128, True, 0.1, fa.FA_DTYPE_FP32,
                         variant=fa.FA_VARIANT_MFMA_B256) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 64, 32, True, 0.1, fa.FA_DTYPE_BF16,
                         variant=fa.FA_VARIANT_MFMA_B128) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 64, 128, True, 0.1, fa.FA_DTYPE_FP32,
                         variant=fa.FA_VARIANT_MFMA_B128_K128) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 64, 128, True, 0.1, fa.FA_DTYPE_BF16, variant=42) == fa.FA_ERR_UNSUPPORTED
    # the ping-pong variants copy whole key tiles: S >= BK (64 or 128 keys)
    for S, var in ((63, fa.FA_VARIANT_MFMA_B256), (1, fa.FA_VARIANT_MFMA_B256), (127, fa.FA_VARIANT_MFMA_B256_K128),
                   (100, fa.FA_VARIANT_MFMA_B256_K128)):
        assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, S, 128, True, 0.1, fa.FA_DTYPE_BF16,
                             variant=var) == fa.FA_ERR_UNSUPPORTED, (S, var)


def test_size_limits_rejected():
    # S * D must stay below 2^31 (32-bit offsets inside one head)
    assert fa.fa_fwd_raw(P, P, P, P, 0, 1, 1, 1 << 24, 128, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_UNSUPPORTED


def test_variant_selection():
    bf16, f32 = fa.FA_DTYPE_BF16, fa.FA_DTYPE_FP32
    assert fa.select_variant(8, 32, 8192, 128, bf16) == fa.FA_VARIANT_MFMA_B256_K128
    assert fa.select_variant(1, 32, 1024, 128, bf16) == fa.FA_VARIANT_SPLIT
    # between the two: at d = 128 the 256-row kernel below 2048 keys, the split
    # kernel from there; at d = 64 the split kernel
    assert fa.select_variant(1, 32, 1792, 128, bf16) == fa.FA_VARIANT_MFMA_B256_K128
    assert fa.select_variant(1, 32, 1792, 64, bf16) == fa.FA_VARIANT_SPLIT
    # at d = 64 one 256-row item per CU still goes to the split kernel
    assert fa.select_variant(1, 32, 2048, 64, bf16) == fa.FA_VARIANT_SPLIT
    assert fa.select_variant(1, 32, 3000, 64, bf16) == fa.FA_VARIANT_MFMA_B256_K128
    assert fa.select_variant(1, 16, 1792, 128, bf16) == fa.FA_VARIANT_SPLIT
    assert fa.select_variant(1, 16, 3000, 128, bf16) == fa.FA_VARIANT_SPLIT
    assert fa.select_variant(2, 4, 7000, 128, bf16) == fa.FA_VARIANT_SPLIT
    assert fa.select_variant(1, 32, 2048, 128, bf16) == fa.FA_VARIANT_MFMA_B256_K128
    # below one whole 128-key tile the ping-pong kernel is not chosen, nor for
    # rows shorter than 384 keys with at most 384 heads
    assert fa.select_variant(4, 80, 100, 128, bf16) == fa.FA_VARIANT_MFMA_B128
    assert fa.select_variant(4, 80, 128, 128, bf16) == fa.FA_VARIANT_MFMA_B128
    assert fa.select_variant(8, 48, 320, 64, bf16) == fa.FA_VARIANT_MFMA_B128
    assert fa.select_variant(8, 64, 256, 128, bf16) == fa.FA_VARIANT_MFMA_B256_K128
    assert fa.select_variant(4, 80, 400, 128, bf16) == fa.FA_VARIANT_MFMA_B256_K128
    assert fa.select_variant(1, 1, 64, 16, f32) == fa.FA_VARIANT_VALU
    assert fa.select_variant(1, 1, 64, 16, bf16) == fa.FA_VARIANT_VALU
    assert fa.select_variant(1, 1, 64, 128, f32) == fa.FA_VARIANT_VALU
    assert fa.select_variant(1, 1, 64, 96, bf16) == -1
    assert fa.select_variant(0, 1, 64, 128, bf16) == -1


@pytest.mark.parametrize("S", [1, 2, 63, 64, 65, 255, 256, 257, 1000, 8192])
@pytest.mark.parametrize("causal", [True, False])
def test_scheduler_tile_counts(S, causal):
    """The library's per-head tile count equals the causal block rule's closed form."""
    for variant, bq, bk in ((fa.FA_VARIANT_MFMA_B256, 256, 64), (fa.FA_VARIANT_MFMA_B256_K128, 256, 128),
                            (fa.FA_VARIANT_MFMA_B128, 128, 64), (fa.FA_VARIANT_MFMA_B128_K128, 128, 128),
                            (fa.FA_VARIANT_SPLIT, 64, 128),
                            (fa.FA_VARIANT_VALU, 64, 32)):
        assert fa.tiles_per_head(S, causal, variant) == causal_kv_tiles(S, bq, bk, causal)
    assert fa.tiles_per_head(S, causal, 0) == 0


def test_scheduler_page_worked_example():
    """16x16 blocks over 64 rows visit 10 tiles (run-output.txt, flash_tiles_visited)."""
    assert causal_kv_tiles(64, 16, 16) == 10


# ---------------------------------------------------------------- the dense, materialising entry point

def test_dense_workspace_bytes():
    """fp32 scores + bf16 probabilities, S rows each, rows padded to 8 elements."""
    assert fa.dense_workspace_bytes(0) == 0
    assert fa.dense_workspace_bytes(1) == 8 * 1 * 6
    assert fa.dense_workspace_bytes(1000) == 1000 * 1000 * 6
    assert fa.dense_workspace_bytes(1001) == 1008 * 1001 * 6
    assert fa.dense_workspace_bytes(8192) == 8192 * 8192 * 6


def _dense(ws=P, ws_bytes=1 << 40, dtype=fa.FA_DTYPE_BF16, D=128, ptrs=(P, P, P, P), B=1, H=1, S=64,
           scale=0.1):
    return fa.fa_dense_fwd_raw(*ptrs, 0, B, H, S, D, True, scale, dtype, ws, ws_bytes)


def test_dense_rejects_before_launch():
    per_head = fa.dense_workspace_bytes(64)
    assert _dense(ws=0) == fa.FA_ERR_INVALID_ARGUMENT                      # no workspace
    assert _dense(ws_bytes=per_head - 1) == fa.FA_ERR_INVALID_ARGUMENT     # smaller than one head
    assert _dense(ws=P + 8) == fa.FA_ERR_INVALID_ARGUMENT                  # misaligned workspace
    assert _dense(ptrs=(P, P, 0, P)) == fa.FA_ERR_INVALID_ARGUMENT
    assert _dense(B=0) == fa.FA_ERR_INVALID_ARGUMENT
    assert _dense(scale=float("nan")) == fa.FA_ERR_INVALID_ARGUMENT
    assert _dense(dtype=fa.FA_DTYPE_FP32) == fa.FA_ERR_UNSUPPORTED         # bf16 only
    assert _dense(D=32) == fa.FA_ERR_UNSUPPORTED                           # D 64 or 128
    assert _dense(dtype=7) == fa.FA_ERR_UNSUPPORTED


def test_bwd_workspace_bytes():
    """One fp32 row dot product per (batch, head, row)."""
    assert fa.bwd_workspace_bytes(0, 1, 5) == 0
    assert fa.bwd_workspace_bytes(2, 3, 0) == 0
    assert fa.bwd_workspace_bytes(2, 3, 5) == 2 * 3 * 5 * 4
    assert fa.bwd_workspace_bytes(8, 32, 8192) == 8 * 32 * 8192 * 4


def _bwd(ws=P, ws_bytes=1 << 40, dtype=fa.FA_DTYPE_BF16, D=128, ptrs=(P,) * 9, B=1, H=1, S=64, scale=0.1):
    return fa.fa_bwd_raw(*ptrs, B, H, S, D, True, scale, dtype, ws, ws_bytes)


def test_bwd_rejects_before_launch():
    """Every invalid call returns its status on the host; nothing is launched (no GPU here)."""
    assert _bwd(ws=0) == fa.FA_ERR_INVALID_ARGUMENT                                 # no workspace
    assert _bwd(ws_bytes=fa.bwd_workspace_bytes(1, 1, 64) - 4) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd(ws=P + 2) == fa.FA_ERR_INVALID_ARGUMENT                             # misaligned workspace
    for i in range(9):                                                               # each pointer NULL
        ptrs = [P] * 9
        ptrs[i] = 0
        assert _bwd(ptrs=tuple(ptrs)) == fa.FA_ERR_INVALID_ARGUMENT, i
    ptrs = [P] * 9
    ptrs[6] = P + 8                                                                  # misaligned dq
    assert _bwd(ptrs=tuple(ptrs)) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd(B=0) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd(S=0) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd(scale=float("inf")) == fa.FA_ERR_INVALID_ARGUMENT
    assert _bwd(dtype=fa.FA_DTYPE_FP32) == fa.FA_ERR_UNSUPPORTED                    # bf16 only
    assert _bwd(D=32) == fa.FA_ERR_UNSUPPORTED                                      # D 64 or 128
    assert _bwd(S=1 << 24, D=128) == fa.FA_ERR_UNSUPPORTED                          # S * D >= 2^31


def test_fwd_workspace_bytes():
    """A constant: 8 pool counters, a done count and one slot per workgroup."""
    assert fa.fwd_workspace_bytes() == 8192


def _fwd_ws(ws=P, ws_bytes=8192, ptrs=(P, P, P, P), B=1, H=1, S=64, D=128, scale=0.1, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_ws_raw(*ptrs, 0, B, H, S, D, True, scale, dtype, ws, ws_bytes)


def test_fwd_ws_rejects_before_launch():
    """fa_fwd_ws checks its workspace, then everything fa_fwd checks; nothing is launched."""
    assert _fwd_ws(ws=0) == fa.FA_ERR_INVALID_ARGUMENT               # no workspace
    assert _fwd_ws(ws_bytes=8191) == fa.FA_ERR_INVALID_ARGUMENT      # too small
    assert _fwd_ws(ws=P + 4) == fa.FA_ERR_INVALID_ARGUMENT           # not 8-byte aligned
    assert _fwd_ws(ptrs=(P, P, 0, P)) == fa.FA_ERR_INVALID_ARGUMENT
    assert _fwd_ws(B=0) == fa.FA_ERR_INVALID_ARGUMENT
    assert _fwd_ws(scale=float("inf")) == fa.FA_ERR_INVALID_ARGUMENT
    assert _fwd_ws(D=48) == fa.FA_ERR_UNSUPPORTED
    assert _fwd_ws(dtype=7) == fa.FA_ERR_UNSUPPORTED


def test_noalloc_validates_on_the_host():
    """fa_fwd_noalloc checks its arguments before it touches the device (its
    scratch is looked up only for a valid call), so these run without a GPU."""
    P = 1 << 20
    assert fa.fa_fwd_noalloc_raw(0, P, P, P, 0, 1, 1, 64, 128, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_fwd_noalloc_raw(P, P, P, P, 0, 0, 1, 64, 128, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_fwd_noalloc_raw(P, P, P, P, 0, 1, 1, 64, 128, True, float("inf"),
                                 fa.FA_DTYPE_BF16) == fa.FA_ERR_INVALID_ARGUMENT
    assert fa.fa_fwd_noalloc_raw(P, P, P, P, 0, 1, 1, 64, 24, True, 0.1, fa.FA_DTYPE_BF16) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_noalloc_raw(P, P, P, P, 0, 1, 1, 64, 128, True, 0.1, 7) == fa.FA_ERR_UNSUPPORTED
    assert fa.load_library().fa_last_hip_error() == 0
