"""fa_fwd_noalloc (the forward for callers that cannot allocate) through the C ABI.

It runs fa_fwd_ws's kernels with the library's own per-device scheduling
scratch instead of a caller's workspace.  Its outputs must equal fa_fwd_ws's
bit for bit on the same inputs (which fa_fwd_ws itself must equal fa_fwd's,
checked against the oracle elsewhere), over calls in a row that reuse the
scratch: a balanced-schedule shape, then a smaller one, then one where the
schedule is static.  A call rejected for its arguments must enqueue nothing.
"""
from __future__ import annotations

import pytest
import torch

import tiled_online_softmax_causal_amd as fa
from gpu_util import case, device_inputs, require_gpu, scale_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    fa.load_library()
    yield
    torch.cuda.synchronize()


def _outputs(q):
    B, H, S, _ = q.shape
    return (torch.full_like(q, float("nan")),
            torch.full((B, H, S), float("nan"), dtype=torch.float32, device=q.device))


def _noalloc(q, k, v, causal=True):
    B, H, S, D = q.shape
    o, lse = _outputs(q)
    st = fa.fa_fwd_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, S, D,
                               causal, scale_of(D), fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.status_str(st)
    torch.cuda.synchronize()
    return o, lse


def _ws(q, k, v, causal=True):
    B, H, S, D = q.shape
    o, lse = _outputs(q)
    ws = torch.zeros(fa.fwd_workspace_bytes(), dtype=torch.uint8, device=q.device)
    st = fa.fa_fwd_ws_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, S, D,
                          causal, scale_of(D), fa.FA_DTYPE_BF16, ws.data_ptr(), ws.numel(),
                          torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.status_str(st)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    return o, lse


@pytest.mark.parametrize("B,H,S,causal", [(2, 32, 4096, True),     # balanced schedule (64 heads, 1024 items)
                                          (1, 64, 2048, True),     # smaller, balanced
                                          (1, 32, 1024, True),     # not resident: static, scratch untouched
                                          (2, 32, 2048, False)])   # non-causal, balanced
def test_noalloc_equals_ws_calls_in_a_row(B, H, S, causal):
    case(f"fa_fwd_noalloc vs fa_fwd_ws bf16 {B}x{H}x{S}x128 causal={causal}")
    q, k, v = device_inputs(B, H, S, 128, seed=S + B)
    o1, l1 = _noalloc(q, k, v, causal)
    o2, l2 = _ws(q, k, v, causal)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # a second call on the same inputs, after the scratch was used: the same again
    o3, l3 = _noalloc(q, k, v, causal)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_noalloc_two_calls_second_smaller():
    """Two calls in a row on the shared scratch, the second with a smaller input."""
    case("fa_fwd_noalloc: 8x32x8192 then 2x32x2048, each vs fa_fwd_ws")
    for (B, H, S) in [(8, 32, 8192), (2, 32, 2048)]:
        q, k, v = device_inputs(B, H, S, 128, seed=7 * S)
        o1, l1 = _noalloc(q, k, v)
        o2, l2 = _ws(q, k, v)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{B}x{H}x{S}"
        del q, k, v, o1, l1, o2, l2
        torch.cuda.empty_cache()


def test_noalloc_rejects_bad_arguments():
    case("fa_fwd_noalloc: invalid arguments enqueue nothing")
    q, k, v = device_inputs(1, 1, 64, 128)
    o = torch.zeros_like(q)
    st = fa.fa_fwd_noalloc_raw(q.data_ptr() + 2, k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, 1, 1, 64, 128, True,
                               0.1, fa.FA_DTYPE_BF16)
    assert st == fa.FA_ERR_INVALID_ARGUMENT
    st = fa.fa_fwd_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 0, 1, 1, 64, 24, True, 0.1,
                               fa.FA_DTYPE_BF16)
    assert st == fa.FA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
