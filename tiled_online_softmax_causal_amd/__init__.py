"""MI355X (gfx950) tiled online-softmax attention forward.

A thin ctypes binding over the C ABI of ``libfa_mi355x.so`` (declared in
``include/fa.h``).  This module only marshals arguments: every step of the
forward pass runs in the library's HIP kernels, and there is no fallback --
if the library is missing or cannot be loaded, the first call raises.

PyTorch supplies device memory and the current stream; nothing else.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libfa_mi355x.so")

FA_DTYPE_FP32, FA_DTYPE_BF16 = 0, 1
FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
(FA_VARIANT_AUTO, FA_VARIANT_MFMA_B256, FA_VARIANT_MFMA_B128, FA_VARIANT_VALU, FA_VARIANT_MFMA_B256_K128,
 FA_VARIANT_SPLIT, FA_VARIANT_MFMA_B128_K128) = 0, 1, 2, 3, 4, 5, 6
VARIANTS = {"auto": 0, "mfma_b256": 1, "mfma_b128": 2, "valu": 3, "mfma_b256_k128": 4, "split": 5,
            "mfma_b128_k128": 6}

# every symbol include/fa.h declares
EXPORTS = ("fa_fwd", "fa_fwd_ws", "fa_fwd_workspace_bytes", "fa_fwd_noalloc", "fa_fwd_variant", "fa_fwd_select_variant",
           "fa_fwd_tiles_per_head",
           "fa_dense_fwd", "fa_dense_workspace_bytes", "fa_bwd", "fa_bwd_workspace_bytes",
           "fa_status_str", "fa_last_hip_error", "fa_version")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: str = LIBRARY_PATH):
    """Load libfa_mi355x.so and declare its C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m tiled_online_softmax_causal_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, f32, i32, p]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_ws.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, f32, i32, p, i64, p]
    lib.fa_fwd_ws.restype = i32
    lib.fa_fwd_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, f32, i32, p]
    lib.fa_fwd_noalloc.restype = i32
    lib.fa_fwd_workspace_bytes.argtypes = []
    lib.fa_fwd_workspace_bytes.restype = i64
    lib.fa_fwd_variant.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, f32, i32, i32, p]
    lib.fa_fwd_variant.restype = i32
    lib.fa_fwd_select_variant.argtypes = [i64, i64, i64, i64, i32]
    lib.fa_fwd_select_variant.restype = i32
    lib.fa_fwd_tiles_per_head.argtypes = [i64, i32, i32]
    lib.fa_fwd_tiles_per_head.restype = i64
    lib.fa_dense_fwd.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i32, f32, i32, p, i64, p]
    lib.fa_dense_fwd.restype = i32
    lib.fa_dense_workspace_bytes.argtypes = [i64]
    lib.fa_dense_workspace_bytes.restype = i64
    lib.fa_bwd.argtypes = [p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i32, f32, i32, p, i64, p]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.fa_bwd_workspace_bytes.restype = i64
    lib.fa_status_str.argtypes = [i32]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = i32
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def version() -> str:
    return load_library().fa_version().decode()


def status_str(status: int) -> str:
    return load_library().fa_status_str(status).decode()


def select_variant(B: int, H: int, S: int, D: int, dtype: int = FA_DTYPE_BF16) -> int:
    return load_library().fa_fwd_select_variant(B, H, S, D, dtype)


def tiles_per_head(S: int, causal: bool, variant: int) -> int:
    return load_library().fa_fwd_tiles_per_head(S, int(bool(causal)), variant)


def kernel_name(variant: int, D: int, causal: bool, balanced: bool = False) -> str:
    """Name prefix of the kernel a variant launches (as profilers print it); ``balanced``
    selects the instance fa_fwd_ws runs when its balanced schedule applies."""
    c = "true" if causal else "false"
    bal = "true" if balanced else "false"
    if variant == FA_VARIANT_MFMA_B256:
        return f"fa::pp::attn_fwd_pingpong<{D}, 64, {c}, {bal}>"
    if variant == FA_VARIANT_MFMA_B256_K128:
        return f"fa::pp::attn_fwd_pingpong<{D}, 128, {c}, {bal}>"
    if variant == FA_VARIANT_MFMA_B128:
        return f"fa::attn_fwd_mfma_bf16<{D}, 1, {c}, 64>"
    if variant == FA_VARIANT_MFMA_B128_K128:
        return f"fa::attn_fwd_mfma_bf16<{D}, 1, {c}, 128>"
    if variant == FA_VARIANT_SPLIT:
        return f"fa::split::attn_fwd_split<{D}, {c}>"
    if variant == FA_VARIANT_VALU:
        return "fa::attn_fwd_valu<"
    raise ValueError(f"unknown variant {variant}")


def fa_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int, S: int,
               D: int, causal: bool, scale: float, dtype: int, stream: int = 0,
               variant: int | None = None) -> int:
    """Call fa_fwd (``variant`` None) or fa_fwd_variant with raw device addresses;
    returns the fa_status code."""
    lib = load_library()
    args = (q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None, lse_ptr or None, B, H, S, D,
            int(bool(causal)), float(scale), dtype)
    if variant is None:
        return lib.fa_fwd(*args, stream or None)
    return lib.fa_fwd_variant(*args, int(variant), stream or None)


def fa_fwd_ws_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int, S: int,
                  D: int, causal: bool, scale: float, dtype: int, ws_ptr: int, ws_bytes: int,
                  stream: int = 0) -> int:
    """Call fa_fwd_ws with raw device addresses; returns the fa_status code."""
    lib = load_library()
    return lib.fa_fwd_ws(q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None, lse_ptr or None,
                         B, H, S, D, int(bool(causal)), float(scale), dtype, ws_ptr or None, ws_bytes,
                         stream or None)


def fa_fwd_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int, S: int,
                       D: int, causal: bool, scale: float, dtype: int, stream: int = 0) -> int:
    """Call fa_fwd_noalloc (the library's own scheduling scratch) with raw device
    addresses; returns the fa_status code."""
    lib = load_library()
    return lib.fa_fwd_noalloc(q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None, lse_ptr or None,
                              B, H, S, D, int(bool(causal)), float(scale), dtype, stream or None)


def fwd_workspace_bytes() -> int:
    """Bytes of the scheduling workspace fa_fwd_ws takes."""
    return load_library().fa_fwd_workspace_bytes()


def _check(status: int):
    if status == FA_OK:
        return
    lib = load_library()
    msg = lib.fa_status_str(status).decode()
    if status == FA_ERR_HIP:
        msg += f" (hipError_t {lib.fa_last_hip_error()})"
    if status in (FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED):
        raise ValueError(msg)
    raise FAError(status, msg)


def fwd(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None,
        return_lse: bool = True, variant="auto", stream=None, workspace=None):
    """Attention forward on ``[B, H, S, D]`` CUDA tensors (bf16 or fp32).

    Returns ``(o, lse)`` -- ``o`` like ``q``, ``lse`` fp32 ``[B, H, S]`` (natural
    log of the softmax denominator, scale included) -- or ``o`` alone when
    ``return_lse`` is false.  ``scale`` defaults to ``1/sqrt(D)``.  The work is
    enqueued on ``stream`` (default: torch's current stream).  With a
    ``workspace`` (a device tensor of at least ``fwd_workspace_bytes()``
    bytes) the call goes through fa_fwd_ws (run-time balancing of the last
    work items across XCDs; the same results), and ``variant`` must be auto.
    Otherwise the automatic variant goes through fa_fwd and an explicit one
    through fa_fwd_variant.
    """
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be device tensors on one device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    dtype = {torch.bfloat16: FA_DTYPE_BF16, torch.float32: FA_DTYPE_FP32}.get(q.dtype)
    if dtype is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda
          or out.device != q.device):
        raise ValueError("out must be a contiguous device tensor like q, on q's device")
    if return_lse and lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous()
                            or not lse.is_cuda or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 [B, H, S] device tensor on q's device")
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        if workspace is not None:
            if variant != FA_VARIANT_AUTO:
                raise ValueError("a workspace call runs the automatic variant")
            if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
                raise ValueError("workspace must be a contiguous device tensor on q's device")
            status = fa_fwd_ws_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else 0, B, H, S, D, causal, scale,
                                   dtype, workspace.data_ptr(), workspace.numel() * workspace.element_size(), st)
        else:
            status = fa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else 0, B, H, S, D, causal, scale,
                                dtype, st, None if variant == FA_VARIANT_AUTO else variant)
    _check(status)
    return (out, lse) if return_lse else out


def dense_workspace_bytes(S: int) -> int:
    """Workspace bytes fa_dense_fwd needs per (batch, head) at sequence length S."""
    return load_library().fa_dense_workspace_bytes(S)


def fa_dense_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                     S: int, D: int, causal: bool, scale: float, dtype: int, ws_ptr: int,
                     ws_bytes: int, stream: int = 0) -> int:
    """Call fa_dense_fwd with raw device addresses; returns the fa_status code."""
    lib = load_library()
    return lib.fa_dense_fwd(q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None,
                            lse_ptr or None, B, H, S, D, int(bool(causal)), float(scale), dtype,
                            ws_ptr or None, int(ws_bytes), stream or None)


def dense_fwd(q, k, v, causal: bool = True, scale: float | None = None, workspace=None,
              max_workspace_bytes: int | None = None, stream=None):
    """The dense, materialising forward on ``[B, H, S, D]`` bf16 CUDA tensors.

    Returns ``(o, lse)`` like :func:`fwd`.  ``workspace`` is a uint8 CUDA tensor
    of at least :func:`dense_workspace_bytes` bytes; without one, a workspace
    for all heads (or ``max_workspace_bytes``, rounded down to whole heads) is
    allocated here, the library itself allocates nothing.
    """
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    if (not (q.is_cuda and k.is_cuda and v.is_cuda) or not (q.device == k.device == v.device)
            or not (q.dtype == k.dtype == v.dtype == torch.bfloat16)):
        raise ValueError("q, k, v must be bf16 device tensors on one device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    per_head = dense_workspace_bytes(S)
    if workspace is None:
        n = B * H if max_workspace_bytes is None else max(1, min(B * H, max_workspace_bytes // per_head))
        workspace = torch.empty(n * per_head, dtype=torch.uint8, device=q.device)
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor on q's device")
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        status = fa_dense_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), B, H, S, D, causal, scale, FA_DTYPE_BF16,
                                  workspace.data_ptr(), workspace.numel(), st)
    _check(status)
    return out, lse


def bwd_workspace_bytes(B: int, H: int, S: int) -> int:
    """Workspace bytes fa_bwd needs: one fp32 row dot product dO_i . O_i per (batch, head, row)."""
    return load_library().fa_bwd_workspace_bytes(B, H, S)


def fa_bwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, do_ptr: int, dq_ptr: int,
               dk_ptr: int, dv_ptr: int, B: int, H: int, S: int, D: int, causal: bool, scale: float,
               dtype: int, ws_ptr: int, ws_bytes: int, stream: int = 0) -> int:
    """Call fa_bwd with raw device addresses; returns the fa_status code."""
    lib = load_library()
    return lib.fa_bwd(q_ptr or None, k_ptr or None, v_ptr or None, o_ptr or None, lse_ptr or None,
                      do_ptr or None, dq_ptr or None, dk_ptr or None, dv_ptr or None, B, H, S, D,
                      int(bool(causal)), float(scale), dtype, ws_ptr or None, int(ws_bytes), stream or None)


def bwd(q, k, v, o, lse, do, causal: bool = True, scale: float | None = None, workspace=None, stream=None):
    """Gradients ``(dq, dk, dv)`` of the forward on ``[B, H, S, D]`` bf16 CUDA tensors.

    ``o`` and ``lse`` are the forward's outputs (:func:`fwd` with the same
    ``causal`` and ``scale``), ``do`` the upstream gradient of ``o``.
    ``workspace`` is an fp32 (or uint8) CUDA tensor of at least
    :func:`bwd_workspace_bytes` bytes; without one it is allocated here, the
    library itself allocates nothing.
    """
    import torch

    ts = (("q", q), ("k", k), ("v", v), ("o", o), ("do", do))
    if q.dim() != 4 or any(t.shape != q.shape for _, t in ts):
        raise ValueError("q, k, v, o, do must share one [B, H, S, D] shape")
    if any(not t.is_cuda or t.dtype != torch.bfloat16 or t.device != q.device for _, t in ts):
        raise ValueError("q, k, v, o, do must be bf16 device tensors on one device")
    for name, t in ts:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, S, D = q.shape
    if (lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda
            or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 [B, H, S] device tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.empty(B * H * S, dtype=torch.float32, device=q.device)
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        status = fa_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, S, D, causal,
                            scale, FA_DTYPE_BF16, workspace.data_ptr(), ws_bytes, st)
    _check(status)
    return dq, dk, dv
