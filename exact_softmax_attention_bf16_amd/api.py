"""Python face of the C ABI: attention() on torch bf16 tensors resident on the GPU.

PyTorch supplies device memory and the current stream; every step of the
computation runs in the HIP kernels behind attn_forward.
"""
from __future__ import annotations

import ctypes
import math
from contextlib import contextmanager

import torch

from . import _lib


def _check(t: torch.Tensor, name: str, like: torch.Tensor | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP (cuda) device, got {t.device}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, L, d], got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if like is not None:
        if t.shape != like.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != q shape {tuple(like.shape)}")
        if t.device != like.device:
            raise ValueError(f"{name} is on {t.device}, q on {like.device}")


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
              causal: bool = False, out: torch.Tensor | None = None) -> torch.Tensor:
    """O = softmax(scale * Q K^T) V for bf16 [B, H, L, d] tensors (HIP kernels only).

    ``scale`` defaults to 1/sqrt(d).  ``out``, if given, must be a contiguous bf16
    tensor of q's shape that overlaps none of the inputs.  Work is queued on the
    current stream of q's device.
    """
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q)
    lib = _lib.load()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, d, float(scale),
            1 if causal else 0)
    if q.device.index == torch.cuda.current_device():
        status = lib.attn_forward(*args, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    else:  # the library launches on the current device: switch to q's for the call
        with torch.cuda.device(q.device):
            status = lib.attn_forward(
                *args, ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream))
    if status != _lib.ATTN_OK:
        raise _lib.AttnError(status)
    return out


def path_for_head_dim(d: int) -> int:
    return _lib.load().attn_path_for_head_dim(int(d))


def workspace_bytes(B: int, H: int, L: int, d: int, causal: bool = False) -> int:
    return _lib.load().attn_workspace_bytes(B, H, L, d, 1 if causal else 0)


@contextmanager
def kernel_timing(result: dict):
    """Record HIP events around every kernel attn_forward queues inside the block.

    On exit ``result`` maps kernel name -> (total ms, launches).
    """
    lib = _lib.load()
    lib.attn_timing_collect(None, None, 0)  # drop stale records
    lib.attn_timing_enable(1)
    try:
        yield result
    finally:
        lib.attn_timing_enable(0)
        n = len(_lib.KERNEL_NAMES)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        st = lib.attn_timing_collect(ms, cnt, n)
        if st != _lib.ATTN_OK:
            raise _lib.AttnError(st, "attn_timing_collect")
        for i, name in enumerate(_lib.KERNEL_NAMES):
            if cnt[i]:
                result[name] = (ms[i], cnt[i])
