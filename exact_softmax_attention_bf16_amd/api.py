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


def _check(t: torch.Tensor, name: str, shape: tuple | None = None,
           device: torch.device | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP (cuda) device, got {t.device}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, heads, L, d], got shape {tuple(t.shape)}")
    if t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have contiguous channels (last stride 1)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}")


def _strides(t: torch.Tensor):
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def _call(fn, q: torch.Tensor, *args) -> None:
    """Call a forward entry point on q's device and its current stream."""
    if q.device.index == torch.cuda.current_device():
        status = fn(*args, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    else:  # the library launches on the current device: switch to q's for the call
        with torch.cuda.device(q.device):
            status = fn(*args, ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream))
    if status != _lib.ATTN_OK:
        raise _lib.AttnError(status, fn.__name__)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
              causal: bool = False, out: torch.Tensor | None = None, return_lse: bool = False,
              window: tuple | None = None):
    """O = softmax(scale * Q K^T) V on bf16 tensors (HIP kernels only).

    q is [B, H, L, d]; k and v are [B, H_kv, L, d] with H_kv dividing H (query
    head h reads key/value head h // (H / H_kv): grouped or multi-query
    attention).  Any strides with contiguous channels are read in place
    (strides must be multiples of 8 elements).  ``scale`` defaults to 1/sqrt(d).
    ``out``, if given, is a bf16 [B, H, L, d] tensor (any strides whose elements
    do not overlap) that overlaps none of the inputs.  With ``return_lse`` the
    result is (out, lse), lse float32 [B, H, L] holding each row's
    log(sum_j exp(scale * q . k_j)).  ``window = (left, right)`` is a sliding
    window: query i sees only keys i - left .. i + right (None on a side:
    unbounded); causal also caps right at 0.  Work is queued on the current
    stream of q's device.
    """
    _check(q, "q")
    B, H, L, d = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("k must be a 4-D tensor [B, H_kv, L, d]")
    H_kv = k.shape[1]
    _check(k, "k", (B, H_kv, L, d), q.device)
    _check(v, "v", (B, H_kv, L, d), q.device)
    if H_kv == 0 and H > 0 or H_kv > 0 and H % H_kv != 0:
        raise ValueError(f"key/value heads ({H_kv}) must divide query heads ({H})")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check(out, "out", (B, H, L, d), q.device)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if return_lse else None
    wl, wr = _window_args(window)
    lib = _lib.load()
    plain = (H_kv == H and lse is None and window is None
             and all(t.is_contiguous() for t in (q, k, v, out)))
    if plain:
        _call(lib.attn_forward, q, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
              B, H, L, d, float(scale), 1 if causal else 0)
    else:
        _call(lib.attn_forward_ex, q, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
              lse.data_ptr() if lse is not None else None, B, H, H_kv, L, d,
              _strides(q), _strides(k), _strides(v), _strides(out), float(scale),
              1 if causal else 0, wl, wr)
    return (out, lse) if return_lse else out


def attention_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                      scale: float | None = None, causal: bool = False) -> torch.Tensor:
    """attention() for callers that cannot allocate device memory (HIP graph
    capture, tight serving loops): contiguous bf16 [B, H, L, d] q, k, v and a
    caller-provided ``out``; the library draws its scratch memory from a fixed
    per-device array instead of allocating (attn_forward_noalloc).  Calls whose
    work may overlap on one GPU race on that array.  Raises AttnError with
    ATTN_ERR_SCRATCH_TOO_SMALL when one head needs more scratch than the array
    holds (d > 128 with L above 7936)."""
    _check(q, "q")
    B, H, L, d = q.shape
    for t, name in ((k, "k"), (v, "v"), (out, "out")):
        _check(t, name, (B, H, L, d), q.device)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _call(_lib.load().attn_forward_noalloc, q, q.data_ptr(), k.data_ptr(), v.data_ptr(),
          out.data_ptr(), B, H, L, d, float(scale), 1 if causal else 0)
    return out


def _window_args(window):
    if window is None:
        return -1, -1
    wl, wr = (-1 if w is None else int(w) for w in window)
    if wl < 0 and window[0] is not None or wr < 0 and window[1] is not None:
        raise ValueError(f"window sides must be >= 0 or None, got {window}")
    return wl, wr


def attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                     max_seqlen: int, scale: float | None = None, causal: bool | str = False,
                     out: torch.Tensor | None = None, return_lse: bool = False,
                     window: tuple | None = None, cu_seqlens_k: torch.Tensor | None = None,
                     max_seqlen_k: int | None = None):
    """Attention over a batch of sequences of different lengths packed along the
    tokens (the cum_seqlen interface of cuDNN's FMHA example): q is
    [total, H, d], k and v [total_k, H_kv, d], cu_seqlens an int32 tensor of
    B + 1 offsets on the same device (sequence b's queries are tokens
    cu_seqlens[b] .. cu_seqlens[b + 1] - 1), max_seqlen >= the longest.  With
    ``cu_seqlens_k`` (and ``max_seqlen_k``) the keys have offsets of their own
    (cross-attention, or a few queries against a cache; query i then stands at
    key position i + Lk - Lq for causal and windows); otherwise they share the
    query offsets.  ``causal="compressed"`` is that example's compressed causal
    mask: with cf = max(1, Lq // Lk) per sequence, query i sees keys
    j <= (i + 1) // cf - 1 (no window allowed).  d must be 32, 64 or 128.
    Returns out [total, H, d] (and lse float32 [total, H] with ``return_lse``);
    rows of tokens in no sequence are left as they were, rows that see no key
    are 0."""
    if isinstance(causal, str):
        if causal != "compressed":
            raise ValueError(f"causal must be a bool or 'compressed', got {causal!r}")
        mask = _lib.ATTN_MASK_COMPRESSED_CAUSAL
    else:
        mask = _lib.ATTN_MASK_CAUSAL if causal else _lib.ATTN_MASK_NONE
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [total, H, d]")
    total, H, d = q.shape
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError(f"{name} must be a 3-D tensor [tokens, heads, d]")
        _check(t.unsqueeze(0), name)
    total_k, H_kv = k.shape[0], k.shape[1]
    if cu_seqlens_k is None and total_k != total:
        raise ValueError("without cu_seqlens_k, k and v must have q's token count")
    if tuple(k.shape) != (total_k, H_kv, d) or tuple(v.shape) != (total_k, H_kv, d):
        raise ValueError(f"k and v must be [total_k, H_kv, d] = [{total_k}, {H_kv}, {d}]")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    if H_kv == 0 and H > 0 or H_kv > 0 and H % H_kv != 0:
        raise ValueError(f"key/value heads ({H_kv}) must divide query heads ({H})")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32
            or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device or cu_seqlens.numel() < 1):
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of B + 1 offsets on q's device")
    cu = cu_seqlens.contiguous()
    B = cu.numel() - 1
    cuk = None
    if cu_seqlens_k is not None:
        if (not isinstance(cu_seqlens_k, torch.Tensor) or cu_seqlens_k.dtype != torch.int32
                or tuple(cu_seqlens_k.shape) != (B + 1,) or cu_seqlens_k.device != q.device):
            raise ValueError("cu_seqlens_k must be an int32 tensor like cu_seqlens")
        if max_seqlen_k is None:
            raise ValueError("cu_seqlens_k needs max_seqlen_k")
        cuk = cu_seqlens_k.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((total, H, d), dtype=torch.bfloat16, device=q.device)
    else:
        if not isinstance(out, torch.Tensor) or out.dim() != 3 or tuple(out.shape) != (total, H, d):
            raise ValueError(f"out must be [total, H, d] = [{total}, {H}, {d}]")
        _check(out.unsqueeze(0), "out", device=q.device)
    lse = torch.empty((total, H), dtype=torch.float32, device=q.device) if return_lse else None
    wl, wr = _window_args(window)
    st = lambda t: (ctypes.c_int64 * 2)(*t.stride()[:2])
    _call(_lib.load().attn_forward_varlen, q, q.data_ptr(), k.data_ptr(), v.data_ptr(),
          out.data_ptr(), lse.data_ptr() if lse is not None else None, cu.data_ptr(), B,
          int(max_seqlen), total, cuk.data_ptr() if cuk is not None else None,
          int(max_seqlen_k) if cuk is not None else 0, total_k, H, H_kv, d, st(q), st(k), st(v),
          st(out), float(scale), mask, wl, wr)
    return (out, lse) if return_lse else out


def attention_packed_qkv(qkv: torch.Tensor, scale: float | None = None, causal: bool = False,
                         out: torch.Tensor | None = None, return_lse: bool = False,
                         window: tuple | None = None):
    """Attention over a packed [B, H, L, 3d] tensor whose last dimension holds
    q, k and v in that order -- the [T, 1, HW, 3C] qkv of the FastVideo Wan2.2
    VAE decoder's attention (frames T as B, one head) -- read in place through
    strides, with no copy.  Returns out [B, H, L, d] (and lse, as attention())."""
    _check(qkv, "qkv")
    if qkv.shape[-1] % 3 != 0:
        raise ValueError(f"qkv's last dimension ({qkv.shape[-1]}) must be 3 * d")
    d = qkv.shape[-1] // 3
    q, k, v = qkv[..., :d], qkv[..., d:2 * d], qkv[..., 2 * d:]
    return attention(q, k, v, scale=scale, causal=causal, out=out, return_lse=return_lse,
                     window=window)


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
