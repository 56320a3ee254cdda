"""Exact softmax attention on MI355X (gfx950): bf16 in/out, fp32 accumulation.

    from exact_softmax_attention_bf16_amd import attention
    o = attention(q, k, v, scale=1/32, causal=False)   # q, k, v: bf16 [B,H,L,d] on the GPU

The computation runs in hand-written HIP kernels behind a C ABI
(include/attn.h, libattn_mi355x.so); this package only marshals arguments.
"""
from ._lib import AttnError, LIB_PATH, load, status_string
from .api import attention, kernel_timing, path_for_head_dim, workspace_bytes

__all__ = ["AttnError", "LIB_PATH", "attention", "kernel_timing", "load", "path_for_head_dim",
           "status_string", "workspace_bytes"]
