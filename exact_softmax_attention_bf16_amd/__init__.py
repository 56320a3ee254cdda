"""Exact softmax attention on MI355X (gfx950): bf16 in/out, fp32 accumulation.

    from exact_softmax_attention_bf16_amd import attention
    o = attention(q, k, v, scale=1/32, causal=False)   # q, k, v: bf16 [B,H,L,d] on the GPU
    o, lse = attention(q, k, v, return_lse=True)       # k, v may have fewer heads; any strides
    o = attention_packed_qkv(qkv)                      # qkv: [T, 1, HW, 3C], read in place
    o = attention_varlen(q, k, v, cu_seqlens, max_seqlen)  # [total, H, d] token-packed batch
    attention_noalloc(q, k, v, out)                    # no device allocation (fixed scratch)

The computation runs in hand-written HIP kernels behind a C ABI
(include/attn.h, libattn_mi355x.so); this package only marshals arguments.
"""
from ._lib import AttnError, LIB_PATH, load, status_string
from .api import (attention, attention_noalloc, attention_packed_qkv, attention_varlen,
                  kernel_timing, path_for_head_dim, workspace_bytes)

__all__ = ["AttnError", "LIB_PATH", "attention", "attention_noalloc", "attention_packed_qkv",
           "attention_varlen", "kernel_timing", "load", "path_for_head_dim", "status_string",
           "workspace_bytes"]
