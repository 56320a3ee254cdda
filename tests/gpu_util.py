"""Helpers for the GPU parity tests (test infrastructure)."""
import numpy as np
import torch

import oracle
from synth import make_qkv
from synth.metrics import within_bar


def to_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 (or any float) tensor -> float64 numpy, exactly."""
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(q, k, v, scale, causal, out=None):
    from exact_softmax_attention_bf16_amd import attention
    dev = torch.device("cuda:0")
    o = attention(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal, out=out)
    torch.cuda.synchronize()
    return o


def check_full(B, H, L, d, scale, causal, seed):
    q, k, v = make_qkv(B, H, L, d, seed)
    o = run_gpu(q, k, v, scale, causal)
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, causal)
    ok, a, r = within_bar(to_f64(o), ref)
    return ok, a, r, o, (q, k, v), ref
