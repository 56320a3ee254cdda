"""attn_forward_noalloc on the GPU: called through the C ABI, its output against
attn_forward's (the entry point it is a variant of) and the oracle, on two calls
in a row with the second smaller, for each path that draws scratch memory:
the large-head-dim two passes (exponentials and statistics; several chunks of
heads when they do not fit the fixed array at once; the values pass's key
split, dropped when its shares do not fit; its 128 x 128 tiles for one head)
and the online path's key split.
"""
import ctypes
import math

import pytest
import torch

import oracle
from synth import make_qkv
from synth.metrics import REL_RMS_BAND, within_bar

from gpu_util import to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def call(fn, q, k, v, out, scale, causal):
    from exact_softmax_attention_bf16_amd import _lib
    B, H, L, d = q.shape
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, d, float(scale),
            1 if causal else 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.ATTN_OK, _lib.status_string(st)


# (B, H, L, d, causal): first call, then a smaller second call
PAIRS = [
    ((6, 1, 3432, 1024, False), (1, 1, 1000, 512, False)),   # 6 frames: two chunks of heads
    ((1, 1, 3432, 1024, False), (1, 1, 700, 256, True)),     # one frame: 128 x 128 values tiles
    ((2, 1, 3432, 1024, False), (1, 1, 1000, 512, False)),   # two frames: split shares 56 MB
    ((1, 1, 4096, 64, False), (1, 1, 1000, 128, True)),      # online key split
    ((2, 1, 2000, 768, True), (1, 2, 300, 192, False)),
    ((1, 1, 6500, 1024, False), (1, 1, 3000, 1024, False)),  # split's shares do not fit: dropped
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_attn_forward(first, second):
    from exact_softmax_attention_bf16_amd import _lib
    lib = _lib.load()
    dev = torch.device("cuda:0")
    for i, (B, H, L, d, causal) in enumerate((first, second)):
        print(f"[noalloc] call {i}: B={B} H={H} L={L} d={d} causal={causal}", flush=True)
        q, k, v = make_qkv(B, H, L, d, 900 + 10 * i + L % 7)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        s = 1.0 / math.sqrt(d)
        o_na = torch.full_like(qd, float("nan"))
        o_ref = torch.empty_like(qd)
        call(lib.attn_forward_noalloc, qd, kd, vd, o_na, s, causal)
        call(lib.attn_forward, qd, kd, vd, o_ref, s, causal)
        torch.cuda.synchronize()
        ok, a, r = within_bar(to_f64(o_na), to_f64(o_ref))
        print(f"[noalloc]   against attn_forward: max_abs={a:.2e} rel_rms={r:.2e}", flush=True)
        assert ok, (a, r)
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, causal)
        ok, a, r = within_bar(to_f64(o_na), ref)
        print(f"[noalloc]   against the oracle: max_abs={a:.2e} rel_rms={r:.2e}", flush=True)
        assert ok and r <= REL_RMS_BAND, (a, r)


def test_noalloc_too_large_is_refused_and_queues_nothing():
    from exact_softmax_attention_bf16_amd import _lib
    lib = _lib.load()
    dev = torch.device("cuda:0")
    L, d = 8000, 1024
    x = torch.zeros(1, 1, L, d, dtype=torch.bfloat16, device=dev)
    out = torch.full_like(x, 7.0)
    st = lib.attn_forward_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), out.data_ptr(), 1, 1,
                                  L, d, 0.03125, 0,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == _lib.ATTN_ERR_SCRATCH_TOO_SMALL
    assert bool((out == 7.0).all())
