"""The split-columns design probe (include/attn_probe.h) computes attention:
its output against the oracle, element by element, at sizes that span
several 64-row workgroups, several 32-key blocks and a ragged tail."""
import ctypes
import os

import pytest
import torch

import oracle
from synth import make_qkv
from synth.metrics import REL_RMS_BAND, within_bar

from gpu_util import to_f64

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE_LIB = os.path.join(ROOT, "exact_softmax_attention_bf16_amd", "libattn_probe.so")


def probe():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"probe library not built: {PROBE_LIB}")
    f = ctypes.CDLL(PROBE_LIB).attn_probe_split_columns
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_void_p]
    return f


@pytest.mark.parametrize("B,H,L", [(1, 1, 1), (1, 2, 63), (2, 1, 200), (1, 1, 417)])
def test_split_columns_probe_matches_oracle(B, H, L):
    d, scale = 1024, 1.0 / 32
    print(f"[probe test] B={B} H={H} L={L}", flush=True)
    q, k, v = make_qkv(B, H, L, d, 11 + L)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.full_like(qd, float("nan"))
    st = probe()(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), B, H, L, d,
                 scale, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, False)
    ok, a, r = within_bar(to_f64(out), ref)
    assert ok and r <= REL_RMS_BAND, (a, r)
