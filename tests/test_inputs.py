"""The seeded generator: deterministic, bf16, the workloads' shapes and seeds."""
import numpy as np
import torch

from synth import WORKLOADS, make_qkv
from synth.metrics import max_abs, rel_rms, within_bar


def test_deterministic_and_ordered():
    a = make_qkv(1, 2, 5, 8, seed=7)
    b = make_qkv(1, 2, 5, 8, seed=7)
    c = make_qkv(1, 2, 5, 8, seed=8)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape == (1, 2, 5, 8)
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    # q, k, v are consecutive draws of one generator, each rounded once to bf16
    g = torch.Generator().manual_seed(7)
    for x in a:
        assert torch.equal(x, torch.randn((1, 2, 5, 8), generator=g).to(torch.bfloat16))


def test_bf16_round_to_nearest_even():
    g = torch.Generator().manual_seed(3)
    f = torch.randn(4096, generator=g)
    bits = f.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = torch.randn(4096, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    assert np.array_equal(got.view(torch.int16).numpy().astype(np.int64) & 0xFFFF, rounded)


def test_workloads():
    w = WORKLOADS
    assert (w["wan_31frame"].B, w["wan_31frame"].L, w["wan_31frame"].d) == (31, 3432, 1024)
    assert w["wan_31frame"].flops() == 4 * 31 * 3432 ** 2 * 1024 == 1495602561024
    assert w["mha_d64_causal"].flops() == 4 * 32 * 64 * 1024 * 1025 // 2
    assert w["mha_d64"].seed == w["mha_d64_causal"].seed
    assert w["tiny_d256"].L == 13 * 22 and w["wan_1frame"].L == 44 * 78
    assert all(abs(x.scale - x.d ** -0.5) < 1e-15 for x in w.values())


def test_metrics():
    ref = np.array([1.0, -2.0, 2.0])
    out = ref + np.array([0.0, 0.01, -0.02])
    assert abs(max_abs(out, ref) - 0.02) < 1e-15
    assert abs(rel_rms(out, ref) - np.sqrt(0.0005) / 3.0) < 1e-15
    assert within_bar(ref, ref)[0]
    assert not within_bar(out, ref)[0]
