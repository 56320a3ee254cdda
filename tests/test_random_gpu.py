"""GPU parity on seeded random configurations of every entry point: head dims,
lengths, heads and key/value groups, masks, windows, layouts and (for the
token-packed entry) separate key lengths, each against the float64 oracle.

The configurations come from one fixed seed, so a failure names a reproducible
case; sizes stay small enough for the oracle to finish in a second or two.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_qkv
from synth.metrics import within_bar

from gpu_util import to_f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LSE_ATOL, LSE_RTOL = 4e-3, 1e-5
HEAD_DIMS = [32, 64, 128, 192, 256, 384, 512, 640, 1024]


@pytest.fixture(autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def _window(rng, L):
    kind = rng.integers(4)
    if kind == 0:
        return None
    left = None if kind == 1 else int(rng.integers(0, L + 1))
    right = None if kind == 2 else int(rng.integers(0, L + 1))
    return (left, right)


def _lse_ok(got, ref):
    empty = np.isneginf(ref)
    if not np.array_equal(np.isneginf(got), empty):
        return False
    g, r = np.where(empty, 0.0, got), np.where(empty, 0.0, ref)
    return bool(np.all(np.abs(g - r) <= LSE_ATOL + LSE_RTOL * np.abs(r)))


def _strided(t, rng):
    """The same values in one of three memory layouts: contiguous, heads
    interleaved in each row ([B, L, H, d]), or inside a wider row."""
    kind = rng.integers(3)
    if kind == 0:
        return t.to(DEV)
    if kind == 1:
        return t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    pad = 8 * int(rng.integers(1, 4))
    wide = torch.zeros(*t.shape[:-1], t.shape[-1] + pad, dtype=t.dtype)
    wide[..., : t.shape[-1]] = t
    return wide.to(DEV)[..., : t.shape[-1]]


@pytest.mark.parametrize("case", range(100))
def test_random_attention(case):
    from exact_softmax_attention_bf16_amd import attention
    rng = np.random.default_rng(9000 + case)
    d = int(rng.choice(HEAD_DIMS))
    B = int(rng.integers(1, 3))
    H_kv = int(rng.integers(1, 3))
    H = H_kv * int(rng.integers(1, 4))
    L = int(rng.integers(1, 700 if d <= 128 else 520))
    causal = bool(rng.integers(2))
    window = _window(rng, L)
    scale = float(rng.choice([1.0 / math.sqrt(d), 0.3, -0.2]))
    q = make_qkv(B, H, L, d, 10000 + case)[0]
    _, k, v = make_qkv(B, H_kv, L, d, 20000 + case)
    o, lse = attention(_strided(q, rng), _strided(k, rng), _strided(v, rng), scale=scale,
                       causal=causal, window=window, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale, causal, window)
    ok, a, r = within_bar(to_f64(o), ref)
    print(f"[random {case}] B={B} H={H}/{H_kv} L={L} d={d} causal={causal} window={window} "
          f"scale={scale:.3f}: max_abs={a:.2e} rel_rms={r:.2e}", flush=True)
    assert ok, (a, r)
    assert _lse_ok(to_f64(lse), oracle.log_sum_exp(to_f64(q), to_f64(k), scale, causal, window))


@pytest.mark.parametrize("case", range(40))
def test_random_varlen(case):
    from exact_softmax_attention_bf16_amd import attention_varlen
    rng = np.random.default_rng(9500 + case)
    d = int(rng.choice([32, 64, 128]))
    nseq = int(rng.integers(1, 6))
    H_kv = int(rng.integers(1, 3))
    H = H_kv * int(rng.integers(1, 4))
    cross = bool(rng.integers(2))
    q_len = [int(x) for x in rng.integers(0, 400, nseq)]
    k_len = [int(x) for x in rng.integers(0, 600, nseq)] if cross else q_len
    causal = bool(rng.integers(2))
    window = _window(rng, max(k_len + [1]))
    seqs = []
    for i in range(nseq):
        q = make_qkv(1, H, q_len[i], d, 30000 + 10 * case + i)[0]
        _, k, v = make_qkv(1, H_kv, k_len[i], d, 40000 + 10 * case + i)
        seqs.append((q, k, v))
    pack = lambda j, heads: torch.cat([s[j][0].transpose(0, 1) for s in seqs], 0).reshape(-1, heads, d).contiguous()
    cu_q = torch.tensor([0] + list(np.cumsum(q_len)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(k_len)), dtype=torch.int32)
    if sum(q_len) == 0:
        return
    kw = dict(cu_seqlens_k=cu_k.to(DEV), max_seqlen_k=max(k_len)) if cross else {}
    o, lse = attention_varlen(pack(0, H).to(DEV), pack(1, H_kv).to(DEV), pack(2, H_kv).to(DEV),
                              cu_q.to(DEV), max(q_len), causal=causal, window=window,
                              return_lse=True, **kw)
    torch.cuda.synchronize()
    s = 1.0 / math.sqrt(d)
    print(f"[random varlen {case}] d={d} H={H}/{H_kv} q={q_len} k={k_len} causal={causal} "
          f"window={window}", flush=True)
    for i, (q, k, v) in enumerate(seqs):
        a0, a1 = int(cu_q[i]), int(cu_q[i + 1])
        if a1 == a0:
            continue
        got = o[a0:a1].transpose(0, 1).unsqueeze(0).cpu()
        gl = to_f64(lse[a0:a1].transpose(0, 1).unsqueeze(0))
        if k_len[i] == 0:
            assert bool((got == 0).all()) and bool(np.isneginf(gl).all()), i
            continue
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, causal, window)
        ok, a, r = within_bar(to_f64(got), ref)
        assert ok, (i, a, r)
        assert _lse_ok(gl, oracle.log_sum_exp(to_f64(q), to_f64(k), s, causal, window)), i


@pytest.mark.parametrize("case", range(20))
def test_random_varlen_compressed(case):
    """The compressed causal mask on random batches: each sequence's keys are
    about Lq / cf of its queries (cf random in 1..16, lengths not multiples)."""
    from exact_softmax_attention_bf16_amd import attention_varlen
    rng = np.random.default_rng(9700 + case)
    d = int(rng.choice([32, 64, 128]))
    nseq = int(rng.integers(1, 6))
    H_kv = int(rng.integers(1, 3))
    H = H_kv * int(rng.integers(1, 4))
    q_len = [int(x) for x in rng.integers(0, 700, nseq)]
    k_len = [max(0, lq // int(rng.integers(1, 17)) + int(rng.integers(-2, 3))) for lq in q_len]
    seqs = []
    for i in range(nseq):
        q = make_qkv(1, H, q_len[i], d, 50000 + 10 * case + i)[0]
        _, k, v = make_qkv(1, H_kv, k_len[i], d, 60000 + 10 * case + i)
        seqs.append((q, k, v))
    if sum(q_len) == 0:
        return
    pack = lambda j, heads: torch.cat([s[j][0].transpose(0, 1) for s in seqs], 0).reshape(-1, heads, d).contiguous()
    cu_q = torch.tensor([0] + list(np.cumsum(q_len)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(k_len)), dtype=torch.int32)
    print(f"[random compressed {case}] d={d} H={H}/{H_kv} q={q_len} k={k_len}", flush=True)
    o, lse = attention_varlen(pack(0, H).to(DEV), pack(1, H_kv).to(DEV), pack(2, H_kv).to(DEV),
                              cu_q.to(DEV), max(q_len), causal="compressed", return_lse=True,
                              cu_seqlens_k=cu_k.to(DEV), max_seqlen_k=max(k_len + [1]))
    torch.cuda.synchronize()
    s = 1.0 / math.sqrt(d)
    for i, (q, k, v) in enumerate(seqs):
        a0, a1 = int(cu_q[i]), int(cu_q[i + 1])
        if a1 == a0:
            continue
        got = o[a0:a1].transpose(0, 1).unsqueeze(0).cpu()
        gl = to_f64(lse[a0:a1].transpose(0, 1).unsqueeze(0))
        if k_len[i] == 0:
            assert bool((got == 0).all()) and bool(np.isneginf(gl).all()), i
            continue
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, "compressed")
        ok, a, r = within_bar(to_f64(got), ref)
        assert ok, (i, a, r)
        lref = oracle.log_sum_exp(to_f64(q), to_f64(k), s, "compressed")
        assert bool((to_f64(got)[0][np.isneginf(lref)[0]] == 0).all()), i  # rows with no key
        assert _lse_ok(gl, lref), i
