"""GPU parity for attn_forward_ex and attn_forward_varlen: packed and permuted
layouts read in place, grouped key/value heads, sliding windows, token-packed
sequences of different lengths and the log-sum-exp output, against the float64
oracle.

Output bar as in test_parity_gpu.py.  LSE bar, from the arithmetic: the kernels
sum the bf16-rounded exponentials they multiply (bf16 keeps 8 significant
bits, so round-to-nearest errs by at most 2^-8 relative per term, hence in the
sum), so the denominator's log is off by at most ln(1 + 2^-8) < 3.90e-3, plus
fp32 rounding of the logits and of the final scaling (well under 1e-5 relative
at these sizes): |lse - ref| <= 4e-3 + 1e-5 |ref|.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_qkv
from synth.metrics import REL_RMS_BAND, within_bar

from gpu_util import to_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LSE_ATOL, LSE_RTOL = 4e-3, 1e-5


@pytest.fixture(autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def _report(name, a, r):
    print(f"[layouts] {name}: max_abs={a:.3e} rel_rms={r:.3e}", flush=True)


def lse_ok(got, ref):
    err = np.abs(to_f64(got) - ref)
    return bool(np.all(err <= LSE_ATOL + LSE_RTOL * np.abs(ref))), float(err.max())


def packed(T, HW, C, seed):
    q, k, v = make_qkv(T, 1, HW, C, seed)
    return torch.cat([q, k, v], dim=-1).contiguous(), (q, k, v)


@pytest.mark.parametrize("C", [64, 128, 256, 1024])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_qkv_in_place(C, causal):
    from exact_softmax_attention_bf16_amd import attention_packed_qkv
    T, HW = 2, 300
    qkv, (q, k, v) = packed(T, HW, C, 100 + C)
    qkv_d = qkv.to(DEV)
    o = attention_packed_qkv(qkv_d, scale=1.0 / math.sqrt(C), causal=causal)
    torch.cuda.synchronize()
    assert o.shape == (T, 1, HW, C)
    assert torch.equal(qkv_d.cpu(), qkv)  # read only
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(C), causal)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"packed qkv C={C} causal={causal}", a, r)
    assert ok, (a, r)


def test_packed_qkv_wan_frames():
    """The decoder's packed layout at its real size: 4 frames of 44 x 78
    positions, C = 1024, every output element against the oracle."""
    from exact_softmax_attention_bf16_amd import attention_packed_qkv
    T, HW, C = 4, 3432, 1024
    qkv, (q, k, v) = packed(T, HW, C, 104)
    o = attention_packed_qkv(qkv.to(DEV), scale=1.0 / 32, causal=False)
    torch.cuda.synchronize()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / 32, False)
    ok, a, r = within_bar(to_f64(o), ref)
    _report("packed qkv 4 x 3432 x 1024", a, r)
    assert ok, (a, r)
    assert r <= REL_RMS_BAND, (r, REL_RMS_BAND)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_permuted_layouts(d, causal):
    """q, k, v and out stored as [B, L, H, d] (heads interleaved in each row)."""
    from exact_softmax_attention_bf16_amd import attention
    B, H, L = 2, 3, 261
    q, k, v = make_qkv(B, H, L, d, 110 + d)
    perm = [t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v)]
    out = torch.empty(B, L, H, d, dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    o = attention(*perm, scale=1.0 / math.sqrt(d), causal=causal, out=out)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(d), causal)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"permuted d={d} causal={causal}", a, r)
    assert ok, (a, r)


@pytest.mark.parametrize("H,H_kv", [(8, 2), (8, 1), (6, 3), (4, 4)])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_key_value_heads(H, H_kv, d, causal):
    from exact_softmax_attention_bf16_amd import attention
    B, L = 2, 257
    q = make_qkv(B, H, L, d, 120 + H)[0]
    _, k, v = make_qkv(B, H_kv, L, d, 121 + H_kv)
    o = attention(q.to(DEV), k.to(DEV), v.to(DEV), scale=1.0 / math.sqrt(d), causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(d), causal)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"H={H} H_kv={H_kv} d={d} causal={causal}", a, r)
    assert ok, (a, r)


def test_zero_stride_broadcast_equals_multi_query():
    """One key/value head given as a head-stride-0 view equals H_kv = 1."""
    from exact_softmax_attention_bf16_amd import attention
    B, H, L, d = 2, 4, 300, 64
    q = make_qkv(B, H, L, d, 130)[0].to(DEV)
    _, k, v = (t.to(DEV) for t in make_qkv(B, 1, L, d, 131))
    o1 = attention(q, k, v)
    o2 = attention(q, k.expand(B, H, L, d), v.expand(B, H, L, d))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("d", [32, 64, 128, 256, 1024])
@pytest.mark.parametrize("L", [1, 130, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_lse(d, L, causal):
    from exact_softmax_attention_bf16_amd import attention
    B, H = 2, 2
    q, k, v = make_qkv(B, H, L, d, 140 + L + d)
    s = 1.0 / math.sqrt(d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = attention(qd, kd, vd, scale=s, causal=causal, return_lse=True)
    o_plain = attention(qd, kd, vd, scale=s, causal=causal)
    torch.cuda.synchronize()
    assert lse.shape == (B, H, L) and lse.dtype == torch.float32
    assert torch.equal(o, o_plain)  # the same kernels; lse is an extra store
    ok, err = lse_ok(lse, oracle.log_sum_exp(to_f64(q), to_f64(k), s, causal))
    print(f"[layouts] lse d={d} L={L} causal={causal}: max err {err:.3e}", flush=True)
    assert ok, err


def test_lse_scale_zero_is_log_count():
    from exact_softmax_attention_bf16_amd import attention
    L = 500
    q, k, v = (t.to(DEV) for t in make_qkv(1, 1, L, 256, 150))
    _, lse = attention(q, k, v, scale=0.0, causal=True, return_lse=True)
    torch.cuda.synchronize()
    ok, err = lse_ok(lse[0, 0], np.log(np.arange(1, L + 1)))
    assert ok, err


@pytest.mark.parametrize("B,L,d,split", [(1, 1100, 256, False), (1, 2100, 512, False),
                                         (12, 2048, 256, True), (10, 1600, 256, True)])
def test_few_heads_with_strided_out_and_lse(B, L, d, split):
    """Few heads: the values pass either runs on 128 x 128 tiles (one head) or
    splits its keys, whose reduction then writes the strided out (row stride
    2d) while the first split writes the LSE."""
    from exact_softmax_attention_bf16_amd import attention, kernel_timing
    q, k, v = make_qkv(B, 1, L, d, 160 + L)
    s = 1.0 / math.sqrt(d)
    big = torch.full((B, 1, L, 2 * d), 7.0, dtype=torch.bfloat16, device=DEV)
    out = big[..., :d]
    res = {}
    with kernel_timing(res):
        o, lse = attention(q.to(DEV), k.to(DEV), v.to(DEV), scale=s, out=out, return_lse=True)
    torch.cuda.synchronize()
    assert ("values_reduce" in res) == split
    assert bool((big[..., d:] == 7.0).all())  # the gaps between rows are untouched
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, False)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"few heads + strided out B={B} L={L} d={d}", a, r)
    assert ok, (a, r)
    ok, err = lse_ok(lse, oracle.log_sum_exp(to_f64(q), to_f64(k), s, False))
    assert ok, err


def test_ex_with_default_strides_equals_attn_forward():
    """attn_forward_ex with NULL strides and H_kv = H is attn_forward."""
    import ctypes
    from exact_softmax_attention_bf16_amd import _lib, attention
    for d in (64, 1024):
        q, k, v = (t.to(DEV) for t in make_qkv(2, 2, 700, d, 170 + d))
        ref = attention(q, k, v)
        out = torch.empty_like(q)
        st = _lib.load().attn_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         None, 2, 2, 2, 700, d, None, None, None, None,
                                         1.0 / math.sqrt(d), 0, -1, -1,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == _lib.ATTN_OK
        assert torch.equal(out, ref)


# ---- sliding windows -------------------------------------------------------------

WINDOWS = [(0, 0), (5, 3), (100, 0), (0, 100), (300, 200), (None, 70), (130, None), (1, 1000)]


@pytest.mark.parametrize("d", [64, 128, 256, 1024])
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
def test_window(d, window, causal):
    from exact_softmax_attention_bf16_amd import attention
    B, H, L = 1, 2, 700
    q, k, v = make_qkv(B, H, L, d, 180 + d)
    s = 1.0 / math.sqrt(d)
    o, lse = attention(q.to(DEV), k.to(DEV), v.to(DEV), scale=s, causal=causal, window=window,
                       return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, causal, window)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"window {window} d={d} causal={causal}", a, r)
    assert ok, (a, r)
    ok, err = lse_ok(lse, oracle.log_sum_exp(to_f64(q), to_f64(k), s, causal, window))
    assert ok, err


@pytest.mark.parametrize("d", [64, 256])
def test_window_of_width_zero_returns_v_exactly(d):
    # one allowed key: p = e / e in fp32 times a bf16 value rounds back to it
    from exact_softmax_attention_bf16_amd import attention
    q, k, v = (t.to(DEV) for t in make_qkv(2, 2, 531, d, 190))
    o = attention(q, k, v, window=(0, 0))
    torch.cuda.synchronize()
    assert torch.equal(o, v)


@pytest.mark.parametrize("d", [64, 1024])
def test_window_limits_equal_unwindowed_and_causal_bitwise(d):
    from exact_softmax_attention_bf16_amd import attention
    L = 600
    q, k, v = (t.to(DEV) for t in make_qkv(1, 2, L, d, 191))
    full = attention(q, k, v)
    causal = attention(q, k, v, causal=True)
    wide = attention(q, k, v, window=(L, L))
    left_only = attention(q, k, v, window=(None, 0))
    torch.cuda.synchronize()
    assert torch.equal(wide, full)
    assert torch.equal(left_only, causal)


@pytest.mark.parametrize("B,L,d,window,split", [(1, 2100, 512, (300, 200), False),
                                                 (1, 1100, 256, (None, 0), False),
                                                 (1, 1500, 256, (600, None), False),
                                                 (12, 2048, 256, (1200, 1200), True),
                                                 (10, 1600, 256, (900, None), True)])
def test_window_with_few_heads(B, L, d, window, split):
    """Few heads: each query tile's band on the 128 x 128 tiles, or divided
    among the workgroups of a key split."""
    from exact_softmax_attention_bf16_amd import attention, kernel_timing
    q, k, v = make_qkv(B, 1, L, d, 192 + L)
    s = 1.0 / math.sqrt(d)
    res = {}
    with kernel_timing(res):
        o, lse = attention(q.to(DEV), k.to(DEV), v.to(DEV), scale=s, window=window, return_lse=True)
    torch.cuda.synchronize()
    assert ("values_reduce" in res) == split
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, False, window)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"few heads window {window} B={B} L={L} d={d}", a, r)
    assert ok, (a, r)
    ok, err = lse_ok(lse, oracle.log_sum_exp(to_f64(q), to_f64(k), s, False, window))
    assert ok, err


def test_window_on_packed_grouped_strided_inputs():
    from exact_softmax_attention_bf16_amd import attention
    B, H, H_kv, L, d = 2, 4, 2, 450, 256
    q = make_qkv(B, H, L, d, 193)[0]
    _, k, v = make_qkv(B, H_kv, L, d, 194)
    perm = [t.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for t in (q, k, v)]
    o = attention(*perm, window=(40, 90), causal=True)
    torch.cuda.synchronize()
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(d), True, (40, 90))
    ok, a, r = within_bar(to_f64(o), ref)
    assert ok, (a, r)


# ---- token-packed sequences of different lengths ----------------------------------

def varlen_batch(lengths, H, H_kv, d, seed, lead=0, tail=0):
    """Per-sequence inputs [1, heads, L, d] and their token-packed [total, heads, d]
    form; `lead` / `tail` tokens before the first and after the last sequence."""
    seqs = []
    for i, L in enumerate(lengths):
        q = make_qkv(1, H, L, d, seed + 2 * i)[0]
        _, k, v = make_qkv(1, H_kv, L, d, seed + 2 * i + 1)
        seqs.append((q, k, v))
    def pack(j, heads):
        parts = [torch.zeros(lead, heads, d, dtype=torch.bfloat16)]
        parts += [s[j][0].transpose(0, 1) for s in seqs]
        parts += [torch.zeros(tail, heads, d, dtype=torch.bfloat16)]
        return torch.cat(parts, dim=0).contiguous()
    cu = torch.tensor([lead] + list(lead + np.cumsum(lengths)), dtype=torch.int32)
    return seqs, pack(0, H), pack(1, H_kv), pack(2, H_kv), cu


def check_varlen(seqs, o, lse, cu, s, causal, window):
    worst = (0.0, 0.0)
    for i, (q, k, v) in enumerate(seqs):
        a0, a1 = int(cu[i]), int(cu[i + 1])
        if a1 == a0:
            continue  # an empty sequence: nothing to compare
        got = o[a0:a1].transpose(0, 1).unsqueeze(0)
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, causal, window)
        ok, a, r = within_bar(to_f64(got), ref)
        assert ok, (i, a, r)
        worst = (max(worst[0], a), max(worst[1], r))
        if lse is not None:
            ok, err = lse_ok(lse[a0:a1].transpose(0, 1).unsqueeze(0),
                             oracle.log_sum_exp(to_f64(q), to_f64(k), s, causal, window))
            assert ok, (i, err)
    return worst


LENGTHS = [1, 300, 17, 129, 0, 1000, 64]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [None, (50, 10)])
def test_varlen(d, H, H_kv, causal, window):
    from exact_softmax_attention_bf16_amd import attention_varlen
    seqs, q, k, v, cu = varlen_batch(LENGTHS, H, H_kv, d, 200 + d)
    s = 1.0 / math.sqrt(d)
    o, lse = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), max(LENGTHS), scale=s,
                              causal=causal, window=window, return_lse=True)
    torch.cuda.synchronize()
    a, r = check_varlen(seqs, o.cpu(), lse.cpu(), cu, s, causal, window)
    _report(f"varlen d={d} H={H}/{H_kv} causal={causal} window={window}", a, r)


def test_varlen_tokens_outside_sequences_untouched_and_strided():
    """Sequences start after 40 unused tokens and end 24 before the last; q, k, v
    are views into one [total, 3, H, d] tensor; out keeps its other rows."""
    from exact_softmax_attention_bf16_amd import attention_varlen
    H, d = 2, 64
    seqs, q, k, v, cu = varlen_batch([200, 77, 513], H, H, d, 230, lead=40, tail=24)
    packed = torch.stack([q, k, v], dim=1).to(DEV)  # [total, 3, H, d]
    total = q.shape[0]
    out = torch.full((total, H, d), 3.0, dtype=torch.bfloat16, device=DEV)
    o = attention_varlen(packed[:, 0], packed[:, 1], packed[:, 2], cu.to(DEV), 600, out=out)
    torch.cuda.synchronize()
    assert bool((o[:40] == 3.0).all()) and bool((o[total - 24:] == 3.0).all())
    check_varlen(seqs, o.cpu(), None, cu, 1.0 / math.sqrt(d), False, None)


def test_varlen_equals_separate_calls_bitwise():
    """Each sequence of a varlen call equals attention() on that sequence alone."""
    from exact_softmax_attention_bf16_amd import attention, attention_varlen
    H, d = 4, 128
    seqs, q, k, v, cu = varlen_batch([333, 128, 5], H, H, d, 240)
    o = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), 333, causal=True)
    for i, (qs, ks, vs) in enumerate(seqs):
        ref = attention(qs.to(DEV), ks.to(DEV), vs.to(DEV), causal=True)
        got = o[int(cu[i]):int(cu[i + 1])].transpose(0, 1).unsqueeze(0)
        assert torch.equal(got, ref), i


# ---- query and key lengths that differ (cross-attention, decoding) -----------

def qk_batch(q_lengths, k_lengths, H, H_kv, d, seed):
    seqs = []
    for i, (lq, lk) in enumerate(zip(q_lengths, k_lengths)):
        q = make_qkv(1, H, lq, d, seed + 3 * i)[0]
        _, k, v = make_qkv(1, H_kv, lk, d, seed + 3 * i + 1)
        seqs.append((q, k, v))
    def pack(j, heads):
        return torch.cat([s[j][0].transpose(0, 1) for s in seqs], dim=0).reshape(-1, heads, d).contiguous()
    cu_q = torch.tensor([0] + list(np.cumsum(q_lengths)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(k_lengths)), dtype=torch.int32)
    return seqs, pack(0, H), pack(1, H_kv), pack(2, H_kv), cu_q, cu_k


def check_qk(seqs, o, lse, cu_q, s, causal, window):
    for i, (q, k, v) in enumerate(seqs):
        a0, a1 = int(cu_q[i]), int(cu_q[i + 1])
        if a1 == a0:
            continue
        got = o[a0:a1].transpose(0, 1).unsqueeze(0)
        gl = lse[a0:a1].transpose(0, 1).unsqueeze(0)
        if k.shape[2] == 0:  # no keys at all: every row is 0
            assert bool((got == 0).all()) and bool(torch.isneginf(gl).all()), i
            continue
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, causal, window)
        ok, a, r = within_bar(to_f64(got), ref)
        assert ok, (i, a, r)
        lref = oracle.log_sum_exp(to_f64(q), to_f64(k), s, causal, window)
        lg = to_f64(gl)
        empty = np.isneginf(lref)
        assert np.array_equal(np.isneginf(lg), empty), i
        assert bool((to_f64(got)[..., empty[0, :, :], :] == 0).all()) if empty.any() else True
        ok, err = lse_ok(torch.from_numpy(np.where(empty, 0.0, lg)), np.where(empty, 0.0, lref))
        assert ok, (i, err)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [None, (40, 20)])
def test_varlen_separate_key_lengths(d, causal, window):
    from exact_softmax_attention_bf16_amd import attention_varlen
    q_len = [1, 37, 300, 128, 0, 90, 200]
    k_len = [500, 37, 64, 700, 10, 0, 130]
    H, H_kv = 4, 2
    seqs, q, k, v, cu_q, cu_k = qk_batch(q_len, k_len, H, H_kv, d, 500 + d)
    s = 1.0 / math.sqrt(d)
    o, lse = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), max(q_len), scale=s,
                              causal=causal, window=window, return_lse=True,
                              cu_seqlens_k=cu_k.to(DEV), max_seqlen_k=max(k_len))
    torch.cuda.synchronize()
    check_qk(seqs, o.cpu(), lse.cpu(), cu_q, s, causal, window)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_one_query_per_sequence(d):
    """One new token per sequence against caches of different lengths."""
    from exact_softmax_attention_bf16_amd import attention_varlen
    k_len = [1, 17, 1000, 4096, 2500, 64, 333, 2048]
    q_len = [1] * len(k_len)
    H, H_kv = 8, 2
    seqs, q, k, v, cu_q, cu_k = qk_batch(q_len, k_len, H, H_kv, d, 600 + d)
    s = 1.0 / math.sqrt(d)
    o, lse = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), 1, scale=s,
                              causal=True, return_lse=True, cu_seqlens_k=cu_k.to(DEV),
                              max_seqlen_k=max(k_len))
    torch.cuda.synchronize()
    check_qk(seqs, o.cpu(), lse.cpu(), cu_q, s, True, None)


def test_queries_past_the_keys_are_zero():
    """Lq > Lk with causal: the first Lq - Lk queries see no key."""
    from exact_softmax_attention_bf16_amd import attention_varlen
    seqs, q, k, v, cu_q, cu_k = qk_batch([300], [100], 2, 2, 64, 700)
    o, lse = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), 300, causal=True,
                              return_lse=True, cu_seqlens_k=cu_k.to(DEV), max_seqlen_k=100)
    torch.cuda.synchronize()
    assert bool((o[:200] == 0).all()) and bool(torch.isneginf(lse[:200]).all())
    check_qk(seqs, o.cpu(), lse.cpu(), cu_q, 0.125, True, None)


# ---- the compressed causal mask (keys compress the queries) ------------------

@pytest.mark.parametrize("d", [32, 64, 128])
def test_varlen_compressed_causal(d):
    """cf = Lq // Lk per sequence (1 when Lq < Lk or Lq == Lk): query i sees keys
    j <= (i + 1) // cf - 1; the first cf - 1 queries see none and give 0."""
    from exact_softmax_attention_bf16_amd import attention_varlen
    q_len = [300, 1000, 128, 37, 64, 257, 1, 0, 95]
    k_len = [100, 64, 128, 500, 0, 16, 1, 7, 32]
    H, H_kv = 4, 2
    seqs, q, k, v, cu_q, cu_k = qk_batch(q_len, k_len, H, H_kv, d, 800 + d)
    s = 1.0 / math.sqrt(d)
    o, lse = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), max(q_len), scale=s,
                              causal="compressed", return_lse=True, cu_seqlens_k=cu_k.to(DEV),
                              max_seqlen_k=max(k_len))
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    check_qk(seqs, o, lse, cu_q, s, "compressed", None)
    # sequence 0 (cf = 3): queries 0 and 1 see no key, query 2 sees key 0 alone
    assert bool((o[:2] == 0).all()) and bool(torch.isneginf(lse[:2]).all())
    assert torch.equal(o[2], seqs[0][2][0, :, 0].repeat_interleave(H // H_kv, 0))


def test_varlen_compressed_causal_with_key_split():
    """One long sequence: few workgroups, so its keys are split; cf = 4."""
    from exact_softmax_attention_bf16_amd import attention_varlen
    seqs, q, k, v, cu_q, cu_k = qk_batch([4096], [1024], 1, 1, 64, 900)
    o, lse = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), 4096,
                              causal="compressed", return_lse=True, cu_seqlens_k=cu_k.to(DEV),
                              max_seqlen_k=1024)
    torch.cuda.synchronize()
    check_qk(seqs, o.cpu(), lse.cpu(), cu_q, 0.125, "compressed", None)


def test_varlen_compressed_causal_equal_lengths_is_causal_bitwise():
    from exact_softmax_attention_bf16_amd import attention_varlen
    seqs, q, k, v, cu = varlen_batch([333, 128, 5], 2, 2, 64, 950)
    a = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), 333, causal=True)
    b = attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), 333, causal="compressed")
    assert torch.equal(a, b)


def test_varlen_compressed_causal_rejects_a_window():
    from exact_softmax_attention_bf16_amd import _lib, attention_varlen
    seqs, q, k, v, cu_q, cu_k = qk_batch([64], [16], 1, 1, 64, 960)
    with pytest.raises(_lib.AttnError) as err:
        attention_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), 64, causal="compressed",
                         window=(8, 0), cu_seqlens_k=cu_k.to(DEV), max_seqlen_k=16)
    assert err.value.status == _lib.ATTN_ERR_BAD_MASK
