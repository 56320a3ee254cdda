"""GPU parity: the HIP path against the CPU float64 oracle on the same seeded inputs.

Bar (element by element): max |o - ref| <= 2e-2 and ||o - ref||_2 / ||ref||_2 <= 5e-3,
with o the kernel's bf16 output converted exactly to float64.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_qkv
from synth.metrics import MAX_ABS_TOL, REL_RMS_BAND, REL_RMS_TOL, within_bar

from gpu_util import check_full, run_gpu, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def _report(name, a, r):
    print(f"[parity] {name}: max_abs={a:.3e} rel_rms={r:.3e}", flush=True)


# ---- the workloads at full size --------------------------------------------

@pytest.mark.parametrize("name", ["tiny_d256", "mha_d64", "mha_d64_causal", "wan_1frame",
                                  "wan_4frame", "wan_31frame"])
def test_workload_full(name):
    """Every output element of every workload at full size (the launch the
    benchmark times) against the oracle, frame by frame; also inside the
    expected error band, so that a precision regression fails even below the bar."""
    w = WORKLOADS[name]
    ok, a, r, *_ = check_full(w.B, w.H, w.L, w.d, w.scale, w.causal, w.seed)
    _report(name, a, r)
    assert ok, (a, r)
    assert r <= REL_RMS_BAND, (r, REL_RMS_BAND)


# ---- ragged tails, head dims, masks ----------------------------------------

SWEEP_L = [1, 2, 15, 17, 63, 64, 65, 127, 129, 255, 257, 286, 513]
SWEEP_D = [32, 64, 128, 192, 256, 512, 1024]


@pytest.mark.parametrize("d", SWEEP_D)
@pytest.mark.parametrize("L", SWEEP_L)
@pytest.mark.parametrize("causal", [False, True])
def test_tail_sweep(L, d, causal):
    ok, a, r, *_ = check_full(2, 2, L, d, 1.0 / math.sqrt(d), causal, seed=1000 + L * 7 + d)
    _report(f"L={L} d={d} causal={causal}", a, r)
    assert ok, (a, r)


@pytest.mark.parametrize("d,L", [(64, 1100), (128, 777), (1024, 700), (256, 1500)])
def test_long_rows_several_tiles(d, L):
    for causal in (False, True):
        ok, a, r, *_ = check_full(1, 3, L, d, 1.0 / math.sqrt(d), causal, seed=77 + L)
        _report(f"L={L} d={d} causal={causal}", a, r)
        assert ok, (a, r)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0])
def test_unusual_scales(d, scale):
    for causal in (False, True):
        ok, a, r, *_ = check_full(1, 2, 300, d, scale, causal, seed=5)
        _report(f"d={d} scale={scale} causal={causal}", a, r)
        assert ok, (a, r)


# ---- invariants on the GPU -------------------------------------------------

@pytest.mark.parametrize("d", [64, 1024])
def test_causal_row0_is_v0_exactly(d):
    q, k, v = make_qkv(2, 2, 200, d, 9)
    o = run_gpu(q, k, v, 1.0 / math.sqrt(d), True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(d, causal):
    q, k, v = make_qkv(1, 2, 333, d, 10)
    v = v[:, :, :1].expand_as(v).contiguous()
    o = run_gpu(q, k, v, 1.0 / math.sqrt(d), causal).cpu().double()
    err = (o - v.double()).abs().max().item()
    assert err <= 2.0 ** -7 * v.double().abs().max().item()


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_mean(d, causal):
    q, k, v = make_qkv(1, 2, 300, d, 11)
    k = k[:, :, :1].expand_as(k).contiguous()
    o = to_f64(run_gpu(q, k, v, 1.0 / math.sqrt(d), causal))
    vf = to_f64(v)
    if causal:
        want = np.cumsum(vf, axis=2) / np.arange(1, 301)[None, None, :, None]
    else:
        want = np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
    ok, a, r = within_bar(o, want)
    assert ok, (a, r)


@pytest.mark.parametrize("d", [64, 1024])
def test_deterministic(d):
    q, k, v = make_qkv(2, 1, 900, d, 12)
    o1 = run_gpu(q, k, v, 1.0 / math.sqrt(d), False)
    o2 = run_gpu(q, k, v, 1.0 / math.sqrt(d), False)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("d", [64, 1024])
def test_canary_and_inputs_untouched(d):
    """Writes stay inside `out`; q, k, v are not modified."""
    B, H, L = 1, 2, 301
    q, k, v = make_qkv(B, H, L, d, 13)
    dev = torch.device("cuda:0")
    n = B * H * L * d
    pad = 4096
    big = torch.full((n + 2 * pad,), 12345.0, dtype=torch.bfloat16, device=dev)
    out = big[pad : pad + n].view(B, H, L, d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    run_gpu(qd, kd, vd, 1.0 / math.sqrt(d), False, out=out)
    assert bool((big[:pad] == 12345.0).all()) and bool((big[pad + n :] == 12345.0).all())
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k) and torch.equal(vd.cpu(), v)
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(d), False)
    assert within_bar(to_f64(out), ref)[0]


def test_empty_problem():
    from exact_softmax_attention_bf16_amd import attention
    x = torch.zeros(2, 3, 0, 64, dtype=torch.bfloat16, device="cuda:0")
    assert attention(x, x, x).shape == x.shape


def test_kernel_timing_records_each_kernel():
    from exact_softmax_attention_bf16_amd import attention, kernel_timing
    q, k, v = (t.cuda() for t in make_qkv(12, 1, 2048, 256, 14))
    res = {}
    with kernel_timing(res):
        attention(q, k, v)
        attention(q, k, v)
    # 12 heads of L=2048, d=256: 96 wide tiles, 384 narrow ones; the values pass splits its keys
    assert set(res) == {"scores", "values", "values_reduce"}
    assert all(c == 2 and ms > 0 for ms, c in res.values())


def test_kernel_timing_without_split():
    from exact_softmax_attention_bf16_amd import attention, kernel_timing
    q, k, v = (t.cuda() for t in make_qkv(16, 1, 1024, 1024, 15))  # 256 workgroups: no split
    res = {}
    with kernel_timing(res):
        attention(q, k, v)
    assert set(res) == {"scores", "values"}


@pytest.mark.parametrize("B,L,d,splits", [(12, 2048, 256, 2), (10, 1600, 256, 3),
                                           (32, 2100, 512, 1)])
def test_values_key_split(B, L, d, splits):
    """Heads too few for the 256 x 256 grid and too many for one round of
    128 x 128 tiles: the values pass divides the keys among 2-3 workgroups and
    sums their fp32 shares (splits == 1: enough heads not to)."""
    from exact_softmax_attention_bf16_amd import attention, kernel_timing
    q, k, v = make_qkv(B, 1, L, d, 30 + splits)
    s = 1.0 / math.sqrt(d)
    res = {}
    with kernel_timing(res):
        o = attention(q.cuda(), k.cuda(), v.cuda(), scale=s)
    torch.cuda.synchronize()
    assert ("values_reduce" in res) == (splits > 1)
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, False)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"key split x{splits} B={B} L={L} d={d}", a, r)
    assert ok and r <= REL_RMS_BAND, (a, r)


@pytest.mark.parametrize("H,L,d,causal", [(1, 1100, 256, False), (1, 1000, 320, False),
                                           (1, 2100, 512, False), (2, 700, 192, False),
                                           (1, 1300, 448, True), (1, 129, 192, False),
                                           (1, 64, 1024, False), (1, 4096, 1024, False),
                                           (3, 600, 1024, True)])
def test_values_narrow_tiles(H, L, d, causal):
    """Few heads: the values pass runs on 128 x 128 tiles, one round, no key
    split (ragged query tiles whose far half is idle, channel tiles half past d,
    one partial tile, exactly 256 tiles), with the LSE."""
    from exact_softmax_attention_bf16_amd import attention, kernel_timing
    q, k, v = make_qkv(1, H, L, d, 40 + L + d)
    s = 1.0 / math.sqrt(d)
    res = {}
    with kernel_timing(res):
        o, lse = attention(q.cuda(), k.cuda(), v.cuda(), scale=s, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert set(res) == {"scores", "values"}
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, causal)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"narrow tiles H={H} L={L} d={d} causal={causal}", a, r)
    assert ok and r <= REL_RMS_BAND, (a, r)
    lref = oracle.log_sum_exp(to_f64(q), to_f64(k), s, causal)
    err = np.abs(to_f64(lse) - lref)
    assert bool((err <= 4e-3 + 1e-5 * np.abs(lref)).all()), float(err.max())


def test_workspace_grows_and_is_reused_on_one_stream():
    """The two-pass workspace of a stream: small call, larger call (the buffer
    grows), small call again, all queued back to back before one sync."""
    from exact_softmax_attention_bf16_amd import attention
    dev = torch.device("cuda:0")
    cases = [(1, 1, 300, 256, 21), (2, 1, 1300, 256, 22), (1, 2, 257, 512, 23)]
    ins = [tuple(t.to(dev) for t in make_qkv(B, H, L, d, s)) for B, H, L, d, s in cases]
    outs = [attention(q, k, v) for q, k, v in ins]
    torch.cuda.synchronize()
    for (B, H, L, d, s), (q, k, v), o in zip(cases, ins, outs):
        ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(d), False)
        ok, a, r = within_bar(to_f64(o), ref)
        _report(f"workspace reuse L={L} d={d}", a, r)
        assert ok


def test_two_streams_do_not_share_workspace():
    """Calls queued on two streams at once (each with its own inputs) both match."""
    from exact_softmax_attention_bf16_amd import attention
    dev = torch.device("cuda:0")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    a = tuple(t.to(dev) for t in make_qkv(1, 1, 1000, 512, 24))
    b = tuple(t.to(dev) for t in make_qkv(1, 1, 1000, 512, 25))
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = attention(*a)
        with torch.cuda.stream(s2):
            ob = attention(*b)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for x, o in ((a, outs[-1][0]), (b, outs[-1][1])):
        ref = oracle.attention(*(to_f64(t) for t in x), 1.0 / math.sqrt(512), False)
        ok, am, r = within_bar(to_f64(o), ref)
        _report("two streams", am, r)
        assert ok
    assert all(torch.equal(p[0], outs[-1][0]) and torch.equal(p[1], outs[-1][1]) for p in outs)


def test_concurrent_host_threads_each_on_its_own_stream():
    """Four host threads call at once, each on a stream of its own, mixing the
    two-pass path and the online path with and without a key split; every call
    equals the same call made alone (the library's workspace map and pools are
    shared between the threads)."""
    import threading

    from exact_softmax_attention_bf16_amd import attention
    dev = torch.device("cuda:0")
    cases = [(1, 1, 700, 64, True), (2, 1, 600, 1024, False), (1, 2, 900, 128, False),
             (1, 1, 1300, 256, True)]
    ins = [tuple(t.to(dev) for t in make_qkv(B, H, L, d, 40 + i))
           for i, (B, H, L, d, _) in enumerate(cases)]
    refs = [attention(q, k, v, causal=c) for (q, k, v), (*_, c) in zip(ins, cases)]
    torch.cuda.synchronize()
    results, errors = {}, []

    def work(i):
        try:
            stream = torch.cuda.Stream()
            q, k, v = ins[i]
            with torch.cuda.stream(stream):
                outs = [attention(q, k, v, causal=cases[i][4]) for _ in range(6)]
            stream.synchronize()
            results[i] = outs
        except Exception as e:  # re-raised below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    if errors:
        raise errors[0]
    for i, ref in enumerate(refs):
        assert all(torch.equal(o, ref) for o in results[i]), cases[i]


def test_concurrent_host_threads_on_one_stream_growing_sizes():
    """Two host threads call at once on the SAME stream, each with sizes that
    grow from call to call (so the stream's workspace buffer is replaced while
    the other thread holds it): every call equals the same call made alone.
    The library leases the stream's buffer for the whole of a call, so the two
    threads' kernels are queued one call after the other, never interleaved."""
    import threading

    from exact_softmax_attention_bf16_amd import attention
    dev = torch.device("cuda:0")
    per_thread = [[(1, 1, 300, 1024), (1, 1, 900, 512), (2, 1, 1400, 256), (1, 1, 2100, 1024)],
                  [(1, 1, 400, 256), (1, 1, 1000, 1024), (1, 1, 1800, 512), (3, 1, 1200, 1024)]]
    ins = [[tuple(t.to(dev) for t in make_qkv(B, H, L, d, 60 + 10 * j + i))
            for i, (B, H, L, d) in enumerate(cs)] for j, cs in enumerate(per_thread)]
    refs = [[attention(*x) for x in row] for row in ins]  # each call alone
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    results, errors = {}, []

    def work(j):
        try:
            with torch.cuda.stream(stream):
                results[j] = [attention(*x) for _ in range(3) for x in ins[j]]
        except Exception as e:  # re-raised below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(j,)) for j in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    stream.synchronize()
    torch.cuda.synchronize()
    if errors:
        raise errors[0]
    for j in range(2):
        n = len(ins[j])
        for r, o in enumerate(results[j]):
            assert torch.equal(o, refs[j][r % n]), (j, per_thread[j][r % n])


# ---- online path with few heads: keys split among workgroups, then combined ----

@pytest.mark.parametrize("B,H,L,d", [(1, 1, 4096, 64), (1, 2, 1000, 128), (2, 4, 1024, 64),
                                     (1, 1, 777, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_online_key_split(B, H, L, d, causal):
    """Shares 8, 4, 4 and 3: each writes fp32 O and (m, l); the combine kernel
    merges them (and writes the LSE)."""
    from exact_softmax_attention_bf16_amd import attention, kernel_timing
    q, k, v = make_qkv(B, H, L, d, 300 + L + d)
    s = 1.0 / math.sqrt(d)
    res = {}
    with kernel_timing(res):
        o, lse = attention(q.cuda(), k.cuda(), v.cuda(), scale=s, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert set(res) == {"online", "online_combine"}
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), s, causal)
    ok, a, r = within_bar(to_f64(o), ref)
    _report(f"online split B={B} H={H} L={L} d={d} causal={causal}", a, r)
    assert ok, (a, r)
    err = np.abs(to_f64(lse) - oracle.log_sum_exp(to_f64(q), to_f64(k), s, causal))
    assert float(err.max()) <= 4e-3 + 1e-5 * float(np.abs(to_f64(lse)).max())


def test_online_key_split_window_strided_out_deterministic():
    from exact_softmax_attention_bf16_amd import attention
    L, d = 3000, 64
    q, k, v = make_qkv(1, 1, L, d, 310)
    big = torch.full((1, 1, L, 2 * d), 5.0, dtype=torch.bfloat16, device="cuda")
    out = big[..., d:]
    o1 = attention(q.cuda(), k.cuda(), v.cuda(), window=(700, 90), out=out).clone()
    o2 = attention(q.cuda(), k.cuda(), v.cuda(), window=(700, 90))
    torch.cuda.synchronize()
    assert bool((big[..., :d] == 5.0).all())
    assert torch.equal(o1, o2)
    ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), 1.0 / math.sqrt(d), False, (700, 90))
    ok, a, r = within_bar(to_f64(o1), ref)
    assert ok, (a, r)


@pytest.mark.parametrize("d", list(range(192, 1025, 64)))
@pytest.mark.parametrize("causal", [False, True])
def test_every_two_pass_head_dim(d, causal):
    """Every multiple of 64 in (128, 1024]: the last 256-channel tile of the
    values pass is partly past d for most of them."""
    ok, a, r, *_ = check_full(1, 2, 300, d, 1.0 / math.sqrt(d), causal, seed=400 + d)
    _report(f"d={d} causal={causal}", a, r)
    assert ok, (a, r)
