#!/usr/bin/env python3
"""Benchmark of exact softmax attention on one MI355X.

One step = one attn_forward call over the whole workload, inputs already in
HBM: by default the full Wan2.2 VAE decode's mid-block attention, 31 frames x
one head, L = 3432 (44x78), d = 1024, scale 1/32, no mask (1.4956 TFLOP).

Prints one JSON line:  TFLOP/s (value), ms per call, % of the bf16 dense MFMA
peak, the dominant kernel's roofline figures (its FLOPs per launch over its
average HIP-event duration inside the timed region), the CPU float64 oracle's
rate on every head of the same workload, and the timed output's error against
that oracle.  Under "runs", the other five workloads (the tiny d = 256 head,
4 x 8 heads at d = 64 with and without the causal mask, 1 and 4 Wan frames),
each timed the same way (events on the kernels' stream around K calls, then
per-call events) and checked against the oracle, with the oracle's time.
Before each workload's W warm-up calls, 0.2 s of untimed calls (settle_s) let
the clocks leave their idle state.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-other-runs]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s & % bf16 MFMA peak (31 frames, L=3432, d=1024); ms/call"
# MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
# The pages' figure for the same 31-frame attention: ATen SDPA (xformers cutlass
# kernel) 8.5 ms on their sm_100a/sm_103a target = 1.4956e12 FLOP / 8.5 ms.
PAGES_ATEN_MS = 8.5

KERNEL_SOURCES = os.path.join(ROOT, "exact_softmax_attention_bf16_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(text: str) -> str:
    """Kernel source with comments and blank lines removed (a comment edit does
    not change the kernel the counters measured)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest() -> str:
    """Digest of the device sources (kernels and the headers they include); the
    host-side C ABI does not change what a kernel moves."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(KERNEL_SOURCES, "*"))):
        if p.endswith((".hip", ".h")):
            h.update(code_text(open(p).read()).encode())
    return h.hexdigest()


def kernel_flops(name: str, w) -> int:
    """Algorithmic FLOPs of one step spent in kernel `name` (2 per multiply-add)."""
    pairs = w.L * (w.L + 1) // 2 if w.causal else w.L * w.L
    per_contraction = 2 * w.B * w.H * pairs * w.d
    return {"online": 2 * per_contraction, "scores": per_contraction,
            "values": per_contraction}.get(name, 0)  # values_reduce: no MFMA work


def measured_traffic(kernel: str, workload: str, launches_per_step: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_digest():
        return None  # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def oracle_cores() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def oracle_check(w, q, k, v, out_gpu):
    """The oracle, as it stands, on every head of the workload: its wall time on
    the host cores, and the GPU output of the timed region against it."""
    import numpy as np
    import torch

    import oracle
    from synth.metrics import REL_RMS_BAND, within_bar
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    got = out_gpu.detach().to("cpu", torch.float64).numpy()
    qf, kf, vf = f64(q), f64(k), f64(v)
    t0 = time.perf_counter()
    ref = np.empty_like(got)
    for b in range(w.B):  # head by head, as the oracle runs on its own
        ref[b:b + 1] = oracle.attention(qf[b:b + 1], kf[b:b + 1], vf[b:b + 1], w.scale, w.causal)
    dt = time.perf_counter() - t0
    ok, a, r = within_bar(got, ref)
    return {"oracle_s": round(dt, 3), "oracle_cores": oracle_cores(), "max_abs": float(f"{a:.4g}"),
            "rel_rms": float(f"{r:.4g}"), "ok": bool(ok and r <= REL_RMS_BAND)}


def time_calls(call, stream, steps: int):
    """ms per call over `steps` back-to-back calls between two events on the
    stream the kernels run on, then the per-call median and minimum over as
    many more calls, each between its own pair of events."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    region = a.elapsed_time(b) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for x, y in ev:
        x.record(stream)
        call()
        y.record(stream)
    torch.cuda.synchronize()
    per = sorted(x.elapsed_time(y) for x, y in ev)
    med = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    return region, med, per[0]


def abi_call(w, qd, kd, vd, out):
    """A closure that calls attn_forward through the C ABI with its arguments
    marshalled once, on the current stream: the per-call host cost is then the
    library's own, not the Python binding's checks."""
    import ctypes

    import torch

    from exact_softmax_attention_bf16_amd._lib import AttnError, load
    f = load().attn_forward
    stream = ctypes.c_void_p(torch.cuda.current_stream(qd.device).cuda_stream)
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), w.B, w.H, w.L, w.d,
            ctypes.c_float(w.scale), int(w.causal), stream)

    def call():
        st = f(*args)
        if st != 0:
            raise AttnError(st)
    return call


SETTLE_S = 0.2  # untimed calls before the warm-up steps, so the clocks have left idle


def settle(call, seconds: float = SETTLE_S):
    """Untimed calls for `seconds` of wall time (synchronising every 10 calls, so
    the time is the GPU's, not the host's enqueue rate): the clocks ramp up from
    their idle state over a fraction of a second."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        call()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def other_run(name: str, steps: int, warmup: int, dev):
    """One of the other workloads: warm up, time (per-kernel timing off), then
    the per-kernel averages over as many more calls, and oracle parity."""
    import torch

    from exact_softmax_attention_bf16_amd import kernel_timing
    from synth import WORKLOADS, make_qkv
    w = WORKLOADS[name]
    q, k, v = make_qkv(w.B, w.H, w.L, w.d, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    call = abi_call(w, qd, kd, vd, out)
    settle(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    region, med, mn = time_calls(call, torch.cuda.current_stream(), steps)
    kt = {}
    with kernel_timing(kt):
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
    flops = w.flops()
    rec = {"B": w.B, "H": w.H, "L": w.L, "d": w.d, "causal": w.causal, "flop": flops,
           "steps": steps, "ms_per_call": round(region, 5),
           "ms_per_call_median": round(med, 5), "ms_per_call_min": round(mn, 5),
           "tflops": round(flops / (region * 1e-3) / 1e12, 3),
           "pct_bf16_mfma_peak": round(100.0 * flops / (region * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 3),
           "kernel_ms": {n: round(t / c, 5) for n, (t, c) in sorted(kt.items())}}
    rec.update(oracle_check(w, q, k, v, out))
    log(f"[bench] {name}: {rec}")
    return rec


def split_columns_probe(args) -> int:
    """The large-d alternative that splits the output columns across waves
    (include/attn_probe.h), timed next to attn_forward on the same workload with
    events on the same stream; its output is checked against the oracle on every
    head.  The probe's L2->CU stream: per workgroup (64 rows) and 32-key block,
    64 KB of K, 64 KB of V and 128 KB of Q."""
    import ctypes

    import torch

    from synth import WORKLOADS, make_qkv

    w = WORKLOADS[args.workload]
    if w.causal or w.d != 1024:
        log("[probe] the split-columns probe is written for d = 1024 without a mask")
        return 2
    path = os.path.join(ROOT, "exact_softmax_attention_bf16_amd", "libattn_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"probe library not built: {path}")
    probe = ctypes.CDLL(path).attn_probe_split_columns
    probe.restype = ctypes.c_int
    probe.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(w.B, w.H, w.L, w.d, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out_a, out_p = torch.empty_like(qd), torch.empty_like(qd)
    two_pass = abi_call(w, qd, kd, vd, out_a)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def split_cols():
        st = probe(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out_p.data_ptr(), w.B, w.H, w.L,
                   w.d, ctypes.c_float(w.scale), sp)
        if st != 0:
            raise RuntimeError(f"attn_probe_split_columns: status {st}")

    steps = max(args.steps // 5, 3)
    for _ in range(args.warmup):
        two_pass()
        split_cols()
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("two_pass", two_pass), ("split_columns", split_cols)):
        region, med, mn = time_calls(fn, stream, steps)
        res[name] = {"ms_per_call": round(region, 4), "ms_median": round(med, 4),
                     "tflops": round(w.flops() / (region * 1e-3) / 1e12, 1),
                     "pct_bf16_mfma_peak": round(100.0 * w.flops() / (region * 1e-3) / 1e12 /
                                                 PEAK_BF16_TFLOPS, 2)}
    wgs = w.B * w.H * ((w.L + 63) // 64)
    stream_bytes = wgs * ((w.L + 31) // 32) * (64 + 64 + 128) * 1024
    res["split_columns"]["l2_to_cu_gb_per_call"] = round(stream_bytes / 1e9, 2)
    res["split_columns"]["l2_to_cu_tb_per_s"] = round(
        stream_bytes / (res["split_columns"]["ms_per_call"] * 1e-3) / 1e12, 2)
    res["split_columns"]["vs_oracle"] = oracle_check(w, q, k, v, out_p)
    rec = {"probe": "split_columns", "workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d,
           "steps": steps, **res}
    print(json.dumps(rec), flush=True)
    return 0


def design_probe(args) -> int:
    """The large-d alternative that materialises S, timed stage by stage.

    S = Q K^T (bf16 out of hipBLASLt, half the bytes of the fp32 S the pages
    write, so a lower bound), P = softmax(S) over keys (torch, fp32 inside,
    bf16 out), O = P V.  The scale is folded into Q beforehand (exact for a
    power of two).  Each stage is timed with events over the same calls."""
    import torch

    from exact_softmax_attention_bf16_amd import attention
    from synth import WORKLOADS, make_qkv

    w = WORKLOADS[args.workload]
    if w.causal or w.d <= 128:
        log("[probe] the probe covers the unmasked large-d workloads")
        return 2
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(w.B, w.H, w.L, w.d, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    n = w.B * w.H
    qs = (qd.float() * w.scale).to(torch.bfloat16).reshape(n, w.L, w.d)
    kt = kd.reshape(n, w.L, w.d).transpose(1, 2).contiguous()  # bmm's right operand, contiguous
    vv = vd.reshape(n, w.L, w.d)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    stages = {"s_gemm": 0.0, "softmax": 0.0, "pv_gemm": 0.0}
    steps = max(args.steps // 5, 3)
    for it in range(args.warmup + steps):
        ev[0].record()
        S = torch.bmm(qs, kt)
        ev[1].record()
        P = torch.softmax(S, dim=-1)
        ev[2].record()
        O = torch.bmm(P, vv)
        ev[3].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            for i, name in enumerate(stages):
                stages[name] += ev[i].elapsed_time(ev[i + 1]) / steps
        del S, P, O
    for _ in range(args.warmup):
        attention(qd, kd, vd, scale=w.scale, causal=False, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        attention(qd, kd, vd, scale=w.scale, causal=False, out=out)
    torch.cuda.synchronize()
    ours = (time.perf_counter() - t0) * 1e3 / steps
    s_bytes = n * w.L * w.L * 2  # one bf16 S (or P) tensor
    line = {"probe": "materialised_S", "workload": w.name,
            "s_gemm_ms": round(stages["s_gemm"], 4), "softmax_ms": round(stages["softmax"], 4),
            "pv_gemm_ms": round(stages["pv_gemm"], 4),
            "total_ms": round(sum(stages.values()), 4),
            "softmax_pass_bytes": 2 * s_bytes,
            "softmax_pass_GBps": round(2 * s_bytes / (stages["softmax"] * 1e-3) / 1e9, 1),
            "hbm_peak_GBps": 8000,
            "attn_forward_ms": round(ours, 4)}
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan_31frame")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (its timing and the parity of the timed output)")
    ap.add_argument("--no-other-runs", action="store_true",
                    help="time only --workload, not the other five runs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 256 MiB device-to-device three times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    ap.add_argument("--split-columns-probe", action="store_true",
                    help="time the one-kernel large-d alternative that splits the output columns "
                         "across waves (libattn_probe.so) next to attn_forward, check it against "
                         "the oracle, and print one JSON line")
    ap.add_argument("--design-probe", action="store_true",
                    help="time the materialised-S alternative for large d from library pieces "
                         "(hipBLASLt bmm for Q K^T and P V, torch softmax between them) next to "
                         "attn_forward on the same workload, and print one JSON line")
    args = ap.parse_args()

    if args.design_probe:
        return design_probe(args)
    if args.split_columns_probe:
        return split_columns_probe(args)

    if args.copy_probe:
        import torch
        n = 256 << 20
        src = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda:0").normal_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 3 copies of {n} bytes")
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the heads are independent: several GPUs would each take whole heads). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from exact_softmax_attention_bf16_amd import kernel_timing
    from synth import WORKLOADS, make_qkv

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} L={w.L} d={w.d} scale={w.scale} causal={w.causal}")
    q, k, v = make_qkv(w.B, w.H, w.L, w.d, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(qd)
    call = abi_call(w, qd, kd, vd, out)

    settle(call)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    log(f"[bench] settle {SETTLE_S} s and warmup {args.warmup} done")

    kt = {}
    with kernel_timing(kt):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/call, {tflops:.1f} TFLOP/s")
    for name, (tot, cnt) in sorted(kt.items()):
        log(f"[bench]   kernel {name}: {tot / cnt:.4f} ms avg over {cnt} launches")

    # Per-call spread, after the timed region: K more calls, each between two
    # events on the stream the kernels run on.
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) for a, b in ev)
    med = per_call[len(per_call) // 2] if len(per_call) % 2 else \
        0.5 * (per_call[len(per_call) // 2 - 1] + per_call[len(per_call) // 2])
    log(f"[bench] per call over {len(per_call)} more calls: median {med:.4f} ms, "
        f"min {per_call[0]:.4f} ms")

    # Roofline of the dominant kernel.
    dom = max((n for n in kt if kernel_flops(n, w) > 0), key=lambda n: kt[n][0])
    tot, cnt = kt[dom]
    launches_per_step = cnt / args.steps
    flop_per_launch = kernel_flops(dom, w) / launches_per_step
    achieved = flop_per_launch / (tot / cnt * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, w.name, launches_per_step),
                "flop_per_launch": flop_per_launch,
                "avg_launch_ms": round(tot / cnt, 5)}

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        log("[bench] oracle on every head of the timed output")
        chk = oracle_check(w, q, k, v, out)
        parity = {key: chk[key] for key in ("max_abs", "rel_rms", "ok")}
        pairs = w.L * (w.L + 1) // 2 if w.causal else w.L * w.L
        cpu = {"value": round(4 * w.B * w.H * pairs * w.d / chk["oracle_s"] / 1e12, 6),
               "unit": "TFLOP/s", "cores": chk["oracle_cores"], "kind": "oracle",
               "sample": (f"all {w.B * w.H} heads (L={w.L}, d={w.d}, every row), "
                          f"{chk['oracle_s']:.1f} s, float64 NumPy")}
        log(f"[bench] cpu baseline: {cpu}; parity {parity}")

    runs = None
    if not args.no_other_runs:
        runs = {}
        for name in ("tiny_d256", "mha_d64", "mha_d64_causal", "wan_1frame", "wan_4frame",
                     "wan_31frame"):
            if name == w.name:
                continue
            small = WORKLOADS[name].flops() < 1e11
            runs[name] = other_run(name, 200 if small else args.steps, max(args.warmup, 10), dev)

    vs = None
    if w.name == "wan_31frame":
        vs = round(PAGES_ATEN_MS / ms, 4)

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms, 5),
        "ms_per_call_median": round(med, 5),
        "ms_per_call_min": round(per_call[0], 5),
        "pct_bf16_mfma_peak_at_min": round(100.0 * flops / (per_call[0] * 1e-3) / 1e12
                                           / PEAK_BF16_TFLOPS, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs,
        "vs_baseline_note": ("pages' ATen SDPA time for this workload, 8.5 ms on their "
                             "sm_100a/sm_103a target (other hardware; context only)"),
        "pct_bf16_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 3),
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) rounded to bf16",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d,
                   "scale": w.scale, "causal": w.causal, "flop_per_step": flops,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "runs": runs,
    }
    print(json.dumps(line), flush=True)
    checks = ([parity] if parity else []) + list((runs or {}).values())
    if not all(c["ok"] for c in checks):
        log("[bench] a timed output is outside the parity bar or the expected error band")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
