#!/usr/bin/env python3
"""Forward + backward causal GQA attention throughput on one MI355X.

One step = attn_fwd then attn_bwd over one batch of synthetic input already resident in HBM; the
backward gets a workspace sized by attn_bwd_qk_workspace_bytes_for, so at the default workload it
runs the delta rows, the dK/dV kernel (which also stores dS) and the dQ kernel that reads the stored
dS (its trailing workgroups add the dK/dV head-split partials). Default workload: B=1, Hq=64, Hkv=8, S=4096, D=128,
bf16, causal. Prints one JSON line.

FLOPs are counted as 4*B*Hq*N*D for the forward, with N = S^2/2 attended pairs under the causal
mask (the exact pair count with a window, S^2 without a mask), and 2.5x that for the backward.
With fewer queries than keys (--workload naming a prefill-chunk or decode shape: Sq queries at
the last Sq of S positions) N = (S^2 - (S-Sq)^2)/2 causal, the exact count with a window, Sq*S
without a mask; sink keys add the exact count of sink keys outside each row's window.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CPU_SAMPLE_PAIRS = 6e8     # attended (query, key) pairs in the CPU oracle sample (the headline: 5.4e8)
METRIC = "fwd+bwd causal attn TFLOP/s & % bf16 MFMA peak (GQA 64/8, d128, S=4096)"
DEFAULT_WORKLOAD = "gqa64x8-s4096-d128"  # the workload METRIC is quoted on
KERNEL_SOURCES = {  # the files a kernel's code and launch configuration come from
    "attn_fwd": ["attn_fwd.hip", "device.h", "tiles.h", "launch.h"],
    "attn_bwd_dkdv": ["attn_dkdv.hip", "device.h", "tiles.h", "launch.h"],
    "attn_bwd_dq": ["attn_bwd.hip", "device.h", "tiles.h", "launch.h"],
    "attn_bwd_prep": ["attn_bwd.hip", "device.h", "launch.h"],
    "attn_bwd_dkdv_reduce": ["attn_dkdv.hip", "device.h", "launch.h"],
    "attn_bwd_dkdv_chunks": ["attn_dkdv.hip", "device.h", "launch.h"],
}


def attended_pairs(S: int, causal: bool, window: int, Sq: int | None = None, sink: int = 0) -> float:
    """Attended (query, key) pairs for Sq queries at the last Sq of S key positions, with `sink`
    leading keys kept visible beside the window."""
    Sq = S if Sq is None else Sq
    off = S - Sq
    if not causal:
        return float(Sq) * S
    if window == 0:
        return (float(S) * S - float(off) * off) / 2.0

    def upto(n):  # sum over positions p < n of min(p + 1, W)
        W = min(window, n)
        return W * (W + 1) / 2.0 + (n - W) * window

    def sinks_upto(n):  # sum over positions p < n of the sink keys before the window: min(n_sink, p-W+1)+
        total = 0.0
        for p in range(window, n):  # only positions whose window starts after key 0
            total += min(sink, p - window + 1)
        return total
    extra = sinks_upto(S) - sinks_upto(off) if sink else 0.0
    return upto(S) - upto(off) + extra


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "causal_attention_fa2_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_profile(kernel: str, workload: str):
    """The committed rocprofv3 counter summary of one kernel on one workload (HBM bytes per launch
    from FETCH_SIZE / WRITE_SIZE, MFMA busy fraction and executed MFMA instructions from the SQ
    counters), if it was taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(f"{kernel}@{workload}")
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the profile summary (None if absent or stale)."""
    rec = load_profile(kernel, workload)
    return None if rec is None else rec.get("bytes_per_launch")


def device_peak_bf16(torch):
    """CUs x 4096 bf16 FLOP/clk/CU x the clock the HIP runtime reports, in TFLOP/s (or None)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded (same soname)
        val = ctypes.c_int(0)
        dev = torch.cuda.current_device()
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, dev) != 0:  # hipDeviceAttributeClockRate
            return None
        clock_khz = val.value
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 63, dev) != 0:  # ...MultiprocessorCount
            return None
        return {"cus": val.value, "clock_mhz": clock_khz / 1e3,
                "tflops": round(val.value * 4096 * clock_khz * 1e3 / 1e12, 1)}
    except OSError:
        return None


def host_info():
    """CPU model and the BLAS numpy uses, for the oracle timing."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                if p.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:
        pass
    return model, blas


def cpu_sample(w, heads: int, cu=None):
    """(query heads, KV groups, query rows, attended pairs per head) of the CPU-oracle sample: the
    first `heads` query heads as whole KV groups; without documents it is then kept to about
    CPU_SAMPLE_PAIRS attended pairs (10-30 s of oracle work) by taking one KV group, then one query
    head, then the last query rows (the oracle takes S_q <= S_k)."""
    G = w.Hq // w.Hkv
    heads = max(G, min(w.Hq, heads // G * G))
    groups = heads // G
    rows = w.n_q
    if cu is not None:
        pairs = sum(attended_pairs(int(b - a), True, w.window) for row in cu
                    for a, b in zip(row[:-1], row[1:]) if b > a) / w.B
        return heads, groups, rows, pairs
    pairs = attended_pairs(w.S, w.causal, w.window, rows, w.sink)
    if w.B * heads * pairs > CPU_SAMPLE_PAIRS:
        heads, groups = G, 1
    if w.B * heads * pairs > CPU_SAMPLE_PAIRS:
        heads = 1
    while rows > 64 and w.B * heads * pairs > CPU_SAMPLE_PAIRS:
        rows //= 2
        pairs = attended_pairs(w.S, w.causal, w.window, rows, w.sink)
    return heads, groups, rows, pairs


def cpu_baseline(w, q, k, v, do, heads: int):
    """The fp64 oracle, timed on this host's cores, on the first `heads` query heads (whole KV
    groups) of the same inputs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the affinity mask instead
        threads = len(os.sched_getaffinity(0))
    cu = None
    if w.docs:
        from causal_attention_fa2_amd.workloads import document_boundaries
        cu = document_boundaries(w)
    heads, groups, rows, pairs = cpu_sample(w, heads, cu)
    r0 = w.n_q - rows
    t0 = time.perf_counter()
    oracle.forward_backward(q[:, :heads, r0:], k[:, :groups], v[:, :groups], do[:, :heads, r0:],
                            w.causal, w.window, w.scale, sink=w.sink, cu_seqlens=cu)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.B * heads * pairs * w.D * 3.5
    model, blas = host_info()
    part = f"the last {rows} of {w.n_q} query rows, " if rows < w.n_q else ""
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on {heads} of {w.Hq} query heads ({groups} KV groups), "
                      f"{part}B={w.B}, Sq={w.n_q}, S={w.S}, D={w.D}: {dt:.2f} s wall",
            "cpu_model": model, "blas": blas}


def bench_paged(w, args, torch, fa) -> int:
    """Forward only: against a paged cache (attn_fwd_paged, or attn_decode_fwd for decode
    workloads) or, for dense decode workloads, attn_decode_fwd. A step is one forward over the
    batch."""
    import numpy as np
    from causal_attention_fa2_amd.workloads import make_inputs, paged_layout
    q, k, v, _ = make_inputs(w)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Sq = w.n_q
    if w.paged:
        kp, vp, table, lens = paged_layout(w, k, v)
        tt, tl = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
        max_keys = table.shape[1] * w.paged
    else:
        kp, vp, lens = k, v, np.full(w.B, w.S, dtype=np.int32)
        max_keys = w.S
    tq, tkp, tvp = (torch.from_numpy(x).to(td).cuda() for x in (q, kp, vp))
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.Hq, Sq), dtype=torch.float32, device="cuda")
    if w.decode:
        ws = torch.empty(fa.attn_decode_workspace_bytes(w.B, w.Hq, w.Hkv, Sq, max_keys, w.D),
                         dtype=torch.uint8, device="cuda")
        extra = dict(block_table=tt, seqlen_k=tl) if w.paged else {}

    def step():
        if w.decode:
            fa.attn_decode_fwd(tq, tkp, tvp, o, lse, ws, w.causal, w.window, w.scale, None, w.sink,
                               **extra)
        else:
            fa.attn_fwd_paged(tq, tkp, tvp, tt, tl, o, lse, w.causal, w.window, w.scale, None, w.sink)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stream = torch.cuda.current_stream()
    evs = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    kms = sorted(a.elapsed_time(b) for a, b in evs)
    kmed = kms[len(kms) // 2]
    eb = 2 if w.dtype == "bf16" else 4
    pairs = sum(attended_pairs(int(n), w.causal, w.window, Sq, w.sink) for n in lens)
    flops = 4.0 * w.Hq * pairs * w.D
    kv_bytes = float(sum(2 * w.Hkv * int(n) * w.D * eb for n in lens))
    qo_bytes = 2.0 * w.B * w.Hq * Sq * w.D * eb + 4.0 * w.B * w.Hq * Sq
    value = flops / (ms * 1e-3) / 1e12
    gbs = (kv_bytes + qo_bytes) / (kmed * 1e-3) / 1e9
    out = {
        "metric": f"attention forward TFLOP/s ({w.name})", "value": round(value, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": Sq, "S_max": w.S,
                   "D": w.D, "block": w.paged, "keys_total": int(lens.sum()), "causal": w.causal,
                   "path": "attn_decode_fwd" if w.decode else "attn_fwd_paged",
                   "window": w.window, "parallelism": "none (1 GPU)"},
        "kernel_ms_median": round(kmed, 4),
        "roofline": {"kernel": "attn_decode + attn_decode_combine" if w.decode else "attn_fwd",
                     "bound": "hbm" if Sq * (w.Hq // w.Hkv) <= 64 else "mfma",
                     "achieved": round(gbs, 1) if Sq * (w.Hq // w.Hkv) <= 64 else
                     round(flops / (kmed * 1e-3) / 1e12, 1),
                     "peak": PEAK_HBM_GBS if Sq * (w.Hq // w.Hkv) <= 64 else PEAK_BF16_TFLOPS,
                     "unit": "GB/s" if Sq * (w.Hq // w.Hkv) <= 64 else "TFLOP/s", "traffic": None},
    }
    r = out["roofline"]
    r["frac"] = round(r["achieved"] / r["peak"], 4)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the shader clock takes about 20 steps of this load to settle: warm-up covers it by default
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-heads", type=int, default=64,
                    help="query heads in the CPU oracle sample (rounded to whole KV groups)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 elementwise copies of MIB MiB (reads MIB, writes MIB): the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention library runs on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import causal_attention_fa2_amd as fa
    from causal_attention_fa2_amd.workloads import WORKLOADS, make_inputs

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 5}), flush=True)
        return 0

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if w.paged or w.decode:
        return bench_paged(w, args, torch, fa)
    q, k, v, do = make_inputs(w)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    tq, tk, tv, tdo = (torch.from_numpy(x).to(td).cuda() for x in (q, k, v, do))
    Sq = w.n_q
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.Hq, Sq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    ws_bytes = fa.attn_bwd_qk_workspace_bytes(w.B, w.Hq, w.Hkv, Sq, w.S, w.D)  # without the sink split
    ws = torch.empty(fa.attn_bwd_qk_workspace_bytes_for(w.B, w.Hq, w.Hkv, Sq, w.S, w.D, w.causal, w.window,
                                                        w.sink), dtype=torch.uint8, device="cuda")
    # the square workloads go through attn_fwd / attn_bwd, packed documents through the _varlen
    # entry points, the others through the _qk entry points
    square = Sq == w.S and not w.sink
    cu = None
    if w.docs:
        from causal_attention_fa2_amd.workloads import document_boundaries
        cu = document_boundaries(w)
        tcu = torch.from_numpy(cu).cuda()

    def fwd():
        if cu is not None:
            fa.attn_fwd_varlen(tq, tk, tv, o, lse, tcu, w.window, w.scale)
        elif square:
            fa.attn_fwd(tq, tk, tv, o, lse, w.causal, w.window, w.scale)
        else:
            fa.attn_fwd_qk(tq, tk, tv, o, lse, w.causal, w.window, w.scale, None, w.sink)

    def bwd():
        if cu is not None:
            fa.attn_bwd_varlen(tq, tk, tv, o, lse, tdo, dq, dk, dv, ws, tcu, w.window, w.scale)
        elif square:
            fa.attn_bwd(tq, tk, tv, o, lse, tdo, dq, dk, dv, ws, w.causal, w.window, w.scale)
        else:
            fa.attn_bwd_qk(tq, tk, tv, o, lse, tdo, dq, dk, dv, ws, w.causal, w.window, w.scale, None,
                           w.sink)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps between two synchronisations
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # fwd, bwd and fwd+bwd separately: HIP events on the launch stream around each repetition
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            out.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in out)
        return {"median": round(ms[len(ms) // 2], 4), "min": round(ms[0], 4)}

    phases = {"fwd": timed(fwd, args.steps), "bwd": timed(bwd, args.steps),
              "fwd+bwd": timed(step, args.steps)}

    # per-kernel durations: HIP events recorded on the launch stream around each kernel
    events = {}

    def hook(kernel, after, hip_stream):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)  # the library launches on torch's current stream (passed as hip_stream)
        events.setdefault(kernel, []).append(ev)

    fa.attn_set_launch_hook(hook)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_hooked = (time.perf_counter() - t1) * 1e3 / args.steps
    fa.attn_set_launch_hook(None)
    kern_ms = {}
    for name, evs in events.items():
        d = [evs[i].elapsed_time(evs[i + 1]) for i in range(0, len(evs), 2)]
        kern_ms[name] = sum(d) / len(d)

    if cu is not None:  # per batch row and document, the same convention per document
        N = sum(attended_pairs(int(b - a), True, w.window) for row in cu for a, b in zip(row[:-1], row[1:])
                if b > a) / w.B
    else:
        N = attended_pairs(w.S, w.causal, w.window, Sq, w.sink)
    unit = 2.0 * w.B * w.Hq * N * w.D  # one GEMM-sized pass over the attended pairs
    fl = {"attn_fwd": 2 * unit, "attn_bwd_dkdv": 4 * unit, "attn_bwd_dq": 1 * unit}
    total_flops = 7 * unit  # forward (2) + backward counted as 2.5x forward (5)
    fl_fwd, fl_bwd = 2 * unit, 5 * unit
    value = total_flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    eb = 2 if w.dtype == "bf16" else 4
    nkv = w.B * w.Hkv * w.S * w.D
    parts = (ws_bytes - 2 * ((w.B * w.Hq * Sq * 4 + 255) // 256 * 256)) // (2 * nkv * 4)
    hbm_bytes = {"attn_bwd_dkdv_reduce": 2 * nkv * (4 * max(parts, 1) + eb),
                 # O and dO in, LSE in, -delta and lse * log2(e) out
                 "attn_bwd_prep": 2 * w.B * w.Hq * Sq * w.D * eb + 12 * w.B * w.Hq * Sq}

    kernels = {}
    for name, t in kern_ms.items():
        rec = {"avg_ms": round(t, 4)}
        if name in fl:
            rec["tflops"] = round(fl[name] / (t * 1e-3) / 1e12, 1)
        elif name in hbm_bytes:
            rec["gbs"] = round(hbm_bytes[name] / (t * 1e-3) / 1e9, 1)
        prof = load_profile(name, w.name)  # counters taken on this kernel source, else absent
        if prof is not None:
            for key in ("mfma_busy", "mfma_insts_per_launch", "bytes_per_launch"):
                if prof.get(key) is not None:
                    rec[key] = prof[key]
            if prof.get("bytes_per_launch"):
                rec["hbm_gbs"] = round(prof["bytes_per_launch"] / (t * 1e-3) / 1e9, 1)
        kernels[name] = rec
    dom = max(kern_ms, key=kern_ms.get)
    if dom in fl:
        ach = fl[dom] / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    else:
        ach = hbm_bytes[dom] / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["traffic"] = load_traffic(dom, w.name)
    prof = load_profile(dom, w.name)
    roof["mfma_busy"] = None if prof is None else prof.get("mfma_busy")

    out = {
        "metric": METRIC if w.name == DEFAULT_WORKLOAD else f"fwd+bwd attn TFLOP/s & % bf16 MFMA peak ({w.name})",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
                   "causal": w.causal, "window": w.window, "parallelism": "none (1 GPU)",
                   **({"Sq": Sq} if Sq != w.S else {}), **({"sink": w.sink} if w.sink else {}),
                   **({"documents": [int(x) for x in cu[0]]} if cu is not None else {})},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "phase_ms": phases,
        "phase_tflops_median": {
            "fwd": round(fl_fwd / (phases["fwd"]["median"] * 1e-3) / 1e12, 1),
            "bwd": round(fl_bwd / (phases["bwd"]["median"] * 1e-3) / 1e12, 1),
            "fwd+bwd": round(total_flops / (phases["fwd+bwd"]["median"] * 1e-3) / 1e12, 1)},
        "device_peak_bf16": device_peak_bf16(torch),
        "ms_per_step_with_kernel_events": round(ms_hooked, 4),
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, do, args.cpu_heads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
