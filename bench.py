#!/usr/bin/env python3
"""Attention forward throughput on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole forward path over the workload's batch of
synthetic input.  The default workload is the largest configuration: the
TileMix-routed causal prefill of 16384 tokens (hdim 128, 32 query heads over
8 kv heads, 4 key tiles per routing bit, bits drawn Bernoulli(0.5)), one
forward call per step; its all-FP16 run (the same inputs and kernel with a
zero bitmask) is timed in the same invocation and reported in the same line.
Inputs are resident in HBM before the timed region starts.  The value is the
throughput convention of the "Nax Refactor" timing tables (ml-explore/mlx
pull request 3271): 4*B*n_qh*qsl*ksl*hdim FLOP per call, halved when causal,
divided by wall time.  Before the W warmup steps, untimed steps run for about
one second (--settle-ms), so that the GPU clock has left its idle level
before anything is timed.

Printed: one JSON line with the metric, a roofline record of the dominant
kernel (its per-launch time measured with HIP events on its own stream, in a
second pass over the same steps, since event records cost GPU time of their
own; routed kernels are priced against the fp16/INT8 mixed MFMA peak of
their drawn bitmask) and the CPU oracle's throughput on a bounded sample of
the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

FP16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU, dense fp16 MFMA
INT8_PEAK_TOPS = 5033.2
METRIC = "attention fwd TFLOP/s (4·B·n_qh·qsl·ksl·d, causal halved) and % MFMA peak"

# The page's fused-kernel figures for the same shapes (hardware not stated on
# the page): TFLOP/s as printed and the printed time per 64 calls.
PAGE_ROWS = {  # (qsl, ksl, hdim, n_qh, n_kvh, causal) -> (t_fus for 64 calls, tflops)
    (1024, 1024, 64, 32, 32, 0): (0.039, 14.263),
    (1024, 1024, 64, 32, 32, 1): (0.022, 12.252),
    (4096, 4096, 128, 32, 8, 1): (0.685, 12.834),
    (512, 4096, 128, 32, 8, 1): (0.168, 6.548),
}

DEFAULT_WORKLOAD = "tilemix_16384_d128_causal"
# named sets of calls per step: the 1024-token pair is the page's first
# two "After" rows (one non-causal and one causal call on the same Q/K/V)
BENCH_SETS = {
    "dense_1024_d64_pair": ["dense_1024_d64", "dense_1024_d64_causal"],
}
for _n in W.WORKLOADS:
    BENCH_SETS.setdefault(_n, [_n])

COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "attention_prefill_amd", "csrc", f) for f in ("attn_kernels.hip", "attn_device.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="before the warmup steps, run untimed steps until this much wall time has "
                         "passed, so that the GPU clock has reached its sustained level (0: none)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(BENCH_SETS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU oracle baseline (default: the process's CPUs, or OMP_NUM_THREADS)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the all-FP16 and dense runs of a routed workload (for profiler runs whose "
                         "per-kernel averages must cover the drawn bitmask only)")
    ap.add_argument("--fp16-compare", action="store_true",
                    help="INT8-cache workloads: also time the fp16 K and V the cache was encoded "
                         "from (routed workloads always time their all-FP16 run and the dense "
                         "kernel on the same inputs)")
    ap.add_argument("--unfused-compare", action="store_true",
                    help="dense fp16 workloads: also time the unfused baseline (score GEMM, masked "
                         "softmax, P.V GEMM) on the same inputs, the page's t_unfs / speed_up")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (reference for HBM byte counters) and exit")
    return ap.parse_args()


class Call:
    """One forward call of a workload with its device inputs."""

    def __init__(self, w, A, torch):
        self.w = w
        q, k, v = W.draw_qkv(w)
        self.host = (q, k, v)
        self.q, self.k, self.v = (torch.from_numpy(a).cuda() for a in (q, k, v))
        self.out = torch.empty_like(self.q)
        self.cu = torch.from_numpy(W.cu_seqlens_of(w.seqlens)).cuda() if w.varlen else None
        r = W.route_for(w)
        self.route_host = r
        self.route = None if r is None else torch.from_numpy(r.view(np.int32)).cuda()
        self.A = A
        self.metric_flop, self.visited_flop = W.workload_flop(w)
        self.zero_route = None if r is None else torch.zeros_like(self.route)
        if w.kv8:
            # the INT8 key/value cache, encoded on the device before timing
            self.k8, self.sk = A.attn_quantize_rows(self.k)
            self.v8, self.sv = A.attn_quantize_rows(self.v)

    def unfused(self, stream):
        """The unfused baseline on the same dense fp16 inputs."""
        self.A.attn_fwd_unfused(self.q, self.k, self.v, self.out, scale=self.w.scale, causal=self.w.causal,
                                stream=stream)

    def prepared(self, stream, route="drawn", fp16_kv=False):
        """One call of the workload as a zero-argument function with its C-ABI
        arguments marshalled once, so that the timed loop measures the library
        and not this script's Python.  route: "drawn" (the workload's bitmask),
        "zero" (same kernel, every tile FP16) or "none" (no bitmask: the dense
        kernel).  fp16_kv: a cache workload's call on the fp16 K and V it was
        encoded from."""
        import ctypes
        w = self.w
        lib = self.A._lib.load()
        vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        B = len(w.seqlens) if w.varlen else w.B
        rt = {"drawn": self.route, "zero": self.zero_route, "none": None}[route]
        common = (B, w.qsl, w.ksl, w.hdim, w.n_qh, w.n_kvh, float(w.scale), int(bool(w.causal)), vp(self.cu), vp(rt),
                  int(w.tiles_per_bit or 4))
        sh = ctypes.c_void_p(stream.cuda_stream)
        if w.kv8 and not fp16_kv:
            fn, args = lib.attn_fwd_kv8_stream, (vp(self.q), vp(self.k8), vp(self.sk), vp(self.v8), vp(self.sv),
                                                 vp(self.out)) + common + (sh,)
        elif w.lowp != "int8" and rt is not None:
            fn, args = lib.attn_fwd_lowp_stream, (vp(self.q), vp(self.k), vp(self.v), vp(self.out)) + common + \
                (self.A._lib.LOWP[w.lowp], sh)
        else:
            fn, args = lib.attn_fwd_stream, (vp(self.q), vp(self.k), vp(self.v), vp(self.out)) + common + (sh,)
        check = self.A._lib._check

        def go():
            check(fn(*args))
        return go


def host_cpu():
    """(logical CPUs of the host, CPUs this process may run on, CPU model)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count() or 1
    return os.cpu_count() or 1, allowed, model


def cpu_baseline(calls, budget_s=12.0, threads=0):
    """The oracle, untuned, on a bounded sample: whole query heads of each call
    (full sequence length, the same inputs), as many as fit the time budget.
    Threads: `threads` if given, else every CPU this process may run on, or
    OMP_NUM_THREADS when the host sets it (the GPU's share of a shared host)."""
    import oracle
    nproc, allowed, model = host_cpu()
    threads = threads or int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or allowed
    flop = secs = 0.0
    samples = []
    for c in calls:
        w = c.w
        q, k, v = c.host
        if w.kv8:
            k8, sk = oracle.quantize_rows(k)
            v8, sv = oracle.quantize_rows(v)
        G = w.n_qh // w.n_kvh
        cu = W.cu_seqlens_of(w.seqlens) if w.varlen else None
        spent = 0.0
        heads = 0
        for h in range(w.n_qh):
            if heads and spent > budget_s / len(calls):
                break
            hk = h // G
            if w.varlen:
                qs, ks, vs = q[h:h + 1], k[hk:hk + 1], v[hk:hk + 1]
            else:
                qs, ks, vs = q[:, h:h + 1], k[:, hk:hk + 1], v[:, hk:hk + 1]
            sl = (slice(hk, hk + 1),) if w.varlen else (slice(None), slice(hk, hk + 1))
            t0 = time.perf_counter()
            if w.kv8:
                oracle.attn_fwd_kv8(np.ascontiguousarray(qs), np.ascontiguousarray(k8[sl]),
                                    np.ascontiguousarray(sk[sl]), np.ascontiguousarray(v8[sl]),
                                    np.ascontiguousarray(sv[sl]), scale=w.scale, causal=w.causal,
                                    cu_seqlens=cu, route=c.route_host, tiles_per_bit=w.tiles_per_bit or 4,
                                    nthreads=threads)
            else:
                oracle.attn_fwd(np.ascontiguousarray(qs), np.ascontiguousarray(ks), np.ascontiguousarray(vs),
                                scale=w.scale, causal=w.causal, cu_seqlens=cu, route=c.route_host,
                                tiles_per_bit=w.tiles_per_bit or 4, lowp=w.lowp, nthreads=threads)
            spent += time.perf_counter() - t0
            heads += 1
        flop += c.metric_flop * heads / w.n_qh
        secs += spent
        samples.append("%s: %d of %d query heads" % (w.name, heads, w.n_qh))
    return {"value": flop / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(samples) + ", full sequence length, same inputs; %.1f s" % secs,
            "host_logical_cpus": nproc, "process_cpus": allowed, "cpu_model": model,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def int8_share(w, route):
    """Share of the visited score (QK^T) pairs that a drawn bitmask sends to
    the low-precision route: bits decoded LSB-first, each (query tile, key
    tile) counted by its causally visible pairs."""
    T = 64
    n_kt = -(-w.ksl // T)
    n_g = -(-n_kt // w.tiles_per_bit)
    bits = np.unpackbits(np.ascontiguousarray(route, dtype=np.uint32).view(np.uint8).reshape(route.shape[0], -1),
                         axis=1, bitorder="little")[:, :n_g].astype(bool)
    off = w.ksl - w.qsl if w.causal else 0
    low = tot = 0
    for qt in range(-(-w.qsl // T)):
        rows = np.arange(qt * T, min(qt * T + T, w.qsl))
        lim = np.minimum(w.ksl, rows + off + 1) if w.causal else np.full(rows.size, w.ksl)
        for kt in range(n_kt):
            pairs = int(np.clip(lim - kt * T, 0, min(T, w.ksl - kt * T)).sum())
            tot += pairs
            if bits[qt, kt // w.tiles_per_bit]:
                low += pairs
    return low / tot if tot else 0.0


def kernel_source_sha256():
    """sha256 over the kernel sources (attn_kernels.hip, then attn_device.h)."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def hbm_traffic(workload, dominant_name):
    """HBM bytes per launch of the dominant kernel of this workload from the
    committed counter summary, or None when the counters were not taken on
    this workload or the kernel source changed since they were."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
        sha = kernel_source_sha256()
        if rec.get("kernel_source_sha256") != sha:
            return None
        ent = rec["workloads"].get(workload, {}).get(dominant_name)
        if not ent:
            return None
        return ent["fetch_kib"] * 1024.0 * rec["fetch_scale"] + ent["write_kib"] * 1024.0 * rec["write_scale"]
    except (OSError, ValueError, KeyError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()           # default priority

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(3):
                dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return

    import attention_prefill_amd as A
    A.load()
    names = BENCH_SETS[args.workload]
    calls = [Call(W.WORKLOADS[n], A, torch) for n in names]
    torch.cuda.synchronize()

    fns = [c.prepared(stream) for c in calls]

    def step():
        for f in fns:
            f()

    # the GPU raises its clock only after tens of milliseconds of sustained
    # work: without this, short workloads are timed partly at idle clocks
    settle_steps = 0
    ts = time.perf_counter()
    while (time.perf_counter() - ts) * 1e3 < args.settle_ms:
        step()
        torch.cuda.synchronize()
        settle_steps += 1
    settle_ms = (time.perf_counter() - ts) * 1e3

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps: calls only
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / args.steps

    # the dominant kernel (the call with the most FLOP): the same steps again,
    # with HIP events recorded around that kernel on its stream.  An event
    # record is a timestamped barrier packet that costs GPU time of its own,
    # so the throughput above is timed without them.
    dom = max(range(len(calls)), key=lambda i: calls[i].visited_flop)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for s in range(args.steps):
        for i, f in enumerate(fns):
            if i == dom:
                ev[s][0].record(stream)
            f()
            if i == dom:
                ev[s][1].record(stream)
    torch.cuda.synchronize()
    te1 = time.perf_counter()

    metric_flop = sum(c.metric_flop for c in calls)
    value = metric_flop / sec_per_step / 1e12
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    dc = calls[dom]
    achieved = dc.visited_flop / (dom_ms * 1e-3) / 1e12
    dw = dc.w
    dom_name = "attn_fwd_kernel hd%d %s%s%s%s" % (dw.hdim, "causal" if dw.causal else "noncausal",
                                                   " varlen" if dw.varlen else "",
                                                   (" routed" + (" fp8" if dw.lowp == "fp8" else ""))
                                                   if dw.tiles_per_bit else "",
                                                   " kv8" if dw.kv8 else "")
    # Peak: dense fp16 MFMA, or for a routed kernel the mixed peak of its
    # drawn bitmask: with a share f of the score FLOP (half of all FLOP) on
    # the INT8 / FP8 MFMA at twice the fp16 rate, the MFMA time floor is
    # F / P16 * (1 - f / 4).
    peak = FP16_PEAK_TFLOPS
    share = None
    if dc.route_host is not None:
        share = int8_share(dw, dc.route_host)
        peak = FP16_PEAK_TFLOPS / (1.0 - share / 4.0)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": hbm_traffic(args.workload, dom_name), "kernel": dom_name,
                "flop_per_launch": dc.visited_flop, "avg_launch_ms": round(dom_ms, 5),
                "ms_per_step_with_events": round((te1 - te0) / args.steps * 1e3, 5)}
    if share is not None:
        roofline.update({"peak_kind": "fp16/%s mixed MFMA for the drawn bitmask" % dw.lowp,
                         "lowp_share_of_score_flop": round(share, 4), "peak_fp16": FP16_PEAK_TFLOPS,
                         "frac_of_fp16_peak": round(achieved / FP16_PEAK_TFLOPS, 4)})

    # the page's figures for the same shapes, combined like the value
    page = []
    for c in calls:
        w = c.w
        key = (w.qsl, w.ksl, w.hdim, w.n_qh, w.n_kvh, int(w.causal))
        if w.B == 1 and not w.varlen and not w.tiles_per_bit and not w.kv8 and key in PAGE_ROWS:
            page.append(PAGE_ROWS[key][0] / 64.0)
    # vs_baseline: the page's own fused figure for exactly this workload (its
    # hardware is not stated: context, not a same-machine speed-up); null for
    # workloads the page does not time
    vs = None
    if len(page) == len(calls):
        vs = round(value / (metric_flop / sum(page) / 1e12), 3)

    w0 = calls[0].w
    cfg = {"workload": args.workload, "B": len(w0.seqlens) if w0.varlen else w0.B, "qsl": w0.qsl,
           "ksl": w0.ksl, "hdim": w0.hdim, "n_qh": w0.n_qh, "n_kvh": w0.n_kvh,
           "causal": [c.w.causal for c in calls] if len(calls) > 1 else w0.causal,
           "seqlens": w0.seqlens, "tiles_per_bit": w0.tiles_per_bit or None, "kv_cache_int8": w0.kv8,
           "low_precision_route": w0.lowp if w0.tiles_per_bit else None,
           "calls_per_step": len(calls)}
    rec = {"metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_steps": settle_steps,
           "settle_ms": round(settle_ms, 1), "ms_per_step": round(sec_per_step * 1e3, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": vs, "dtype": "fp16",
           "data": "synthetic: i.i.d. N(0,1) Q/K/V cast to fp16 (numpy default_rng, seeded)" +
                   ("; K and V as an INT8 key/value cache encoded on the device"
                    if any(c.w.kv8 for c in calls) else ""),
           "config": cfg, "pct_fp16_peak": round(100 * value / FP16_PEAK_TFLOPS, 2),
           "roofline": roofline}
    def time_route(route, fp16_kv=False):
        rf = [c.prepared(stream, route, fp16_kv) for c in calls]
        for _ in range(args.warmup):
            for f in rf:
                f()
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for _ in range(args.steps):
            for f in rf:
                f()
        torch.cuda.synchronize()
        return (time.perf_counter() - ta) / args.steps

    if vs is not None:
        rec["vs_baseline_note"] = "the page's fused time for these shapes; its hardware is not stated"
    if any(c.route is not None for c in calls) and not args.no_compare:
        # the all-FP16 run of the same inputs (the same kernel with a zero
        # bitmask) and, for context, the dense kernel with no bitmask at all;
        # the three are timed in interleaved rounds (K steps each, medians
        # over the rounds), so that clock drift over the run does not favour
        # whichever runs first
        rounds = {"drawn": [], "zero": [], "none": []}
        for _ in range(3):
            for r in rounds:
                rounds[r].append(time_route(r))
        med = {r: float(np.median(v)) for r, v in rounds.items()}
        rec["all_fp16_ms_per_step"] = round(med["zero"] * 1e3, 5)
        rec["all_fp16_tflops"] = round(metric_flop / med["zero"] / 1e12, 3)
        rec["routed_ms_per_step_interleaved"] = round(med["drawn"] * 1e3, 5)
        rec["routed_speedup_vs_all_fp16"] = round(med["zero"] / med["drawn"], 4)
        rec["dense_no_bitmask_ms_per_step"] = round(med["none"] * 1e3, 5)
        rec["routed_speedup_vs_dense"] = round(med["none"] / med["drawn"], 4)
    if args.fp16_compare and any(c.w.kv8 for c in calls):
        # the same call on the fp16 K and V the cache was encoded from
        kv16_step = time_route("drawn", fp16_kv=True)
        rec["fp16_kv_ms_per_step"] = round(kv16_step * 1e3, 5)
        rec["kv8_speedup_vs_fp16_kv"] = round(kv16_step / sec_per_step, 4)
    if args.unfused_compare and all(not c.w.varlen and not c.w.tiles_per_bit and not c.w.kv8 for c in calls):
        # the page's other column: the same step through the unfused baseline
        for _ in range(args.warmup):
            for c in calls:
                c.unfused(stream)
        torch.cuda.synchronize()
        ta = time.perf_counter()
        for _ in range(args.steps):
            for c in calls:
                c.unfused(stream)
        torch.cuda.synchronize()
        unf_step = (time.perf_counter() - ta) / args.steps
        rec["unfused_ms_per_step"] = round(unf_step * 1e3, 5)
        rec["fused_speedup_vs_unfused"] = round(unf_step / sec_per_step, 3)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(calls, threads=args.cpu_threads)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
