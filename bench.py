#!/usr/bin/env python3
"""Benchmark: per-token weight sweep of 64 synthetic 27B-shaped decoder
layers (q, k, v, o, gate, up, down; 10.16 GB of PN-packed weights), M = 1,
on one MI355X.

A step is one token: every one of the 448 GEMVs, each with its own fp16
input, all inputs resident in HBM before timing starts.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--schedule token|layer|gemv|token_rot]
                  [--config 3|4] [--math mfma|valu] [--no-cpu-baseline]

--config 4 runs the same sweep with M = 8 activation rows per matrix (the
small-batch kernels; --math picks their arithmetic, the other one is timed
beside it; --m 16 gives the k = 15 verification width).

value = algorithmic bytes per token (packed weights + fp16 inputs + fp32
outputs) / step time, in GB/s; tokens/s is reported beside it.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PN GEMV achieved HBM GB/s (% of peak) + 27B-shaped layer-sweep tokens/s"
PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
# Sources of the kernel each counted workload times (the M = 1 one-launch
# sweep: gemv_rows; M > 1: gemm_stream): the committed counters are valid for
# one hash of these.
KERNEL_SOURCES = {
    "m1": ["bit_quantized_decode_pn3t_amd/csrc/pn_gemv_rows.hip",
           "bit_quantized_decode_pn3t_amd/csrc/pn_device.h"],
    "smallm": ["bit_quantized_decode_pn3t_amd/csrc/pn_smallm.hip",
               "bit_quantized_decode_pn3t_amd/csrc/pn_device.h"],
    "prefill": ["bit_quantized_decode_pn3t_amd/csrc/pn_prefill.hip",
                "bit_quantized_decode_pn3t_amd/csrc/pn_device.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_hash(kind):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kind):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_hash") != kernel_hash(kind):
        return None
    return e.get("bytes_per_launch")


def per_config_timing(B, synth, torch):
    """Workloads 0-2 one call at a time: HIP events around every call, >= 50
    timed calls after 10 warm-up calls, queued on the GPU ahead of their
    execution, rotating weight copies so that workloads 1 and 2 come from HBM
    rather than the 256 MB last-level cache.
    Workload 2's codes are random bytes of its shape: its quantized weights
    come from the oracle, and the bytes moved are the same."""
    import numpy as np

    def stats(ms, nbytes):
        a = np.sort(np.array(ms))
        q = lambda f: float(a[min(len(a) - 1, int(f * len(a)))])
        return {"us_p10": round(q(0.1) * 1e3, 2), "us_p50": round(q(0.5) * 1e3, 2),
                "us_p90": round(q(0.9) * 1e3, 2), "gbps_p50": round(nbytes / (q(0.5) * 1e-3) / 1e9, 1),
                "bytes_per_call": nbytes, "calls": len(ms)}

    # A call takes longer to issue from Python than the smaller launches take
    # to run, so the calls are queued behind a short spin kernel: the events
    # then bracket each launch as the GPU runs it back to back, not the host's
    # issue time.
    def spin_cycles_per_ms():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1 << 20)
        b.record()
        torch.cuda.synchronize()
        return (1 << 20) / max(a.elapsed_time(b), 1e-3)

    cpm = spin_cycles_per_ms()

    def timed(fn, copies, calls=60, warm=10):
        t0 = time.perf_counter()
        for i in range(warm):
            fn(i % copies)
        torch.cuda.synchronize()
        issue_ms = (time.perf_counter() - t0) * 1e3 / warm  # per call, an upper bound
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        torch.cuda._sleep(int(cpm * (2.0 * issue_ms * calls + 5.0)))
        for i, (a, b) in enumerate(ev):
            a.record()
            fn(i % copies)
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    out = {}
    dev = torch.device("cuda")
    c0 = synth.config0()
    w0 = torch.from_numpy(c0["W"]).to(dev)
    x0 = torch.from_numpy(c0["x"]).to(dev)
    y0 = torch.empty(c0["N"], dtype=torch.float32, device=dev)
    ms = timed(lambda i: B.pn_gemv("pn3t", w0, 256, 5120, x0, y0), 1, calls=200)
    out["workload0_pn3t_256x5120"] = dict(stats(ms, c0["W"].nbytes + 5120 * 2 + 256 * 4),
                                          note="L2-resident: a latency, not an HBM rate")
    c1 = synth.config1()
    w1 = [torch.from_numpy(c1["W"]).to(dev) for _ in range(8)]
    x1 = torch.from_numpy(c1["x"]).to(dev)
    y1 = torch.empty(c1["N"], dtype=torch.float32, device=dev)
    ms = timed(lambda i: B.pn_gemv("pn4t", w1[i], 5120, 17408, x1, y1), 8)
    out["workload1_pn4t_5120x17408"] = dict(stats(ms, c1["W"].nbytes + 17408 * 2 + 5120 * 4), copies=8)
    del w1
    g = synth.rng(2, 0, 3)
    wg = [torch.from_numpy(synth.random_blocks(g, "pn3t", 17408, 5120)).to(dev) for _ in range(4)]
    wu = [torch.from_numpy(synth.random_blocks(g, "pn3t", 17408, 5120)).to(dev) for _ in range(4)]
    x2 = torch.from_numpy(synth.activation(g, 5120)).to(dev)
    yg = torch.empty(17408, dtype=torch.float32, device=dev)
    yu = torch.empty(17408, dtype=torch.float32, device=dev)
    ms = timed(lambda i: B.pn_gemv2("pn3t", wg[i], wu[i], 17408, 5120, x2, yg, yu), 4)
    out["workload2_gate_up_2x17408x5120"] = dict(stats(ms, 2 * wg[0].numel() + 5120 * 2 + 2 * 17408 * 4),
                                                 copies=4, codes="random bytes of the shape")
    del wg, wu
    torch.cuda.empty_cache()
    return out


PEAK_TFLOPS_F16 = 2500.0  # MI355X dense fp16 MFMA, AMD's published figure


def prefill_timing(B, synth, torch, m=512, layer_only=False):
    """Prefill of one 27B-shaped decoder layer (q, k, v, o, gate, up, down;
    weights decoded inside the MFMA GEMM) for an m-token prompt chunk, in
    the four launches a decoder can make in dependency order: {q, k, v} and
    {gate, up} as pn_gemm_prefill_group launches (products whose inputs are
    ready together), {o} and {down} as pn_gemm_prefill.  The launches are
    queued back to back behind a short spin kernel (so that the host's issue
    time is not measured), HIP events around them, median of 10.  The seven
    products one launch each, and each product alone, are timed the same
    way.  Flops = 2 m N K per product.  layer_only: the four launches only
    (13 layers: 3 untimed, 10 timed), for the counter runs."""
    import numpy as np
    from bit_quantized_decode_pn3t_amd.sweep import LAYER_GROUPS
    dev = torch.device("cuda")
    g = synth.rng(5, 0, 0)
    mats = []
    flops = 0
    for name, t, n, k in synth.SWEEP_LAYER:
        w = torch.from_numpy(synth.random_blocks(g, t, n, k)).to(dev)
        x = torch.from_numpy(synth.activation(g, k, m)).to(dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        mats.append((name, t, n, k, w, x, y))
        flops += 2 * m * n * k
    # each product reads its weights and its X once and writes its Y once
    algo = sum(w.numel() + 2 * m * k + 4 * m * n for _, t, n, k, w, x, y in mats)

    def call(e):
        name, t, n, k, w, x, y = e
        B.pn_gemm_prefill(t, w, n, k, x, k, m, y, n)

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(1 << 20)
    b.record()
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(a.elapsed_time(b), 1e-3)

    def queued(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda._sleep(int(cycles_per_ms * 10.0))  # longer than the host takes to queue the calls
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    def grouped():
        for grp in LAYER_GROUPS:
            if len(grp) == 1:
                call(mats[grp[0]])
            else:
                B.pn_gemm_prefill_group([(t, w, n, k, x, k, m, y, n)
                                         for _, t, n, k, w, x, y in (mats[i] for i in grp)])

    if layer_only:
        total_ms = queued(grouped)
        return {"ms_per_layer": round(total_ms, 4), "layers_run": 13, "algorithmic_bytes_per_layer": algo}
    per = {}
    for e in mats:
        ms = queued(lambda: call(e))
        per[e[0]] = {"ms": round(ms, 4), "tflops": round(2 * m * e[2] * e[3] / (ms * 1e-3) / 1e12, 1)}
    groups = {}
    for grp in LAYER_GROUPS:
        if len(grp) > 1:
            sub = [mats[i] for i in grp]
            ms = queued(lambda: B.pn_gemm_prefill_group([(t, w, n, k, x, k, m, y, n) for _, t, n, k, w, x, y in sub]))
            gf = sum(2 * m * e[2] * e[3] for e in sub)
            groups["+".join(e[0] for e in sub)] = {"ms": round(ms, 4), "tflops": round(gf / (ms * 1e-3) / 1e12, 1)}
    single_ms = queued(lambda: [call(e) for e in mats])
    total_ms = queued(grouped)
    del mats
    torch.cuda.empty_cache()
    tf = flops / (total_ms * 1e-3) / 1e12
    return {"workload": "prefill of one 27B-shaped layer, %d-token chunk" % m, "tokens": m,
            "schedule": "4 launches in dependency order: {q,k,v} grouped, {o}, {gate,up} grouped, {down}",
            "ms_per_layer": round(total_ms, 4), "tflops": round(tf, 1),
            "tokens_per_s_64_layers": round(m / (64 * total_ms * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_TFLOPS_F16, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_TFLOPS_F16, 4),
                         "traffic": measured_traffic("prefill_layer_m512", "prefill"),
                         "algorithmic_bytes_per_layer": algo,
                         "kernel": "gemm_prefill",
                         "note": "the layer's four launches queued back to back, events around the four"},
            "seven_launches": {"ms_per_layer": round(single_ms, 4),
                               "tflops": round(flops / (single_ms * 1e-3) / 1e12, 1),
                               "note": "each product its own pn_gemm_prefill launch"},
            "groups": groups,
            "per_matrix": per,
            "kernel_hash": kernel_hash("prefill")}


def layer_read_floor(B, torch, layers):
    """What the four-launches-per-layer schedule can reach at best: the
    library's streaming-read probe in place of each of its launches ({q,k,v},
    {o}, {gate,up}, {down} of every layer, one HIP graph, 8 rotating copies
    of a layer's buffers so that every launch reads from HBM), no arithmetic.
    The probe reads whole 1 KiB instructions per wave, so each launch reads
    a little less than the group it stands for; the rate uses the bytes read."""
    from bit_quantized_decode_pn3t_amd import sweep as S
    from bit_quantized_decode_pn3t_amd import synth
    sizes = [sum(synth.row_bytes(synth.SWEEP_LAYER[j][1], synth.SWEEP_LAYER[j][3]) * synth.SWEEP_LAYER[j][2]
                 for j in grp) for grp in S.LAYER_GROUPS]
    copies = 8
    bufs = [[torch.ones(sz // 4096 * 4096, dtype=torch.uint8, device="cuda") for sz in sizes] for _ in range(copies)]
    scratch = torch.empty(B.pn_read_probe_scratch_bytes() // 4, dtype=torch.int32, device="cuda")
    got = []

    def step():
        got.clear()
        for l in range(layers):
            for b in bufs[l % copies]:
                got.append(B.pn_read_probe(b, b.numel(), scratch, scratch.numel() * 4))

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = 10
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nread = sum(got)
    del g, bufs, scratch
    torch.cuda.empty_cache()
    return {"launches_per_token": len(got), "bytes_per_token": nread, "ms_per_token": round(ms, 4),
            "gbps": round(nread / (ms * 1e-3) / 1e9, 1),
            "note": "read probe in place of every launch of the layer schedule (HIP graph); "
                    "the same bytes in one launch run at read_ceiling_gbps"}


def host_read_gbps():
    """Host memory read rate (numpy sum over 1 GiB of uint64, best of 3)."""
    import numpy as np
    a = np.ones(1 << 27, dtype=np.uint64)
    best = None
    for _ in range(3):
        t0 = time.perf_counter()
        a.sum()
        dt = time.perf_counter() - t0
        best = dt if best is None or dt < best else best
    return round(a.nbytes / best / 1e9, 2)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(layers, threads, m=None):
    """The oracle (fp64 decode + GEMV, C, OpenMP over rows) on a bounded
    sample of the sweep: the first `layers` layers, scaled to one token."""
    from bit_quantized_decode_pn3t_amd import synth
    from oracle import pnref

    used = pnref.set_threads(threads)
    recs = synth.sweep_matrices(layers=layers, m=m, config=3 if m is None else 4, threads=min(16, threads))
    sample_bytes = sum(r["W"].nbytes for r in recs)
    pnref.gemv_f64(recs[0]["type"], recs[0]["W"][:64], 64, recs[0]["K"],
                   recs[0]["x"] if m is None else recs[0]["x"][0])  # warm
    t0 = time.perf_counter()
    for r in recs:
        if m is None:
            pnref.gemv_f64(r["type"], r["W"], r["N"], r["K"], r["x"])
        else:
            pnref.gemm_f64(r["type"], r["W"], r["N"], r["K"], r["x"])
    dt = time.perf_counter() - t0
    return dt, sample_bytes, used


def token_timing(B, torch, sw, steps, warmup):
    """Time the one-launch token schedule of `sw`: HIP events on the launch
    stream around every launch (one kernel per step), after `warmup` runs."""
    sw.prepare("token")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        sw.step("token")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        sw.step("token")
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in evs], B.pn_variant_name(B.pn_last_variant())


def smallm_m8_timing(B, torch, sw, steps, m=8):
    """The M = 8 verification-batch sweep (the same resident weights, an 8-row
    activation batch per matrix): one grouped launch per token with the MFMA
    arithmetic (the library's pick: gemm_rows) and with the VALU arithmetic,
    each with its kernel's roofline from per-launch events."""
    v = sw.batch_view(m)
    bytes_per_token = v.weight_bytes + v.act_bytes
    out = {"workload": "64-layer 27B-shaped sweep, M=%d, token schedule" % m, "bytes_per_token": bytes_per_token}
    try:
        for math in ("mfma", "valu"):
            B.pn_set_smallm_math(math)
            v.close()  # a plan keeps the arithmetic it was created with
            wall, ev_ms, variant = token_timing(B, torch, v, steps, 5)
            kern_ms = sum(ev_ms) / len(ev_ms)
            achieved = bytes_per_token / (kern_ms * 1e-3) / 1e9
            workload = "sweep64_m%d_token_%s" % (m, math)
            out[math] = {"ms_per_token": round(wall / steps * 1e3, 4), "tokens_per_s": round(steps / wall, 2),
                         "gbps": round(bytes_per_token / (wall / steps) / 1e9, 1), "variant": variant,
                         "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS,
                                      "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                                      "traffic": measured_traffic(workload, "smallm"),
                                      "kernel": variant.replace("_group", ""), "kernel_avg_ms": round(kern_ms, 4),
                                      "algorithmic_bytes_per_launch": bytes_per_token}}
            log("M=%d token %s: %.4f ms per token (%s)" % (m, math, kern_ms, variant))
    finally:
        B.pn_set_smallm_math("mfma")
        v.close()
        del v
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--schedule", default="token", choices=["token", "layer", "gemv", "token_rot"])
    ap.add_argument("--config", type=int, default=3, choices=[3, 4],
                    help="3: the 64-layer sweep at M = 1 (the default); 4: the same sweep with M activation "
                         "rows per matrix (--m, 8 by default)")
    ap.add_argument("--math", default="mfma", choices=["mfma", "valu"],
                    help="small-batch arithmetic (--config 4)")
    ap.add_argument("--m", type=int, default=8, help="activation rows with --config 4 (1..16)")
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other schedules")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill layer's four launches (for counter runs); prints their JSON")
    ap.add_argument("--cpu-layers", type=int, default=None,
                    help="layers in the oracle's sample (default 64 at M=1, 8 at M=8)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the one-call timings of workloads 0-2")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one device copy of this many MiB (a kernel of known traffic "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_quantized_decode_pn3t_amd import _binding as B
    from bit_quantized_decode_pn3t_amd import sweep as S
    from bit_quantized_decode_pn3t_amd import synth

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read, %d written" % (n, n))
        del src, dst
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_timing(B, synth, torch, layer_only=True)}), flush=True)
        return
    m = None if args.config == 3 else args.m
    schedule = args.schedule
    if m is not None and schedule == "layer":
        print("--config 4 runs the token and gemv schedules", file=sys.stderr)
        sys.exit(2)
    if m is not None:
        B.pn_set_smallm_math(args.math)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))  # input generation
    cpu_threads = len(os.sched_getaffinity(0))  # the oracle: every core of the affinity mask

    t0 = time.perf_counter()
    log("generating %d layers (M=%s) with %d threads" % (args.layers, m or 1, threads))
    sw = S.Sweep(layers=args.layers, m=m, threads=threads)
    torch.cuda.synchronize()
    bytes_per_token = sw.weight_bytes + sw.act_bytes
    log("resident: %.3f GB weights, %d matrices, %.1f s" % (sw.weight_bytes / 1e9, len(sw.mats),
                                                            time.perf_counter() - t0))

    def run_timed(sched, steps, warmup, per_step_events):
        use_graph = sched in ("layer", "gemv")
        g = sw.capture(sched) if use_graph else None
        if not use_graph:
            sw.prepare(sched)
        stream = torch.cuda.current_stream()

        def one():
            if g is not None:
                g.replay()
            else:
                sw.step(sched)

        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)] if per_step_events else []
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            if per_step_events:
                evs[i][0].record(stream)
            one()
            if per_step_events:
                evs[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        ev_ms = [a.elapsed_time(b) for a, b in evs]
        return wall, ev_ms, B.pn_variant_name(B.pn_last_variant())

    log("timing %d steps (%d warmup), schedule %s" % (args.steps, args.warmup, schedule))
    wall, ev_ms, variant = run_timed(schedule, args.steps, args.warmup,
                                     per_step_events=(schedule == "token"))
    ms_per_step = wall / args.steps * 1e3
    value = bytes_per_token / (wall / args.steps) / 1e9
    tok_s = args.steps / wall

    workload = "sweep64_m1_%s" % schedule if m is None else "sweep64_m%d_%s_%s" % (m, schedule, args.math)
    kind = "m1" if m is None else "smallm"
    if schedule == "token":
        # one launch per step: the events bracket exactly the dominant kernel
        kern_ms = sum(ev_ms) / len(ev_ms)
        achieved = bytes_per_token / (kern_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_GBPS, 4), "traffic": measured_traffic(workload, kind),
                    "kernel": variant.replace("_group", ""),
                    "variant": variant, "kernel_avg_ms": round(kern_ms, 4),
                    "kernel_ms_min_p50_max": [round(min(ev_ms), 4), round(sorted(ev_ms)[len(ev_ms) // 2], 4),
                                              round(max(ev_ms), 4)],
                    "algorithmic_bytes_per_launch": bytes_per_token}
    else:
        roofline = {"bound": "hbm", "achieved": round(value, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                    "frac": round(value / PEAK_GBPS, 4), "traffic": measured_traffic(workload, kind),
                    "kernel": variant, "note": "step wall time over %d launches" % sw.launches(schedule)}

    launches = sw.launches(schedule)
    secondary = {}
    if not args.no_secondary:
        if m is None:
            others = [(o, None) for o in ("layer", "gemv", "token_rot") if o != schedule]
        else:
            other_math = "valu" if args.math == "mfma" else "mfma"
            others = [(o, args.math) for o in ("token", "gemv") if o != schedule] + [(schedule, other_math)]
        for other, math in others:
            if math is not None:
                B.pn_set_smallm_math(math)
                sw.close()  # plans keep the arithmetic they were created with
            w2, _, var2 = run_timed(other, args.steps, 2, False)
            key = other if math is None else "%s_%s" % (other, math)
            secondary[key] = {"tokens_per_s": round(args.steps / w2, 2),
                              "gbps": round(bytes_per_token / (w2 / args.steps) / 1e9, 1),
                              "launches_per_token": sw.launches(other), "variant": var2}
            if other == "token_rot":
                secondary[key]["ms_per_token"] = round(w2 / args.steps * 1e3, 4)
                secondary[key]["note"] = ("inputs in the unrotated basis: one Hadamard rotation launch over "
                                          "all 448 inputs, then the token launch")
            log("schedule %s: %.1f tok/s" % (key, args.steps / w2))
        if m is not None:
            B.pn_set_smallm_math(args.math)
    smallm = None
    if m is None and not args.no_secondary:
        log("M=8 verification-batch sweep on the same weights")
        smallm = smallm_m8_timing(B, torch, sw, args.steps)
    sw.close()
    del sw
    torch.cuda.empty_cache()

    # read ceiling of the device, measured with the library's streaming-read probe
    buf = torch.zeros(8 << 30, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(B.pn_read_probe_scratch_bytes() // 4, dtype=torch.int32, device="cuda")
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        nread = B.pn_read_probe(buf, buf.numel(), scratch, scratch.numel() * 4)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None or ms < best else best
    read_ceiling = nread / (best * 1e-3) / 1e9
    del buf, scratch
    torch.cuda.empty_cache()
    log("read ceiling %.1f GB/s" % read_ceiling)
    layer_floor = None
    if m is None and not args.no_secondary:
        log("read floor of the four-launches-per-layer schedule")
        layer_floor = layer_read_floor(B, torch, args.layers)
        # time per launch beyond what its bytes take at the one-launch read rate
        layer_floor["per_launch_overhead_us"] = round(
            (layer_floor["ms_per_token"] * 1e-3 - layer_floor["bytes_per_token"] / (read_ceiling * 1e9))
            / layer_floor["launches_per_token"] * 1e6, 2)
        log("layer schedule read floor %.1f GB/s" % layer_floor["gbps"])

    per_config = None
    if not args.no_configs and m is None:
        log("one-call timings of workloads 0-2")
        per_config = per_config_timing(B, synth, torch)
    prefill = None
    if not args.no_secondary and m is None:
        log("prefill of one layer, 512-token chunk")
        prefill = prefill_timing(B, synth, torch)

    cpu = None
    if not args.no_cpu_baseline:
        cpu_layers = args.cpu_layers or (64 if m is None else 8)
        log("cpu baseline: oracle on %d layers, %d threads" % (cpu_layers, cpu_threads))
        dt, sample_bytes, used = cpu_baseline(cpu_layers, cpu_threads, m)
        weights_per_token = sum(synth.row_bytes(t, k) * n for _, t, n, k in synth.SWEEP_LAYER) * args.layers
        token_fraction = sample_bytes / weights_per_token
        cpu = {"value": round(token_fraction / dt, 4), "unit": "tok/s", "cores": used, "kind": "oracle",
               "sample": "first %d of %d layers (%.2f GB packed, %.1f%% of a token) in %.2f s; "
                         "fp64 decode+%s, OpenMP over rows on every core of the affinity mask"
                         % (cpu_layers, args.layers, sample_bytes / 1e9, 100 * token_fraction, dt,
                            "GEMV" if m is None else "GEMM (M=%d)" % m),
               "gbps_packed": round(sample_bytes / dt / 1e9, 3),
               "affinity_cores": cpu_threads, "cpu_model": cpu_model(), "host_read_gbps": host_read_gbps()}
        if m is None and not args.no_secondary:
            m8_layers = 8
            log("cpu baseline: oracle at M=8 on %d layers" % m8_layers)
            dt8, bytes8, used8 = cpu_baseline(m8_layers, cpu_threads, 8)
            cpu["m8"] = {"value": round(bytes8 / weights_per_token / dt8, 4), "unit": "tok/s", "cores": used8,
                         "sample": "first %d layers (%.2f GB packed) at M=8 in %.2f s; the oracle decodes each "
                                   "row once per activation row" % (m8_layers, bytes8 / 1e9, dt8)}
        one_layers = max(1, cpu_layers // 8)
        dt1, bytes1, _ = cpu_baseline(one_layers, 1, m)
        cpu["one_thread"] = {"value": round(bytes1 / weights_per_token / dt1, 4), "unit": "tok/s",
                             "sample": "first %d layers in %.2f s" % (one_layers, dt1)}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "pn3t/pn4t weights, fp16 activations, fp32 accumulate",
        "data": "synthetic (seeded random codes and fp16 scales; fp16 N(0,1) activations)",
        "config": {"workload": "64-layer 27B-shaped sweep, M=%d, %s schedule%s" % (
                       m or 1, schedule, "" if m is None else ", %s arithmetic" % args.math),
                   "layers": args.layers, "gemvs_per_token": 7 * args.layers,
                   "bytes_per_token": bytes_per_token, "schedule": schedule,
                   "launches_per_token": launches},
        "tokens_per_s": round(tok_s, 2),
        "frac_of_peak": round(value / PEAK_GBPS, 4),
        "read_ceiling_gbps": round(read_ceiling, 1),
        "frac_of_read_ceiling": round(value / read_ceiling, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "other_schedules": secondary,
        "layer_schedule_read_floor": layer_floor,
        "per_config": per_config,
        "prefill": prefill,
        "smallm_m8": smallm,
        "kernel_hash": kernel_hash(kind),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
