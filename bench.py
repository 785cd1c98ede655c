"""Benchmark of the rotated W4A4 linear layer on one MI355X.

One step = the whole online path on one batch of one workload:
rq_rotate_quant (the workload's online transform + per-token INT4) followed
by the INT4 GEMM with its dequantization epilogue (rq_w4a4_linear, or
rq_mixed_outlier_linear with FP16 outlier columns).  Weights are rotated and
quantized once beforehand (offline, untimed).  The default workload is the
LLaMA-2-7B-shaped projection: T=2048, K=N=4096, 4096-point Walsh-Hadamard.

Inputs cycle through enough buffer sets (>640 MB) that HBM, not the 256 MB
Infinity Cache, serves them.  The K timed steps are one HIP graph replay,
bracketed by events on the stream the kernels run on; per-kernel durations
come from events around graphs of back-to-back launches of one call.

Prints one JSON line.  `roofline` is the dominant kernel (the GEMM) against
its bound: INT8 MFMA dense peak, or HBM at decode sizes (T <= 32);
`roofline.traffic` comes from the rocprofv3 counter record under profiles/
when one exists for this kernel, workload and kernel source, else null.
`--counters` instead launches calibration kernels of known traffic and the
two calls a few times, for `rocprofv3 --pmc FETCH_SIZE` / `WRITE_SIZE` runs.

`--workload quik8_down` runs the same step at 8 bits (QUIK-8B's form for
the LLaMA-2-70B down projection: T=4096, K=28672, N=8192, 896 fp16 outlier
columns; rq_w8a8_linear on INT8 matrix cores); `--workload quik8_decode` is
that layer at decode (T=8), reported in GB/s against HBM.

`--weight-prep` (with quik_prefill, quik_decode or quik8_down) times QUIK's
offline weight side instead: rq_search_weight_clip (the per-channel clip
ratio by linear search over 100 ratios) and rq_prepare_weights with those
ratios; the roofline is the search kernel's fp64 error arithmetic.

`--sweep` adds the quantizer alone at 16K and 64K tokens (the batch's rows
repeated) to the line, under rotate_quant.sweep; it is off by default so
that a kernel trace of the default run holds one launch shape per kernel.

`--workload kv` measures the KV-cache quantizer instead: one step quantizes
one attention layer's keys (R3, a 128-point Walsh-Hadamard per head) and
values, group-wise asymmetric INT4 with groups of 128 channels, in one
rq_kv_cache_quant launch; the line reports GB/s with that launch as the
roofline kernel, and the two single-tensor launches timed beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 rotated-linear TOPS (T=2048,K=N=4096) + rotate-quant GB/s, % roofline"
METRIC8 = "W8A8 QUIK-8B down-projection TOPS + INT8 quantizer GB/s, % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA
FP64_PEAK_TFLOPS = 78.6        # MI355X dense FP64 MFMA
CALIB_BYTES = 512 << 20        # calibration fill / sum for the counter runs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b",
                    choices=["tiny", "llama7b", "gsr", "flat", "quik_prefill", "quik_decode", "quik8_down",
                             "quik8_decode", "kv"])
    ap.add_argument("--sets", type=int, default=0, help="buffer sets cycled per step (0: >640 MB)")
    ap.add_argument("--reps", type=int, default=5, help="repetitions of each per-kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the quantizer alone at 16K and 64K tokens (rotate_quant.sweep)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--weight-prep", action="store_true",
                    help="time QUIK's offline weight side instead: clip linear search + per-channel quantization")
    ap.add_argument("--fused-decode", action="store_true",
                    help="also time decode batches (T = 1 .. 16 of the workload's rows) as the quantizer + linear "
                         "calls and as the one fused call (rotate_quant_decode)")
    ap.add_argument("--counters", action="store_true",
                    help="launch the calibration kernels and each call a few times, print one line")
    return ap.parse_args()


def gemm_kernel(T, Kb, n_out=0, bits=4):
    """The GEMM kernel the library dispatches to (launch_gemm's rules)."""
    if bits == 8:
        return "gemm_decode8" if T <= 32 else "gemm_ra"
    if Kb % 64 == 0 and T <= 16 and T * (Kb // 16 + n_out // 8) <= 4096:
        return "gemm_decode16"
    if Kb % 64 == 0 and T <= 32:
        return "gemm_decode"
    if Kb % 64 == 0 and T >= 256:
        return "gemm_ra"
    return "gemm_w4a4"


def quant_kernel(wl, T):
    """The quantizer kernel the library dispatches to (run_quant's rules)."""
    if wl.bits == 8:
        return "split_quant8"
    if wl.rot in ("hadamard", "gsr") and wl.K == 4096:
        return "fwht4096_mfma"
    if wl.rot == "kron":
        return "kron64_mfma" if wl.K == 4096 else "kron_quant"
    return "split_quant" if wl.rot == "none" else "rowlds_quant"


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def oracle_leg(fn, seconds, per_run, unit, sample):
    """Times fn (one oracle run over the sample) twice: with every BLAS thread,
    then limited to one thread; each leg repeats fn for about `seconds`.
    `value` is the all-threads rate (per_run units per run, divided by 1e9 or
    1e12 for GB/s or TOPS); `cores` is the BLAS thread count of that leg."""
    from threadpoolctl import threadpool_info, threadpool_limits
    scale = 1e12 if unit == "TOPS" else 1e9

    def leg():
        runs = 0
        t0 = time.perf_counter()
        while True:
            fn()
            runs += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return runs, el

    cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    runs, el = leg()
    with threadpool_limits(limits=1):
        runs1, el1 = leg()
    return {"value": per_run * runs / el / scale, "unit": unit, "cores": int(cores), "kind": "oracle",
            "value_1core": per_run * runs1 / el1 / scale, "nproc": len(os.sched_getaffinity(0)),
            "cpu_model": _cpu_model(),
            "sample": f"{sample}; {runs} runs in {el:.1f} s on {cores} threads, {runs1} runs in {el1:.1f} s on 1"}


def cpu_baseline(inp, wl, seconds):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    from oracle import rq_oracle as o
    kind = wl.rot
    kw = {"block": wl.block} if kind == "gsr" else {}
    if kind == "kron":
        kw = {"p1": inp["p1"], "p2": inp["p2"], "chan_scale": inp["s"]}
    idx = inp["outlier_ch"] if wl.asym else None
    wq = o.prepare_weights(inp["w"], kind, outlier_idx=idx, bits=wl.bits, **kw)   # offline side, untimed
    ts = min(256, inp["x"].shape[0])
    xs = inp["x"][:ts]

    def run():
        xq = o.rotate_quant(xs, kind, clip=wl.clip_x, asym=wl.asym, outlier_idx=idx, bits=wl.bits, **kw)
        o.linear(xq, wq)

    return oracle_leg(run, seconds, 2.0 * ts * wl.N * wl.K, "TOPS",
                      f"{ts} of {inp['x'].shape[0]} tokens of the {wl.name} workload (full K={wl.K}, N={wl.N}), "
                      f"rotate+quantize+INT GEMM+dequant; weight prep untimed")


KV_METRIC = "KV-cache quantizer GB/s (R3 on keys + group-wise asymmetric INT4 of keys and values), % HBM roofline"


def kv_bytes(T, K, g):
    """Algorithmic HBM bytes of one KV quantizer launch: fp16 in, packed codes,
    fp32 scale and int32 zero point per group out."""
    return T * K * 2 + T * K // 2 + T * (K // g) * 8


def cpu_baseline_kv(inp, wl, seconds):
    """The oracle on a bounded sample of the kv workload's tokens."""
    from oracle import rq_oracle as o
    ts = min(256, inp["x"].shape[0])
    xs, vs = inp["x"][:ts], inp["v"][:ts]

    def run():
        o.kv_rotate_quant(xs, group=wl.block, rotate=True)
        o.kv_rotate_quant(vs, group=wl.block, rotate=False)

    return oracle_leg(run, seconds, 2 * kv_bytes(ts, wl.K, wl.block), "GB/s",
                      f"{ts} of {inp['x'].shape[0]} tokens of the kv workload (keys with R3, values without, "
                      f"{wl.K} channels, g={wl.block})")


def main_kv(args, torch, rq, prof, workloads):
    """One step = the KV-cache quantization of one attention layer over the
    batch: keys rotated by R3 (per-head Walsh-Hadamard) and values, each
    quantized group-wise asymmetric INT4, in one rq_kv_cache_quant launch.
    The two single-tensor rq_kv_rotate_quant launches are timed beside it."""
    dev = torch.device("cuda:0")
    wl = workloads.get("kv")
    inp = workloads.make_inputs("kv", with_weights=False)
    T, K, g = wl.T, wl.K, wl.block
    per = kv_bytes(T, K, g)
    S = args.sets if args.sets > 0 else max(2, -(-(640 << 20) // (2 * per)))
    ks = [torch.from_numpy(inp["x"]).to(dev) for _ in range(S)]
    vs = [torch.from_numpy(inp["v"]).to(dev) for _ in range(S)]

    def bufs():
        return (torch.empty((T, K // 2), dtype=torch.uint8, device=dev),
                torch.empty((T, K // g), dtype=torch.float32, device=dev),
                torch.empty((T, K // g), dtype=torch.int32, device=dev))
    kq = [bufs() for _ in range(S)]
    vq = [bufs() for _ in range(S)]

    def keys(i):
        rq.rq_kv_rotate_quant(ks[i], group=g, rotate=True, out=kq[i])

    def values(i):
        rq.rq_kv_rotate_quant(vs[i], group=g, rotate=False, out=vq[i])

    def step(i):
        rq.rq_kv_cache_quant(ks[i], vs[i], group=g, rotate_k=True, rotate_v=False, out_k=kq[i], out_v=vq[i])

    kernel = f"group_quant_pair<{g // 4}, true, false>"
    if args.counters:
        calib = torch.empty(CALIB_BYTES // 8, dtype=torch.float64, device=dev)
        for _ in range(3):
            calib.fill_(1.0)
        for _ in range(3):
            calib.sum()
        sc = min(S, 16)
        for i in range(4 * sc):
            step(i % sc)
        torch.cuda.synchronize()
        print(json.dumps({"counters": "done", "workload": wl.name, "calib_bytes": CALIB_BYTES,
                          "quant_kernel": kernel}), flush=True)
        return

    for i in range(max(args.warmup, S)):
        step(i % S)
    torch.cuda.synchronize()
    eager = [t.clone() for t in kq[0] + vq[0]]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def capture(fn, count):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gr, stream=stream):
                for j in range(count):
                    fn(j % S)
        torch.cuda.synchronize()
        return gr

    for i in range(S):   # the single-tensor launches give the same outputs
        keys(i)
        values(i)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(kq[0] + vq[0], eager)), "single launches differ from the pair"
    g_step = capture(step, args.steps)
    reps_per_graph = max(S, 32)
    g_pair = capture(step, reps_per_graph)
    g_keys = capture(keys, reps_per_graph)
    g_vals = capture(values, reps_per_graph)
    for _ in range(2):   # graph replays reproduce the eager result
        for t in kq[0] + vq[0]:
            t.zero_()
        torch.cuda.synchronize()
        g_step.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(kq[0] + vq[0], eager)), "graph replay differs from eager"

    def timed(gr, launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        out = []
        gr.replay()
        torch.cuda.synchronize()
        for _ in range(args.reps):
            with torch.cuda.stream(stream):
                e0.record(stream)
                gr.replay()
                e1.record(stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1) / 1e3 / launches)
        return float(np.median(out))

    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g_step.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    step_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    pair_s = timed(g_pair, reps_per_graph)
    key_s = timed(g_keys, reps_per_graph)
    val_s = timed(g_vals, reps_per_graph)
    gbs = 2 * per / pair_s / 1e9
    traffic = prof.read_traffic(os.path.join(ROOT, "profiles", f"group_quant_pair_{wl.name}_traffic.txt"),
                                "group_quant_pair")
    rec = {
        "metric": KV_METRIC,
        "value": round(2 * per / step_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"kv: keys fp16 [{T},{K}] -> R3 ({g}-point Walsh-Hadamard per head) + "
                               f"group-wise asymmetric INT4 (g={g}); values fp16 [{T},{K}] -> group-wise INT4",
                   "T": T, "K": K, "group": g, "buffer_sets": S, "footprint_MB": round(S * 2 * per / 2**20)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                     "algorithmic_bytes_per_launch": 2 * per, "avg_launch_us": round(pair_s * 1e6, 3)},
        "single_launches": {
            "keys": {"kernel": f"group_quant<{g // 4}, true>", "avg_launch_us": round(key_s * 1e6, 3),
                     "achieved": round(per / key_s / 1e9, 1), "unit": "GB/s",
                     "frac": round(per / key_s / 1e9 / HBM_PEAK_GBS, 4)},
            "values": {"kernel": f"group_quant<{g // 4}, false>", "avg_launch_us": round(val_s * 1e6, 3),
                       "achieved": round(per / val_s / 1e9, 1), "unit": "GB/s",
                       "frac": round(per / val_s / 1e9 / HBM_PEAK_GBS, 4)}},
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_kv(inp, wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


FP64_VECTOR_PEAK_TFLOPS = 78.6  # MI355X fp64 vector: 256 CUs x 128 flops/clock (64 FMA) x 2.4 GHz


def main_weight_prep(args, torch, rq, prof, workloads):
    """QUIK's weight side on the GPU (unrotated workloads): the per-channel
    clip ratio by linear search over 100 ratios, then per-channel symmetric
    quantization of the normal columns with those ratios and the outlier
    split.  One step = both calls on the workload's W."""
    from oracle import rq_oracle as o
    dev = torch.device("cuda:0")
    wl = workloads.get(args.workload)
    assert wl.rot == "none", "weight-prep timing is for the unrotated (QUIK) workloads"
    inp = workloads.make_inputs(args.workload)
    N, K, n_out, bits, steps = wl.N, wl.K, wl.n_out, wl.bits, 100
    w = torch.from_numpy(inp["w"]).to(dev)
    idx = torch.from_numpy(inp["outlier_ch"][:n_out].astype(np.int32)).to(dev) if n_out else None
    clip = torch.empty((N,), dtype=torch.float32, device=dev)
    wq = {}

    def search():
        rq.rq_search_weight_clip(w, outlier_idx=idx, bits=bits, steps=steps, out=clip)

    def quant():
        wq.update(rq.rq_prepare_weights(w, rq.Rotation("none"), outlier_idx=idx, bits=bits, row_clip=clip))

    for _ in range(max(1, args.warmup // 10)):
        search()
        quant()
    torch.cuda.synchronize()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    reps = max(1, min(args.steps, 10))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        search()
        quant()
    e1.record()
    e1.synchronize()
    step_s = e0.elapsed_time(e1) / 1e3 / reps
    search_s = timed(search, reps)
    quant_s = timed(quant, reps)
    kint = K - n_out
    flops = 4.0 * N * kint * steps      # per value and ratio: d = w - s q, d * d + acc, in fp64
    w_bytes = N * K * 2
    rec = {
        "metric": "QUIK weight prep GB/s of fp16 weights (clip linear search over 100 ratios + per-channel quantization)",
        "value": round(w_bytes / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": max(1, args.warmup // 10),
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} weights: W fp16 [{N},{K}], {n_out} fp16 outlier columns, "
                               f"INT{bits} per channel, {steps} clip ratios", "N": N, "K": K, "n_out": n_out,
                   "bits": bits, "ratios": steps},
        "roofline": {"bound": "alu", "achieved": round(flops / search_s / 1e12, 2),
                     "peak": FP64_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / search_s / 1e12 / FP64_VECTOR_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "clip_search", "flops_per_launch": flops, "avg_launch_us": round(search_s * 1e6, 1),
                     "note": "fp64 vector ALU arithmetic: 4 fp64 flops per value and ratio (the error term), the "
                             "exact fp32 codes beside them not counted; peak = 256 CUs x 128 fp64 flops per clock "
                             "x 2.4 GHz"},
        "quantize": {"kernel": "split_quant8" if bits == 8 else "split_quant", "avg_launch_us": round(quant_s * 1e6, 1),
                     "achieved_GBps": round((w_bytes + N * (kint if bits == 8 else kint // 2)) / quant_s / 1e9, 1)},
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        rows = 64
        oidx = inp["outlier_ch"][:n_out] if n_out else None
        rec["cpu_baseline"] = oracle_leg(
            lambda: o.search_weight_clip(inp["w"][:rows], outlier_idx=oidx, bits=bits, steps=steps),
            args.cpu_seconds, rows * K * 2, "GB/s", f"{rows} of {N} weight rows, clip search only")
    print(json.dumps(rec), flush=True)


def quant_sweep(torch, rq, x0, rot, wl, idx, bits, Kqb, n_out, reps, stream):
    """The workload's quantizer alone at larger token counts (16K and 64K
    tokens: rows of the batch repeated, so the distribution is the same):
    per-launch time from a graph of back-to-back launches over buffer sets
    totalling more than 640 MB, median of `reps` replays."""
    dev = x0.device
    T0, K = x0.shape
    mixed = wl.asym
    out = []
    for T in (16384, 65536):
        if T <= T0 or T % T0:
            continue
        per = T * K * 2 + T * Kqb + T * 8 + T * n_out * 2
        S = max(2, -(-(640 << 20) // per))
        xs = [x0.repeat(T // T0, 1) for _ in range(S)]
        qs = [{"q": torch.empty((T, Kqb), dtype=torch.uint8, device=dev),
               "scale": torch.empty((T,), dtype=torch.float32, device=dev),
               "zero": torch.empty((T,), dtype=torch.int32, device=dev) if mixed else None,
               "x_out": torch.empty((T, n_out), dtype=torch.float16, device=dev) if mixed else None}
              for _ in range(S)]

        def call(i):
            rq.rq_rotate_quant(xs[i], rot, clip=wl.clip_x, asym=mixed, outlier_idx=idx, out=qs[i], bits=bits)

        for i in range(S):
            call(i)
        torch.cuda.synchronize()
        n = max(S, 8)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for j in range(n):
                    call(j % S)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(reps):
            with torch.cuda.stream(stream):
                ev0.record(stream)
                g.replay()
                ev1.record(stream)
            ev1.synchronize()
            times.append(ev0.elapsed_time(ev1) / 1e3 / n)
        sec = float(np.median(times))
        nbytes = T * K * 2 + T * Kqb + T * 4 + (T * 4 + T * n_out * 2 if mixed else 0)
        out.append({"T": T, "kernel": quant_kernel(wl, T), "avg_launch_us": round(sec * 1e6, 2),
                    "achieved_GBps": round(nbytes / sec / 1e9, 1),
                    "frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4), "buffer_sets": S})
        del g, xs, qs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def fused_decode_sweep(torch, rq, x0, w_q, rot, wl, idx, reps, stream):
    """Decode batches of the workload (its first T rows, T = 1, 2, 4, 8, 16)
    through the two calls (rq_rotate_quant, then rq_w4a4_linear or
    rq_mixed_outlier_linear) and through the one fused call
    (rq_rotate_quant_decode_linear); per-step time of graphs of back-to-back
    steps over weight copies totalling more than 640 MB, median of `reps`."""
    dev = x0.device
    mixed = wl.asym
    N = w_q["q"].shape[0]
    wbytes = sum(v.numel() * v.element_size() for k, v in w_q.items() if v is not None and k != "_workspace")
    S = max(2, -(-(640 << 20) // wbytes))
    ws = [{k: (v.clone() if v is not None and k != "_workspace" else v) for k, v in w_q.items()} for _ in range(S)]
    out = []
    for T in (1, 2, 4, 8, 16):
        if T > x0.shape[0]:  # a workload with fewer rows (the T = 8 decode batch) stops there
            break
        xs = [x0[:T].clone() for _ in range(S)]
        ys = [torch.empty((T, N), dtype=torch.float16, device=dev) for _ in range(S)]
        K = x0.shape[1]
        n_out = wl.n_out if mixed else 0
        xq = [{"q": torch.empty((T, (K - n_out) // 2), dtype=torch.uint8, device=dev),
               "scale": torch.empty((T,), dtype=torch.float32, device=dev),
               "zero": torch.empty((T,), dtype=torch.int32, device=dev) if mixed else None,
               "x_out": torch.empty((T, n_out), dtype=torch.float16, device=dev) if mixed else None}
              for _ in range(S)]

        def two(i):
            rq.rq_rotate_quant(xs[i], rot, clip=wl.clip_x, asym=mixed, outlier_idx=idx, out=xq[i])
            if mixed:
                rq.rq_mixed_outlier_linear(xq[i]["q"], xq[i]["scale"], xq[i]["zero"], ws[i]["q"], ws[i]["scale"],
                                           ws[i]["rowsum"], xq[i]["x_out"], ws[i]["w_out"], out=ys[i])
            else:
                rq.rq_w4a4_linear(xq[i]["q"], xq[i]["scale"], ws[i]["q"], ws[i]["scale"], out=ys[i])

        def fused(i):
            rq.rq_rotate_quant_decode_linear(xs[i], rot, ws[i]["q"], ws[i]["scale"],
                                             ws[i]["rowsum"] if mixed else None, ws[i]["w_out"], asym=mixed,
                                             clip=wl.clip_x, outlier_idx=idx, out=ys[i])

        row = {"T": T}
        for name, fn in (("two_calls_us", two), ("fused_us", fused)):
            for i in range(S):
                fn(i)
            torch.cuda.synchronize()
            n = max(S, 32)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for j in range(n):
                        fn(j % S)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            times = []
            for _ in range(reps):
                with torch.cuda.stream(stream):
                    ev0.record(stream)
                    g.replay()
                    ev1.record(stream)
                ev1.synchronize()
                times.append(ev0.elapsed_time(ev1) / 1e3 / n)
            row[name] = round(float(np.median(times)) * 1e6, 2)
            del g
        two(0)
        torch.cuda.synchronize()
        y_two = ys[0].clone()
        fused(0)
        torch.cuda.synchronize()
        row["equal"] = bool(torch.equal(y_two, ys[0]))
        row["fused_wins"] = row["fused_us"] < row["two_calls_us"]
        out.append(row)
        del xs, ys, xq
    del ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import online_rotation_amd as rq
    from online_rotation_amd import prof
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "kv":
        return main_kv(args, torch, rq, prof, workloads)
    if args.weight_prep:
        return main_weight_prep(args, torch, rq, prof, workloads)
    dev = torch.device("cuda:0")
    wl = workloads.get(args.workload)
    inp = workloads.make_inputs(args.workload)
    T, K, N = wl.T, wl.K, wl.N
    if wl.rot == "kron":
        rot = rq.Rotation("kron", p1=torch.from_numpy(inp["p1"]).to(dev),
                          p2=torch.from_numpy(inp["p2"]).to(dev),
                          chan_scale=torch.from_numpy(inp["s"]).to(dev))
    else:
        rot = rq.Rotation(wl.rot, block=wl.block)

    x0 = torch.from_numpy(inp["x"]).to(dev)
    w0 = torch.from_numpy(inp["w"]).to(dev)
    T = x0.shape[0]
    mixed = wl.asym
    idx = torch.from_numpy(inp["outlier_ch"]).to(dev) if mixed else None
    n_out = wl.n_out if mixed else 0
    Kq = K - n_out                                       # codes per row through the integer path
    bits = wl.bits
    Kqb = Kq if bits == 8 else Kq // 2                   # code bytes per row
    wq0 = rq.rq_prepare_weights(w0, rot, outlier_idx=idx, bits=bits)  # offline weight side
    del w0
    torch.cuda.synchronize()

    # enough buffer sets that inputs come from HBM, not the 256 MB Infinity Cache
    w_bytes = N * Kqb + N * 4 + (N * 4 + N * n_out * 2 if mixed else 0)
    x_bytes = T * K * 2 + T * Kqb + T * 8 + T * n_out * 2 + T * N * 2
    # (at most 512 sets: the tiny workload is latency-bound and would need thousands)
    S = args.sets if args.sets > 0 else min(512, max(2, -(-(640 << 20) // (w_bytes + x_bytes))))
    xs = [x0.clone() for _ in range(S)]
    wqs = [{k: (v.clone() if v is not None and k != "_workspace" else v) for k, v in wq0.items()}
           for _ in range(S)]
    xq = [{"q": torch.empty((T, Kqb), dtype=torch.uint8, device=dev),
           "scale": torch.empty((T,), dtype=torch.float32, device=dev),
           "zero": torch.empty((T,), dtype=torch.int32, device=dev) if mixed else None,
           "x_out": torch.empty((T, n_out), dtype=torch.float16, device=dev) if mixed else None}
          for _ in range(S)]
    ys = [torch.empty((T, N), dtype=torch.float16, device=dev) for _ in range(S)]
    footprint = S * (w_bytes + x_bytes)

    def rotate(i):
        rq.rq_rotate_quant(xs[i], rot, clip=wl.clip_x, asym=mixed, outlier_idx=idx, out=xq[i], bits=bits)

    def gemm(i):
        if bits == 8:
            rq.rq_w8a8_linear(xq[i]["q"], xq[i]["scale"], xq[i]["zero"], wqs[i]["q"], wqs[i]["scale"],
                              wqs[i]["rowsum"], xq[i]["x_out"], wqs[i]["w_out"], out=ys[i])
        elif mixed:
            rq.rq_mixed_outlier_linear(xq[i]["q"], xq[i]["scale"], xq[i]["zero"], wqs[i]["q"],
                                       wqs[i]["scale"], wqs[i]["rowsum"], xq[i]["x_out"],
                                       wqs[i]["w_out"], out=ys[i])
        else:
            rq.rq_w4a4_linear(xq[i]["q"], xq[i]["scale"], wqs[i]["q"], wqs[i]["scale"], out=ys[i])

    def step(i):
        rotate(i)
        gemm(i)

    if args.counters:
        # calibration: a float64 fill writes CALIB_BYTES, a float64 sum reads
        # them (the only float64 kernels in the run); then four passes over
        # the buffer sets, so that the median launch is a steady-state one
        calib = torch.empty(CALIB_BYTES // 8, dtype=torch.float64, device=dev)
        for _ in range(3):
            calib.fill_(1.0)
        for _ in range(3):
            calib.sum()
        sc = min(S, 16)
        for i in range(4 * sc):
            step(i % sc)
        torch.cuda.synchronize()
        print(json.dumps({"counters": "done", "workload": wl.name, "calib_bytes": CALIB_BYTES,
                          "gemm_kernel": gemm_kernel(T, Kqb, n_out, bits), "quant_kernel": quant_kernel(wl, T)}),
              flush=True)
        return

    # eager warmup (also the reference for the graph-replay check)
    for i in range(max(args.warmup, S)):
        step(i % S)
    torch.cuda.synchronize()
    y_eager = ys[0].clone()

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())

    def capture(fn, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for j in range(count):
                    fn(j % S)
        torch.cuda.synchronize()
        return g

    g_step = capture(step, args.steps)
    reps_per_graph = max(S, 32)
    g_rot = capture(rotate, reps_per_graph)
    g_gemm = capture(gemm, reps_per_graph)

    # graph replays reproduce the eager result (checked on every replay)
    for _ in range(2):
        ys[0].zero_()
        torch.cuda.synchronize()
        g_step.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys[0], y_eager), "graph replay differs from eager execution"

    def timed(g, launches, reps):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        out = []
        g.replay()
        torch.cuda.synchronize()
        for _ in range(reps):
            with torch.cuda.stream(stream):
                ev0.record(stream)
                g.replay()
                ev1.record(stream)
            ev1.synchronize()
            out.append(ev0.elapsed_time(ev1) / 1e3 / launches)
        return float(np.median(out))

    # the timed region: exactly args.steps steps
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g_step.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    step_s = ev0.elapsed_time(ev1) / 1e3 / args.steps

    rot_s = timed(g_rot, reps_per_graph, args.reps)
    gemm_s = timed(g_gemm, reps_per_graph, args.reps)

    ops = 2.0 * T * N * Kq + 2.0 * T * N * n_out      # INT4 part + fp16 outlier part
    rq_bytes = T * K * 2 + T * Kqb + T * 4 + (T * 4 + T * n_out * 2 if mixed else 0)
    gemm_tops = ops / gemm_s / 1e12
    rq_gbs = rq_bytes / rot_s / 1e9
    gemm_bytes = w_bytes + T * Kqb + T * 8 + T * n_out * 2 + T * N * 2
    gk, qk = gemm_kernel(T, Kqb, n_out, bits), quant_kernel(wl, T)
    decode = gk.startswith("gemm_decode")
    traffic = prof.read_traffic(os.path.join(ROOT, "profiles", f"{gk}_{wl.name}_traffic.txt"), gk)
    if decode:
        roof = {"bound": "hbm", "achieved": round(gemm_bytes / gemm_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gemm_bytes / gemm_s / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": gk, "algorithmic_bytes_per_launch": gemm_bytes}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4), "traffic": traffic,
                "kernel": gk, "ops_per_launch": ops, "note": "integer ops against the INT8 MFMA peak"}
    roof["avg_launch_us"] = round(gemm_s * 1e6, 3)
    quant = {"kernel": qk, "bound": "hbm", "achieved": round(rq_gbs, 1), "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(rq_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": rq_bytes,
             "avg_launch_us": round(rot_s * 1e6, 3)}
    if qk == "kron64_mfma":   # the FP64 transform: 2 x 64^3 multiply-adds per token
        fl = 2.0 * 2 * 64 ** 3 * T
        quant["fp64_tflops"] = round(fl / rot_s / 1e12, 2)
        quant["fp64_frac"] = round(fl / rot_s / 1e12 / FP64_PEAK_TFLOPS, 4)
    rec = {
        "metric": METRIC8 if bits == 8 else METRIC,
        "value": round(ops / step_s / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if bits == 8 else "int4",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: rotate({wl.rot}) + per-token INT{bits}"
                               f"{' asymmetric + fp16 outliers' if mixed else ''} + W{bits}A{bits} linear, "
                               f"X fp16 [{T},{K}], W int{bits} [{N},{Kq}]" + (f" + fp16 [{N},{n_out}]" if mixed else ""),
                   "T": T, "K": K, "N": N, "rotation": wl.rot, "block": wl.block, "n_out": n_out,
                   "clip_x": wl.clip_x, "buffer_sets": S, "footprint_MB": round(footprint / 2**20)},
        "roofline": roof,
        "rotate_quant": quant,
        "gpu": torch.cuda.get_device_name(0),
    }
    if args.fused_decode and bits == 4 and (wl.rot == "none" or (wl.rot in ("hadamard", "gsr") and K == 4096)):
        rec["fused_decode"] = fused_decode_sweep(torch, rq, x0, wq0, rot, wl, idx, args.reps, stream)
    if args.sweep and T >= 2048:
        del xs, wqs, xq, ys, g_step, g_rot, g_gemm
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        rec["rotate_quant"]["sweep"] = quant_sweep(torch, rq, x0, rot, wl, idx, bits, Kqb, n_out, args.reps, stream)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
