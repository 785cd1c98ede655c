"""Benchmark of the rotated W4A4 linear layer on one MI355X.

One step = the whole online path on one batch: rq_rotate_quant (4096-point
Walsh-Hadamard + per-token INT4) followed by rq_w4a4_linear (INT4 GEMM,
INT32 accumulation, fp16 dequant), LLaMA-2-7B-shaped T=2048, K=N=4096.
Weights are rotated and quantized once beforehand (offline, untimed).

Inputs cycle through enough buffer sets (>512 MB) that HBM, not the 256 MB
Infinity Cache, serves them.  Steps are captured in a HIP graph and replayed
so host launch cost does not enter the timing; per-kernel durations come from
HIP events on the launch stream around graphs of back-to-back launches of one
kernel.

Prints one JSON line (see the fields below).
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
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b",
                    choices=["tiny", "llama7b", "gsr", "flat", "quik_prefill", "quik_decode"])
    ap.add_argument("--sets", type=int, default=0, help="buffer sets cycled per step (0: >640 MB)")
    ap.add_argument("--reps", type=int, default=5, help="repetitions of each per-kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def cpu_baseline(inp, wl, seconds):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    from oracle import rq_oracle as o
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    kind = wl.rot
    kw = {"block": wl.block} if kind == "gsr" else {}
    if kind == "kron":
        kw = {"p1": inp["p1"], "p2": inp["p2"], "chan_scale": inp["s"]}
    idx = inp["outlier_ch"] if wl.asym else None
    wq = o.prepare_weights(inp["w"], kind, outlier_idx=idx, **kw)   # offline side, untimed
    ts = min(256, inp["x"].shape[0])
    xs = inp["x"][:ts]
    runs = 0
    t0 = time.perf_counter()
    while True:
        xq = o.rotate_quant(xs, kind, clip=wl.clip_x, asym=wl.asym, outlier_idx=idx, **kw)
        o.linear(xq, wq)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    ops = 2.0 * ts * wl.N * wl.K * runs
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{ts} of {inp['x'].shape[0]} tokens of the {wl.name} workload (full K={wl.K}, N={wl.N}), "
                      f"rotate+quantize+INT GEMM+dequant, {runs} runs in {el:.1f} s; weight prep untimed"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import online_rotation_amd as rq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
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
    Kq = K - n_out                                       # codes per row through the INT4 path
    wq0 = rq.rq_prepare_weights(w0, rot, outlier_idx=idx)  # offline weight side
    del w0
    torch.cuda.synchronize()

    # enough buffer sets that inputs come from HBM, not the 256 MB Infinity Cache
    w_bytes = N * Kq // 2 + N * 4 + (N * 4 + N * n_out * 2 if mixed else 0)
    x_bytes = T * K * 2 + T * Kq // 2 + T * 8 + T * n_out * 2 + T * N * 2
    S = args.sets if args.sets > 0 else max(2, -(-(640 << 20) // (w_bytes + x_bytes)))
    xs = [x0.clone() for _ in range(S)]
    wqs = [{k: (v.clone() if v is not None and k != "_workspace" else v) for k, v in wq0.items()}
           for _ in range(S)]
    xq = [{"q": torch.empty((T, Kq // 2), dtype=torch.uint8, device=dev),
           "scale": torch.empty((T,), dtype=torch.float32, device=dev),
           "zero": torch.empty((T,), dtype=torch.int32, device=dev) if mixed else None,
           "x_out": torch.empty((T, n_out), dtype=torch.float16, device=dev) if mixed else None}
          for _ in range(S)]
    ys = [torch.empty((T, N), dtype=torch.float16, device=dev) for _ in range(S)]
    footprint = S * (w_bytes + x_bytes)

    def rotate(i):
        rq.rq_rotate_quant(xs[i], rot, clip=wl.clip_x, asym=mixed, outlier_idx=idx, out=xq[i])

    def gemm(i):
        if mixed:
            rq.rq_mixed_outlier_linear(xq[i]["q"], xq[i]["scale"], xq[i]["zero"], wqs[i]["q"],
                                       wqs[i]["scale"], wqs[i]["rowsum"], xq[i]["x_out"],
                                       wqs[i]["w_out"], out=ys[i])
        else:
            rq.rq_w4a4_linear(xq[i]["q"], xq[i]["scale"], wqs[i]["q"], wqs[i]["scale"], out=ys[i])

    def step(i):
        rotate(i)
        gemm(i)

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
    rq_bytes = T * K * 2 + T * (Kq // 2) + T * 4 + (T * 4 + T * n_out * 2 if mixed else 0)
    gemm_tops = ops / gemm_s / 1e12
    rq_gbs = rq_bytes / rot_s / 1e9
    gemm_bytes = w_bytes + T * Kq // 2 + T * 8 + T * n_out * 2 + T * N * 2
    decode = T <= 64                                  # weight-streaming regime
    rec = {
        "metric": METRIC,
        "value": round(ops / step_s / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: rotate({wl.rot}) + per-token INT4"
                               f"{' asymmetric + fp16 outliers' if mixed else ''} + W4A4 linear, "
                               f"X fp16 [{T},{K}], W int4 [{N},{Kq}]" + (f" + fp16 [{N},{n_out}]" if mixed else ""),
                   "T": T, "K": K, "N": N, "rotation": wl.rot, "block": wl.block, "n_out": n_out,
                   "clip_x": wl.clip_x, "buffer_sets": S, "footprint_MB": round(footprint / 2**20)},
        "roofline": ({"bound": "hbm", "kernel": "gemm_w4a4", "achieved": round(gemm_bytes / gemm_s / 1e9, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gemm_bytes / gemm_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                      "bytes_per_launch": gemm_bytes, "avg_launch_us": round(gemm_s * 1e6, 3)}
                     if decode else
                     {"bound": "mfma", "kernel": "gemm_w4a4", "achieved": round(gemm_tops, 1),
                      "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                      "frac": round(gemm_tops / INT8_PEAK_TOPS, 4), "traffic": None,
                      "avg_launch_us": round(gemm_s * 1e6, 3)}),
        "rotate_quant": {"bound": "hbm", "kernel": {"hadamard": "fwht4096_mfma", "gsr": "fwht4096_mfma",
                                                   "kron": "kron_quant", "none": "rowlds_quant"}[wl.rot],
                         "achieved": round(rq_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(rq_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": rq_bytes,
                         "avg_launch_us": round(rot_s * 1e6, 3)},
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
