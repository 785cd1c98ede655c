"""The benchmark's one-line JSON contract: field names and types, the
roofline arithmetic, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, timeout):
    r = subprocess.run([sys.executable, "-u", BENCH] + args, cwd=ROOT, capture_output=True, text=True,
                       timeout=timeout)
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    return r.returncode, (json.loads(lines[-1]) if lines else None), r


def test_more_than_one_gpu_is_refused():
    rc, line, r = _run(["--gpus", "2"], timeout=120)
    assert rc == 2, r.stderr
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def _check_common(d, steps, warmup):
    for k, t in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                 ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                 ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)]:
        assert isinstance(d[k], t), (k, d[k])
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["scaling"] == "weak" and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert isinstance(d["config"]["workload"], str)
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=2e-3)
    assert r["traffic"] is None or r["traffic"] > 0


@pytest.mark.gpu
def test_default_line():
    rc, d, r = _run(["--steps", "3", "--warmup", "1", "--no-cpu-baseline"], timeout=600)
    assert rc == 0, r.stderr[-2000:]
    _check_common(d, 3, 1)
    assert d["unit"] == "TOPS" and d["dtype"] == "int4"
    assert d["config"]["T"] == 2048 and d["config"]["K"] == 4096 and d["config"]["N"] == 4096
    assert d["roofline"]["bound"] == "mfma" and d["roofline"]["peak"] == 5000.0
    # the step's TOPS: 2 T N K integer ops per step over the measured step time
    assert d["value"] == pytest.approx(2 * 2048 * 4096 * 4096 / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-3)
    q = d["rotate_quant"]
    assert q["bound"] == "hbm" and q["frac"] == pytest.approx(q["achieved"] / q["peak"], rel=2e-3)
    assert q["bytes_per_launch"] == 20979712


@pytest.mark.gpu
def test_kv_line():
    rc, d, r = _run(["--workload", "kv", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"], timeout=600)
    assert rc == 0, r.stderr[-2000:]
    _check_common(d, 3, 1)
    assert d["unit"] == "GB/s" and d["roofline"]["bound"] == "hbm" and d["roofline"]["peak"] == 8000.0


@pytest.mark.gpu
def test_sweep_entries():
    rc, d, r = _run(["--workload", "gsr", "--sweep", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                    timeout=600)
    assert rc == 0, r.stderr[-2000:]
    _check_common(d, 2, 1)
    sw = d["rotate_quant"]["sweep"]
    assert [e["T"] for e in sw] == [16384, 65536]
    for e in sw:
        assert e["avg_launch_us"] > 0 and 0 < e["frac"] < 1
        # bytes of the gsr quantizer per token (8192 in, 2048 codes, 4 scale) over the launch time
        assert e["achieved_GBps"] == pytest.approx(e["T"] * 10244 / e["avg_launch_us"] / 1e3, rel=2e-3)


@pytest.mark.gpu
def test_weight_prep_line():
    rc, d, r = _run(["--workload", "quik_prefill", "--weight-prep", "--steps", "1", "--warmup", "1",
                     "--no-cpu-baseline"], timeout=600)
    assert rc == 0, r.stderr[-2000:]
    _check_common(d, 1, 1)
    assert d["unit"] == "GB/s" and d["roofline"]["kernel"] == "clip_search"
    assert d["quantize"]["kernel"] == "split_quant" and d["quantize"]["avg_launch_us"] > 0
