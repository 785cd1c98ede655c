"""Host logic of the rocprofv3 summaries (online_rotation_amd/prof.py): the
calibrated traffic record, its staleness check and the SQ counter summary,
on synthetic counter files (no GPU)."""
import csv
import os

import pytest

from online_rotation_amd import prof


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


CAL = 1 << 20
READ_K, WRITE_K = "ReduceOp<double>", "FillFunctor<double>"
KERNEL = "void rq::gemm_ra<false, 1, 4>(rq::GemmArgs, int, int)"


def _traffic_dirs(tmp_path):
    # calibration: the read kernel reports 2x its bytes in FETCH_SIZE, the
    # write kernel exactly its bytes in WRITE_SIZE; the kernel's three
    # dispatches have a median of 3000 KiB fetched and 500 KiB written
    fd, wd = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write_counters(fd, [(READ_K, "FETCH_SIZE", 2 * CAL / 1024), (KERNEL, "FETCH_SIZE", 2900),
                         (KERNEL, "FETCH_SIZE", 3000), (KERNEL, "FETCH_SIZE", 9000)])
    _write_counters(wd, [(WRITE_K, "WRITE_SIZE", CAL / 1024), (KERNEL, "WRITE_SIZE", 500),
                         (KERNEL, "WRITE_SIZE", 400), (KERNEL, "WRITE_SIZE", 600)])
    return fd, wd


def test_traffic_record_scales_by_the_calibration_and_reads_back(tmp_path, capsys):
    fd, wd = _traffic_dirs(tmp_path)
    out = str(tmp_path / "rec.txt")
    prof.main(["traffic", fd, wd, "--kernel", "gemm_ra", "--read-kernel", READ_K, "--write-kernel", WRITE_K,
               "--calib-bytes", str(CAL), "--out", out])
    capsys.readouterr()
    rec = dict(line.split(": ", 1) for line in open(out).read().splitlines() if not line.startswith("#"))
    assert float(rec["fetch_factor"]) == pytest.approx(0.5)
    assert float(rec["write_factor"]) == pytest.approx(1.0)
    assert float(rec["fetch_bytes_per_launch"]) == pytest.approx(3000 * 1024 * 0.5)
    assert float(rec["write_bytes_per_launch"]) == pytest.approx(500 * 1024)
    assert prof.read_traffic(out, "gemm_ra") == pytest.approx(3000 * 512 + 500 * 1024)
    # another kernel's name, or sources that changed since, give no figure
    assert prof.read_traffic(out, "split_quant") is None
    stale = open(out).read().replace(rec["source_sha256"].strip(), "0" * 64)
    with open(out, "w") as f:
        f.write(stale)
    assert prof.read_traffic(out, "gemm_ra") is None
    assert prof.read_traffic(str(tmp_path / "missing.txt"), "gemm_ra") is None


def test_traffic_refuses_an_ambiguous_kernel_match(tmp_path, capsys):
    fd, wd = _traffic_dirs(tmp_path)
    _write_counters(fd, [(READ_K, "FETCH_SIZE", 2048), (KERNEL, "FETCH_SIZE", 1),
                         (KERNEL.replace("1, 4", "2, 4"), "FETCH_SIZE", 1)])
    with pytest.raises(SystemExit):
        prof.main(["traffic", fd, wd, "--kernel", "gemm_ra", "--read-kernel", READ_K, "--write-kernel", WRITE_K,
                   "--calib-bytes", str(CAL)])


def test_sq_summary_derived_figures(tmp_path, capsys):
    d1, d2 = str(tmp_path / "p1"), str(tmp_path / "p2")
    _write_counters(d1, [(KERNEL, "SQ_WAVES", 1024), (KERNEL, "SQ_INSTS_VALU", 2048 * 1024),
                         (KERNEL, "SQ_VALU_MFMA_BUSY_CYCLES", 400), ("other", "SQ_WAVES", 5)])
    _write_counters(d2, [(KERNEL, "SQ_BUSY_CU_CYCLES", 250), (KERNEL, "SQ_INSTS_MFMA", 1000),
                         (KERNEL, "SQ_INSTS_LDS", 200), (KERNEL, "SQ_LDS_BANK_CONFLICT", 50)])
    out = str(tmp_path / "sq.txt")
    prof.main(["sq", d1, d2, "--kernel", "gemm_ra", "--mfma-ops", "65536", "--command", "cmd one", "--out", out])
    capsys.readouterr()
    rec = dict(line.split(": ", 1) for line in open(out).read().splitlines() if not line.startswith("#"))
    assert rec["command"] == "cmd one"
    assert float(rec["mfma_ops_per_dispatch"]) == 1000 * 65536
    assert float(rec["mfma_busy_share"]) == pytest.approx(400 / (4 * 250), abs=1e-3)
    assert float(rec["valu_insts_per_wave"]) == pytest.approx(2048)
    assert float(rec["lds_conflict_cycles_per_lds_inst"]) == pytest.approx(0.25)
    assert rec["source_sha256"] == prof.source_hash("gemm_ra")


def test_kernel_stats_sorted_by_total(tmp_path):
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "TotalDurationNs"])
        w.writeheader()
        w.writerow({"Name": "a", "Calls": 2, "AverageNs": 10.0, "TotalDurationNs": 20.0})
        w.writerow({"Name": "b", "Calls": 1, "AverageNs": 50.0, "TotalDurationNs": 50.0})
    assert [r[0] for r in prof.kernel_stats(str(d))] == ["b", "a"]


def test_every_kernel_source_exists():
    for kernel in prof.KERNEL_SOURCES:
        assert len(prof.source_hash(kernel)) == 64
