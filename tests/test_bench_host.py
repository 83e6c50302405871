"""Host logic of bench.py (no GPU): the oracle CPU baseline on one and several threads, and the
summary of the reader's HBM counters from rocprofv3 counter CSVs."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from q8_activation_quant_amd import workloads as W  # noqa: E402


@pytest.mark.parametrize("config", [1, 4])
def test_cpu_baseline_runs_on_one_and_several_threads(config):
    wl = W.make(config, small=True)
    for threads in (1, 3):
        us, reps = bench.cpu_baseline(wl, budget_s=0.5, threads=threads)
        assert us > 0 and reps >= 1


def test_cpu_threads_and_model():
    assert 1 <= bench.cpu_threads() <= 16
    assert isinstance(bench.cpu_model(), str)


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, i, k, c, v])


def test_pmc_summary_scales_counters_by_the_copy(tmp_path):
    # two reader dispatches and the 256 MiB copy; FETCH_SIZE reports half of the copy's reads
    reader = "void (anonymous namespace)::mmvq_tiled_kernel<3, 0, 2>((anonymous namespace)::ReadArgs)"
    copy = "__amd_rocclr_copyBuffer"
    f = tmp_path / "fetch.csv"
    w = tmp_path / "write.csv"
    _csv(f, [(reader, "FETCH_SIZE", 100.0), (reader, "FETCH_SIZE", 300.0), (copy, "FETCH_SIZE", 131072.0)])
    _csv(w, [(reader, "WRITE_SIZE", 10.0), (reader, "WRITE_SIZE", 10.0), (copy, "WRITE_SIZE", 262144.0)])
    d = bench.pmc_summarize(1, None, str(f), str(w), out_dir=str(tmp_path))
    assert d["calibration"]["read_scale"] == 2.0 and d["calibration"]["write_scale"] == 1.0
    assert d["hbm_read_bytes_per_launch"] == 200 * 1024 * 2
    assert d["hbm_write_bytes_per_launch"] == 10 * 1024
    assert d["reader_dispatches"] == 2
    name = bench.pmc_file(1)
    assert json.load(open(tmp_path / (name + ".json")))["hbm_bytes_per_launch"] == 200 * 2048 + 10240
    assert (tmp_path / (name + ".md")).exists()
