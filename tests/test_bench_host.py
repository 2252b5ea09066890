"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the conversion of rocprofv3
counter files into HBM bytes per launch, and the shape of the oracle baseline record."""

import csv
import os
import subprocess
import sys

import numpy as np

import bench
from mla_workloads import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_counters(tmp_path):
    """A 1 MiB copy probe that reads as 512 KiB of FETCH_SIZE (factor 2) and 1,024 KiB of
    WRITE_SIZE (factor 1); decode dispatches whose counter is split over two rows (summed) and
    whose median is taken over dispatches."""
    probe = bench.COPY_PROBE_KERNEL + "<float>"
    dec = "void mla::decode_mfma_kernel<1, false>(...)"
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(1, probe, 512.0), (2, dec, 600.0), (2, dec, 400.0), (3, dec, 1100.0),
                                       (4, dec, 900.0), (5, "other", 7.0)])
    _counter_csv(write, "WRITE_SIZE", [(1, probe, 1024.0), (2, dec, 30.0), (3, dec, 50.0), (4, dec, 40.0)])
    rec = bench.traffic_from_counters("wl", str(fetch), str(write), 1)
    assert rec["read_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["read_bytes_per_launch"] == round(1000.0 * 1024 * 2)  # median of 1000, 1100, 900 KiB
    assert rec["write_bytes_per_launch"] == 40 * 1024
    assert rec["hbm_bytes_per_launch"] == rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["kernel_source_sha"] == bench._kernel_sha() and rec["copy_probe_bytes"] == 1 << 20


def test_cpu_baseline_record():
    w = gen.Workload(name="cpu_tiny", seed=5, kind="decode", batch=3, ctx_range=(20, 90), random_pages=True)
    inp = gen.make_decode_inputs(w)
    rec = bench.cpu_baseline(inp, seconds=0.0)  # stops after the first sequence
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0
    assert isinstance(rec["cores"], int) and rec["cores"] >= 1 and rec["cpu_model"]
    assert rec["sample"].startswith("first 1 of 3 sequences")
    assert f"({int(inp['lens'][0])} cached tokens" in rec["sample"]
    assert np.isfinite(rec["value"])


def _prefill_tiny():
    w = gen.Workload(name="cpu_tiny_prefill", seed=6, kind="prefill", batch=2, ctx_range=(5, 40), q_len=3,
                     random_pages=True)
    return gen.make_prefill_inputs(w)


def test_cpu_baselines_of_the_other_benches():
    """The oracle legs of the FP8, verify, unabsorbed-prefill and precomposed benches, on tiny
    workloads: each returns the record fields in its bench's own unit."""
    w = gen.Workload(name="cpu_tiny", seed=5, kind="decode", batch=3, ctx_range=(20, 90), random_pages=True)
    rec = bench.cpu_baseline_fp8(gen.make_decode_inputs(w), seconds=0.0)
    assert rec["unit"] == "GB/s" and rec["value"] > 0 and "656-byte FP8 rows" in rec["sample"]
    inp = _prefill_tiny()
    rec = bench.cpu_baseline_verify(inp, seconds=0.0)
    assert rec["unit"] == "tokens/s" and rec["value"] > 0 and rec["sample"].startswith("first 1 of 6 draft rows")
    rec = bench.cpu_baseline_prefill(inp, seconds=0.0, unabsorbed=True)
    assert rec["unit"] == "TFLOP/s" and rec["value"] > 0 and "unabsorbed attention" in rec["sample"]
    wp = gen.Workload(name="cpu_tiny_pc", seed=7, kind="precomposed", batch=4, n_heads=2, d_c=16, d_r=4, d_k=8,
                      d_v=8, d_cq=12, d_model=20)
    rec = bench.cpu_baseline_precomposed(gen.make_precomposed_inputs(wp), seconds=0.0)
    assert rec["unit"] == "ms" and rec["value"] > 0 and rec["kind"] == "oracle"
    for r in (rec,):
        assert isinstance(r["cores"], int) and r["cpu_model"]
