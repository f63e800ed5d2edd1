"""CPU tests of the benchmark's host logic: the one-GPU contract, the split of the timed steps
into trials, the byte counts the GB/s figures divide by, the digest that keys the stored HBM
counters, and the counter ingestion's arithmetic on a synthetic rocprofv3 counter file."""
import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
import bench  # noqa: E402

VERIFY = "void vg::vg_mfma_h<1, 1, 1, false, true, true, true, false>(vg::MfmaArgs)"


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("steps", [1, 7, 20, 200, 201])
@pytest.mark.parametrize("trials", [1, 7, 50])
def test_trials_partition_the_timed_steps(steps, trials):
    sizes = bench.trial_sizes(steps, trials)
    assert sum(sizes) == steps
    assert len(sizes) == min(trials, steps)
    assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1


@pytest.mark.parametrize("name", ["mlp_up_affine2_k5120_n17408", "mlp_up_sign1_k5120_n17408",
                                  "mlp_up_affine1_k5120_n17408"])
def test_packed_bytes_count_codes_scales_and_biases(name):
    fmt, K, N, _, _ = bench.WORKLOADS[name]
    case = bench.workload_case(name, seed=0, N=16)   # a 16-row slice: the count is per row
    per_row = {"affine2": K // 4 + 2 * 2 * K // 64, "sign1": K // 8 + 2 * K // 128,
               "affine1": K // 8 + 2 * 2 * K // 128}[fmt]
    assert bench.packed_bytes(case) == 16 * per_row
    if name == "mlp_up_affine2_k5120_n17408":
        assert N * per_row == 27852800   # the figure the bench line's GB/s divide by


def _copy_sources(dst):
    for p in bench.KERNEL_SOURCES:
        os.makedirs(os.path.dirname(os.path.join(dst, p)), exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), os.path.join(dst, p))


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    _copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_source_digest()
    src = os.path.join(str(tmp_path), bench.KERNEL_SOURCES[0])
    with open(src, "a") as f:
        f.write("\n// a comment line\n/* a block\n   comment */\n")
    assert bench.kernel_source_digest() == d0
    with open(src, "a") as f:
        f.write("\nint vg_digest_probe;\n")
    assert bench.kernel_source_digest() != d0


def _counter_file(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_ingest_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    t = str(tmp_path)
    fill = "void at::native::vectorized_elementwise_kernel<4>(int)"
    stream = "void vg::vg_stream_read_kernel<4>(unsigned int __vector(4) const*, unsigned long, unsigned int*)"
    _counter_file(f"{t}/f", [(fill, "FETCH_SIZE", 10.5), (VERIFY, "FETCH_SIZE", 14000.0),
                             (VERIFY, "FETCH_SIZE", 14100.0), (stream, "FETCH_SIZE", 99999.0)])
    _counter_file(f"{t}/w", [(VERIFY, "WRITE_SIZE", 576.0), (VERIFY, "WRITE_SIZE", 576.0)])
    # a 256 MiB copy that the counters read as 131072 KiB fetched (factor 2) and 262144 KiB
    # written (factor 1)
    _counter_file(f"{t}/cf", [("copyBuffer", "FETCH_SIZE", 131072.0)])
    _counter_file(f"{t}/cw", [("copyBuffer", "WRITE_SIZE", 262144.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", f"{t}/traffic.json")
    assert bench.ingest_counters(f"{t}/f", f"{t}/w", f"{t}/cf", f"{t}/cw", "wl", 8) == 0
    ent = json.load(open(f"{t}/traffic.json"))["kernels"]["vg_mfma_h/wl/M8"]
    assert ent["fetch_bytes"] == round(14050.0 * 1024 * 2.0)
    assert ent["write_bytes"] == 576 * 1024
    assert ent["hbm_bytes_per_launch"] == ent["fetch_bytes"] + ent["write_bytes"]
    assert ent["dispatches"] == [2, 2]
    digest = bench.kernel_source_digest()
    assert ent["source_digest"] == digest
    assert bench.load_traffic("vg_mfma_h/wl/M8", digest) == ent["hbm_bytes_per_launch"]
    assert bench.load_traffic("vg_mfma_h/wl/M8", "0" * 16) is None   # stale once the code changes


def test_ingest_refuses_a_run_with_two_verify_kernels(tmp_path, monkeypatch):
    t = str(tmp_path)
    other = VERIFY.replace("vg_mfma_h<1, 1, 1, false, true, true, true, false>", "vg_mfma_q<1, 1, 1, false, true, true, false, false>")
    _counter_file(f"{t}/f", [(VERIFY, "FETCH_SIZE", 1.0), (other, "FETCH_SIZE", 1.0)])
    for d in ("w", "cf", "cw"):
        _counter_file(f"{t}/{d}", [])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", f"{t}/traffic.json")
    assert bench.ingest_counters(f"{t}/f", f"{t}/w", f"{t}/cf", f"{t}/cw", "wl", 8) == 1
    assert not os.path.exists(f"{t}/traffic.json")
