"""Host logic of bench.py, on the CPU: the algorithmic bytes U behind
roofline.achieved, the counter calibration behind roofline.traffic, and the
one-GPU rule."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


@pytest.fixture(scope="module")
def kk():
    import compressed_decode_attention_kk_amd as kk
    kk.lib()
    return kk


def test_algorithmic_bytes_of_the_uniform_workloads(kk):
    """U = B*T*(row_stride + 4) per anchor + the queries read + the fp32
    outputs, written out by hand for the two uniform 28-layer workloads:
    d = 512, b = 16 (rows of 1152 B) and d = 256, b = 8 (rows of 320 B)."""
    L, H, B, T, dR = 28, 28, 32, 8192, 64
    for wid, d, row in ((1, 512, 1152), (2, 256, 320)):
        cache = L * B * T * (row + 4)
        q = L * B * H * (d + dR) * 2          # bf16 queries
        out = L * B * H * d * 4
        U, cache_only = bench.algorithmic_bytes(kk, synth.workload(wid))
        assert cache_only == cache
        assert U == cache + q + out
    assert bench.algorithmic_bytes(kk, synth.workload(1))[0] == 8_565_358_592
    assert bench.algorithmic_bytes(kk, synth.workload(2))[0] == 2_419_916_800


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            # one dispatch reported in two parts (per-agent rows are summed)
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib / 2})
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib / 2})
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "OTHER", "Counter_Value": 1e9})


def test_traffic_from_calibrates_on_the_copies(tmp_path):
    """Two steps (decode + merge each) and three 1 GiB copies.  FETCH_SIZE is
    made to read half the copy's bytes and WRITE_SIZE all of them, so the
    factors are 2 and 1 and the per-step bytes follow exactly."""
    gib_kib = 1024 * 1024
    dec = "void kk::(anonymous namespace)::decode_kernel<3, 0>(kk::DecodeArgs)"
    mrg = "kk::(anonymous namespace)::merge_kernel(kk::DecodeArgs)"
    cp = "__amd_rocclr_copyBuffer"
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counters(f, "FETCH_SIZE", [(dec, 1000.0), (mrg, 100.0), (dec, 1200.0), (mrg, 100.0)] +
                    [(cp, gib_kib / 2)] * 3 + [("other_kernel", 5e6)])
    _write_counters(w, "WRITE_SIZE", [(dec, 10.0), (mrg, 30.0), (dec, 10.0), (mrg, 30.0)] + [(cp, gib_kib)] * 3)
    rec = bench.traffic_from(str(f), str(w), 1024, "x")
    fc, wc = rec["counters"]["FETCH_SIZE"], rec["counters"]["WRITE_SIZE"]
    assert fc["steps"] == 2 and fc["copy_dispatches"] == 3 and fc["decode_and_merge_dispatches"] == 4
    assert fc["copy_factor"] == pytest.approx(2.0) and wc["copy_factor"] == pytest.approx(1.0)
    assert fc["bytes_per_step"] == pytest.approx((1000 + 100 + 1200 + 100) / 2 * 1024 * 2)
    assert wc["bytes_per_step"] == pytest.approx((10 + 30) * 1024)
    assert rec["hbm_bytes_per_step"] == pytest.approx(fc["bytes_per_step"] + wc["bytes_per_step"])
    assert rec["kernel_source_sha256"] == bench.kernel_source_digest()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
