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


def test_uniform_table_mode(kk):
    """--uniform D,B: eight anchors of one (d, b) in the 14B shape; U written
    out by hand for d = 512, b = 4 (rows of 288 B), and the mode refuses the
    other steps before touching a GPU."""
    w = synth.uniform_workload(512, 4)
    assert (w.n_layers, w.n_heads, w.batch, w.seq_len, w.r, w.d_rope) == (8, 40, 32, 8192, 512, 64)
    assert w.anchors() == list(range(8)) and all(l.d == 512 and l.bits == 4 for l in w.layers)
    L, H, B, T = 8, 40, 32, 8192
    U, cache = bench.algorithmic_bytes(kk, w)
    assert cache == L * B * T * (288 + 4)
    assert U == cache + L * B * H * 576 * 2 + L * B * H * 512 * 4 == 645_136_384
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--uniform", "512,4", "--gqa"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--uniform" in r.stderr


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


def _write_trace(path, rows):
    cols = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
            "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
            "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(cols)
        for i, (name, t0, t1) in enumerate(rows):
            wr.writerow(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, i + 1, 7, name, i + 1, t0, t1, 0, 0, 128, 0, 96,
                         256, 1, 1, 256 * 100, 1, 1])


def test_trace_summary_times_the_timed_dispatches_only(tmp_path):
    """Set-up writes, 2 warmup steps (slow), then 3 timed steps of decode +
    merge: only the last 3 of each kernel are averaged; the per-step sums
    and spans follow from the timestamps (ns)."""
    dec = "void kk::(anonymous namespace)::decode_kernel<3, 0>(kk::DecodeArgs)"
    mrg = "void kk::(anonymous namespace)::merge_kernel(kk::DecodeArgs)"
    wr = "void kk::(anonymous namespace)::write_kernel<4>(kk::WriteArgs)"
    rows, t = [], 0
    for _ in range(5):
        rows.append((wr, t, t + 1000)); t += 2000
    for step, d in enumerate([9000, 8000, 1000, 1200, 1400]):     # warmup 2, timed 3 (us * 1000)
        rows.append((dec, t, t + d)); t += d
        rows.append((mrg, t, t + 100)); t += 100 + 50000
    rows.append((dec.replace("decode_kernel", "gemm_kernel"), t, t + 99000))   # one set-up launch, not a step kernel
    f = tmp_path / "trace.csv"
    _write_trace(f, rows)
    md = bench.trace_summary(str(f), steps=3, warmup=2)
    assert "gemm_kernel" not in md
    line = [l for l in md.splitlines() if l.startswith("| decode_kernel<3, 0>")][0].split("|")
    assert line[8].strip() == "3" and float(line[9]) == pytest.approx(1.2)       # timed calls, avg us
    assert float(line[10]) == pytest.approx(1.0) and float(line[12]) == pytest.approx(1.4)
    assert "write_kernel" not in md
    assert "sum of kernel durations: avg 1.3 us" in md and "last end: avg 1.3 us" in md


def test_pmc_summary_derives_the_rates(tmp_path):
    """Two dispatches of the decode kernel with fixed counters: per-wave
    counts and the normalised rates follow the stated formulas."""
    dec = "void kk::(anonymous namespace)::decode_kernel<3, 0>(kk::DecodeArgs)"
    cnt = {"SQ_WAVES": 1000.0, "SQ_INSTS_VALU": 5.0e6, "SQ_INSTS_MFMA": 1.0e6, "GRBM_GUI_ACTIVE": 8.0e6,
           "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 1024 * 1.0e6, "SQ_ACTIVE_INST_VALU": 0.5 / 4 * 1024 * 1.0e6,
           "SQ_WAVE_CYCLES": 7.0 / 4 * 256 * 1.0e6, "TCC_HIT_sum": 30.0, "TCC_MISS_sum": 70.0,
           "SQ_LDS_BANK_CONFLICT": 5.0, "SQ_ACTIVE_INST_LDS": 50.0}
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    f = tmp_path / "pmc.csv"
    with open(f, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(cols)
        for disp in (1, 2):
            for c, v in cnt.items():
                wr.writerow([disp, disp, "Agent 1", 1, 1, 1, 256, 7, dec, 256, 0, 0, 128, 0, 96, c, v, 0, 1])
            wr.writerow([disp, disp, "Agent 1", 1, 1, 1, 256, 8, "other", 256, 0, 0, 8, 0, 16, "SQ_WAVES", 1.0, 0, 1])
    md = bench.pmc_summary([str(f)])
    vals = {l.split("|")[1].strip(): l.split("|")[2].strip() for l in md.splitlines() if l.count("|") == 3}
    assert float(vals["kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs)"]) == pytest.approx(1.0e6)
    assert float(vals["SQ_INSTS_VALU per wave"]) == pytest.approx(5000.0)
    assert float(vals["VALU instructions per MFMA instruction"]) == pytest.approx(5.0)
    assert float(vals["MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles)"]) == pytest.approx(0.25)
    assert float(vals["VALU active: 4 x SQ_ACTIVE_INST_VALU / (SIMDs x cycles)"]) == pytest.approx(0.5)
    assert float(vals["mean resident waves per CU: 4 x SQ_WAVE_CYCLES / (CUs x cycles)"]) == pytest.approx(7.0)
    assert float(vals["L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS)"]) == pytest.approx(0.3)
    # the dispatch count is per pass, also when a counter is collected in several passes
    assert "dispatches per pass: 2" in md
    md2 = bench.pmc_summary([str(f), str(f)])
    assert "dispatches per pass: 2" in md2
    vals2 = {l.split("|")[1].strip(): l.split("|")[2].strip() for l in md2.splitlines() if l.count("|") == 3}
    assert vals2 == vals


def test_depth_variants_of_the_14b_table(kk):
    """--depth: own_cache keeps every layer's rows and widths but gives each
    inheriting layer its own cache (the cache bytes grow by the inheritors'
    rows); anchors_only keeps the 33 anchors and their cache bytes."""
    w = synth.workload(3)
    own = synth.depth_variant(w, "own_cache")
    only = synth.depth_variant(w, "anchors_only")
    assert synth.depth_variant(w, "shared") is w
    assert own.n_layers == w.n_layers == 48 and len(own.anchors()) == 48 and len(w.anchors()) == 33
    assert [own.d_eff(l) for l in range(48)] == [w.d_eff(l) for l in range(48)]
    assert [own.bits_eff(l) for l in range(48)] == [w.bits_eff(l) for l in range(48)]
    assert [s.sm_scale for s in own.layers] == [s.sm_scale for s in w.layers]
    assert only.n_layers == 33 and only.anchors() == list(range(33))
    assert [(s.d, s.bits) for s in only.layers] == [(w.layers[a].d, w.layers[a].bits) for a in w.anchors()]
    U, cache = bench.algorithmic_bytes(kk, w)
    U_own, cache_own = bench.algorithmic_bytes(kk, own)
    U_only, cache_only = bench.algorithmic_bytes(kk, only)
    inh = [l for l in range(48) if w.layers[l].anchor != l]
    extra = sum(w.batch * w.seq_len * (kk.row_stride_bytes(w.d_eff(l), w.d_rope, w.bits_eff(l)) + 4) for l in inh)
    assert cache_own == cache + extra and U_own - U == extra
    assert cache_only == cache and U_only < U
    with pytest.raises(ValueError):
        synth.depth_variant(w, "other")
