"""Benchmark one decode step of compressed MLA attention on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload 3]

A step is one kk_decode_attn call over every layer of the workload (by
default the Qwen2.5-14B-shaped mixed 4x table: 48 layers, 40 heads, r = 512,
d_R = 64, batch 32, 8192 cached tokens per sequence) with the caches, queries
and sequence lengths already resident in HBM.  Prints one JSON line.

roofline.achieved = algorithmic bytes of one step / mean device time of one
step (HIP events on the launch stream; a step is the decode launch plus the
small split-merge launch).  Algorithmic bytes U = anchor caches once (rows +
scales) + the d_eff + d_R query values read per layer + the fp32 outputs
written.

roofline.traffic (HBM bytes per step) comes from two rocprofv3 counter passes
over this same command with --calibration-copy-mib: FETCH_SIZE, then
WRITE_SIZE.  Each counter is scaled by what it reads for a device-to-device
copy of known size, and the result is stored with a digest of the kernel
sources by

    python bench.py --traffic-from FETCH.csv WRITE.csv

It is reported as null when the kernel sources have changed since.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0     # dense fp16/bf16 MFMA, MI355X


def algorithmic_bytes(kk, w):
    """U = sum_anchors B*T*(row_stride + 4) + sum_l B*H*(d_eff + d_R)*sizeof(q) + sum_l B*H*d_eff*4."""
    qsize = 4 if str(w.q_dtype) == "torch.float32" else 2
    cache = sum(w.batch * w.seq_len * (kk.row_stride_bytes(w.layers[a].d, w.d_rope, w.layers[a].bits) + 4)
                for a in w.anchors())
    q = sum(w.batch * w.n_heads * (w.d_eff(l) + w.d_rope) * qsize for l in range(w.n_layers))
    out = sum(w.batch * w.n_heads * w.d_eff(l) * 4 for l in range(w.n_layers))
    return cache + q + out, cache


def epilogue_bytes(w, d_v, d_model):
    """Per step: W_UV blocks on the kept coordinates + W_O (bf16), o_lat read, v written and read, y written."""
    H = w.n_heads
    tot = 0
    for l in range(w.n_layers):
        d = w.d_eff(l)
        tot += H * d_v * d * 2 + d_model * H * d_v * 2
        tot += w.batch * H * d * 4 + 2 * w.batch * H * d_v * 4 + w.batch * d_model * 4
    return tot


def gqa_bytes(kk, w):
    """Per step: each anchor's codes of every KV head plus one scale per token,
    the queries read and the fp32 outputs written."""
    qsize = 4 if str(w.q_dtype) == "torch.float32" else 2
    cache = sum(w.batch * w.seq_len * (w.n_kv_heads * kk.row_stride_bytes(w.d_head, w.d_head, w.layers[a].bits) + 4)
                for a in w.anchors())
    return cache + w.n_layers * w.batch * w.n_q_heads * w.d_head * (qsize + 4)


def useful_flops(w):
    """Q.K and P.V multiply-adds per step: B*T*(2H(d+d_R) + 2Hd) per layer."""
    return sum(w.batch * w.seq_len * (2 * w.n_heads * (w.d_eff(l) + w.d_rope) + 2 * w.n_heads * w.d_eff(l))
               for l in range(w.n_layers))


# sources the decode step is built from (its kernels, launch descriptors and planner)
DECODE_SOURCES = ("kk_decode_kernel.h", "kk_decode.hip", "kk_internal.h", "kk_host.cpp")


def kernel_source_digest():
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        p = os.path.join(ROOT, "compressed_decode_attention_kk_amd", "csrc", name)
        with open(p, "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(workload_name):
    """HBM bytes per step from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload_name}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_step")


DECODE_KERNELS = ("decode_kernel", "merge_kernel")
COPY_KERNEL = "copyBuffer"


def _counter_rows(path, counter):
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = r["Dispatch_Id"]
            rows.setdefault(key, [r["Kernel_Name"], 0.0])
            rows[key][1] += float(r["Counter_Value"])
    return list(rows.values())


def traffic_from(fetch_csv, write_csv, copy_mib, workload_name):
    """HBM bytes per step from rocprofv3 FETCH_SIZE / WRITE_SIZE passes (KiB per
    dispatch), each calibrated on the copies of known size in the same run."""
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, name)
        # the calibration copies: FETCH_SIZE counts about half of a copy's
        # bytes here, so the cut sits well below that (smaller copies stay out)
        copies = [v for k, v in rows if COPY_KERNEL in k and v * 1024 > 0.25 * copy_mib * 2 ** 20]
        if not copies:
            raise SystemExit(f"no calibration copy dispatch found in {path}")
        factor = copy_mib * 2 ** 20 / (sum(copies) / len(copies) * 1024)
        dec = [(k, v) for k, v in rows if any(n in k for n in DECODE_KERNELS)]
        n_steps = sum(1 for k, _ in dec if DECODE_KERNELS[0] in k)      # one decode launch per step
        per_step = sum(v for _, v in dec) * 1024 / max(n_steps, 1)
        out[name] = {"raw_bytes_per_step": per_step, "copy_factor": factor, "bytes_per_step": per_step * factor,
                     "steps": n_steps, "decode_and_merge_dispatches": len(dec), "copy_dispatches": len(copies)}
    rec = {"workload": workload_name, "kernel_source_sha256": kernel_source_digest(),
           "hbm_bytes_per_step": out["FETCH_SIZE"]["bytes_per_step"] + out["WRITE_SIZE"]["bytes_per_step"],
           "counters": out, "calibration_copy_mib": copy_mib,
           "method": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, over bench.py --steps 3 --warmup 1 "
                     "--no-cpu-baseline --calibration-copy-mib M; sum over the decode_kernel and merge_kernel "
                     "dispatches / number of decode_kernel dispatches, each counter scaled by the copy bytes / "
                     "the counter bytes of the copies"}
    return rec


def _short_kernel(name):
    """'void kk::(anonymous namespace)::decode_kernel<3, 0>(kk::DecodeArgs)' -> 'decode_kernel<3, 0>'."""
    import re
    m = re.search(r"(\w+(?:<[^()]*>)?)\(", name)
    return m.group(1) if m else name[:60]


STEP_KERNELS = ("append_kernel", "store_kernel", "decode_kernel", "merge_kernel", "gemm_kernel", "gemm_lds_kernel")


def trace_summary(trace_csv, steps, warmup, kernels=STEP_KERNELS):
    """Durations of the step's kernels in a rocprofv3 --kernel-trace CSV of
    `bench.py --steps K --warmup W`: of each kernel in `kernels` (the cache
    writes of the set-up are not among them), the last K * (calls per step)
    dispatches are the timed ones.  Returns markdown."""
    import csv
    import statistics
    with open(trace_csv) as f:
        rows = [r for r in csv.DictReader(f) if "kk::" in r["Kernel_Name"] and
                _short_kernel(r["Kernel_Name"]).split("<")[0] in kernels]
    by = {}
    for r in rows:
        by.setdefault(_short_kernel(r["Kernel_Name"]), []).append(r)
    lines = ["| kernel | VGPR | AGPR | SGPR | static LDS B | scratch B | workgroups | timed calls | avg us | min us | "
             "p50 us | max us | all calls | all avg us |", "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    timed_all = []
    for k, rs in sorted(by.items(), key=lambda kv: -sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                                                       for r in kv[1])):
        rs.sort(key=lambda r: int(r["Start_Timestamp"]))
        per_step = round(len(rs) / (steps + warmup))
        if per_step == 0:           # launched outside the steps (a set-up call)
            continue
        timed = rs[-steps * per_step:]
        timed_all += timed
        us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
        us_all = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        r0 = rs[-1]
        wgs = int(r0["Grid_Size_X"]) // max(int(r0["Workgroup_Size_X"]), 1)
        lines.append(f"| {k} | {r0['VGPR_Count']} | {r0['Accum_VGPR_Count']} | {r0['SGPR_Count']} | "
                     f"{r0['LDS_Block_Size']} | {r0['Scratch_Size']} | {wgs} | {len(us)} | "
                     f"{sum(us) / len(us):.1f} | {min(us):.1f} | {statistics.median(us):.1f} | {max(us):.1f} | "
                     f"{len(us_all)} | {sum(us_all) / len(us_all):.1f} |")
    timed_all.sort(key=lambda r: int(r["Start_Timestamp"]))
    n = len(timed_all) // steps
    busy, span = [], []
    for i in range(steps):
        g = timed_all[i * n:(i + 1) * n]
        busy.append(sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in g) / 1e3)
        span.append((max(int(r["End_Timestamp"]) for r in g) - min(int(r["Start_Timestamp"]) for r in g)) / 1e3)
    lines.append("")
    lines.append(f"Timed steps: {steps} ({n} library dispatches each). Per step, sum of kernel durations: "
                 f"avg {sum(busy) / steps:.1f} us (min {min(busy):.1f}, max {max(busy):.1f}); first start to "
                 f"last end: avg {sum(span) / steps:.1f} us.")
    return "\n".join(lines)


def pmc_summary(csvs, kernel="decode_kernel", n_cus=256, n_xcds=8):
    """Counters of the `kernel` dispatches in rocprofv3 --pmc CSVs (one pass per
    file), averaged over those dispatches, with derived rates.  Returns markdown.
    Normalisation (stated with each rate): GRBM_GUI_ACTIVE sums the 8 XCDs, so
    kernel cycles = GRBM_GUI_ACTIVE / 8; the SQ *_CYCLES counters count per
    SIMD in units of 4 cycles where noted."""
    import csv
    vals = {}
    names = set()
    ndisp = 0
    for path in csvs:
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel not in r["Kernel_Name"]:
                    continue
                names.add(_short_kernel(r["Kernel_Name"]))
                key = (r["Dispatch_Id"], r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (d, c), v in per.items():
            vals.setdefault(c, []).append(v)
        ndisp = max(ndisp, len({d for d, _ in per}))
    avg = {c: sum(v) / len(v) for c, v in vals.items()}
    lines = [f"Kernel: {', '.join(sorted(names))}; dispatches per pass: {ndisp}", "",
             "| counter | mean per dispatch |", "|---|---|"]
    for c in sorted(avg):
        lines.append(f"| {c} | {avg[c]:.4g} |")
    der = []
    cyc = avg.get("GRBM_GUI_ACTIVE", 0.0) / n_xcds
    simds = 4 * n_cus
    waves = avg.get("SQ_WAVES")
    if cyc:
        der.append(("kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs)", f"{cyc:.4g}"))
    if waves:
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_SMEM",
                  "SQ_INSTS_BRANCH"):
            if c in avg:
                der.append((f"{c} per wave", f"{avg[c] / waves:.1f}"))
    if "SQ_INSTS_VALU" in avg and "SQ_INSTS_MFMA" in avg and avg["SQ_INSTS_MFMA"]:
        der.append(("VALU instructions per MFMA instruction", f"{avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f}"))
    if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        der.append(("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles)",
                    f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (simds * cyc):.3f}"))
    if cyc and "SQ_ACTIVE_INST_VALU" in avg:
        der.append(("VALU active: 4 x SQ_ACTIVE_INST_VALU / (SIMDs x cycles)",
                    f"{4 * avg['SQ_ACTIVE_INST_VALU'] / (simds * cyc):.3f}"))
    if cyc and "SQ_WAVE_CYCLES" in avg:
        der.append(("mean resident waves per CU: 4 x SQ_WAVE_CYCLES / (CUs x cycles)",
                    f"{4 * avg['SQ_WAVE_CYCLES'] / (n_cus * cyc):.2f}"))
    if avg.get("SQ_ACTIVE_INST_LDS"):
        der.append(("LDS bank-conflict cycles per LDS-active cycle: SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS",
                    f"{avg.get('SQ_LDS_BANK_CONFLICT', 0.0) / avg['SQ_ACTIVE_INST_LDS']:.4f}"))
    if cyc and "SQ_LDS_BANK_CONFLICT" in avg:
        der.append(("LDS bank-conflict cycles per CU cycle: SQ_LDS_BANK_CONFLICT / (CUs x cycles)",
                    f"{avg['SQ_LDS_BANK_CONFLICT'] / (n_cus * cyc):.4f}"))
    if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg and avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"]:
        der.append(("L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS)",
                    f"{avg['TCC_HIT_sum'] / (avg['TCC_HIT_sum'] + avg['TCC_MISS_sum']):.3f}"))
    if "SQ_WAIT_INST_ANY" in avg and avg.get("SQ_WAVE_CYCLES"):
        der.append(("share of wave time waiting on any dependency: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
                    f"{avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.3f}"))
    if der:
        lines += ["", "| derived | value |", "|---|---|"] + [f"| {a} | {b} |" for a, b in der]
    return "\n".join(lines)


def copy_bandwidth(torch, mib: int = 1024, reps: int = 5) -> float:
    """Measured device-to-device copy rate (GB/s, bytes read + written) on the
    launch stream: the practical streaming ceiling the achieved rate is set
    against besides the 8 TB/s peak."""
    n = mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:                                      # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """The oracle (unchanged) on the host cores: decode of whole (layer, sequence)
    pairs of the same workload until the time budget is used."""
    import numpy as np
    import torch
    from oracle import kk_oracle as ko
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:                                    # pragma: no cover
        cores = os.cpu_count() or 1
    ql, qr = synth.queries(w, "cuda")
    done, spent, nbytes = 0, 0.0, 0
    qsize = 4 if str(w.q_dtype) == "torch.float32" else 2
    pairs = [(l, s) for s in range(w.batch) for l in range(w.n_layers)]
    cache = {}
    for (l, s) in pairs:
        a = w.layers[l].anchor
        if (a, s) not in cache:
            cache.clear()
            lat, rope, _ = synth.source_rows(w, a, "cuda", seqs=[s])
            packed, scales, _ = ko.write_cache(lat[0].cpu().numpy(), rope[0].cpu().numpy(), w.d_eff(l), w.bits_eff(l))
            cache[(a, s)] = (packed, scales)
            del lat, rope
        packed, scales = cache[(a, s)]
        q_lat = ql[l, s].float().cpu().numpy().astype(np.float64)
        q_rope = qr[l, s].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        ko.decode_layer(q_lat, q_rope, packed, scales, w.d_eff(l), w.d_rope, w.bits_eff(l), w.layers[l].sm_scale,
                        w.seq_len)
        spent += time.perf_counter() - t0
        done += 1
        d = w.d_eff(l)
        nbytes += (packed.nbytes + scales.nbytes + w.n_heads * (d + w.d_rope) * qsize + w.n_heads * d * 4)
        if spent >= budget_s:
            break
    return {"value": done / spent, "unit": "layer*tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "effective_gbps": nbytes / spent / 1e9,
            "sample": f"{done} (layer, sequence) decodes of the same workload (unpack, dequantize, fp64 attention "
                      f"over {w.seq_len} tokens, {w.n_heads} heads), {spent:.1f} s of CPU time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--uniform", metavar="D,B", default=None,
                    help="time 8 anchor layers of kept width D and bit width B in the 14B shape "
                         "(40 heads, B=32, T=8192) instead of a numbered workload")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append", action="store_true",
                    help="time kk_append_decode (write each sequence's newest token into every anchor, then decode)")
    ap.add_argument("--hetero", action="store_true",
                    help="time kk_multi_decode_attn on the heterogeneous 14B batch (four tables, 8 sequences each)")
    ap.add_argument("--epilogue", action="store_true",
                    help="time kk_latent_epilogue (W_UV per head, then W_O; 14B shapes d_v = 128, d_model = 5120) "
                         "on the decode output")
    ap.add_argument("--gqa", action="store_true",
                    help="time kk_gqa_decode_attn: the grouped-query 14B model (40 query / 8 KV heads of 128) with "
                         "the frozen 4x precision + depth table, 16 sequences x 16384 tokens")
    ap.add_argument("--depth", choices=["shared", "own_cache", "anchors_only"], default="shared",
                    help="decode step only: the table as is, with every inheriting layer given a cache of its own "
                         "(same width and bits as its anchor), or with the inheriting layers left out")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, run 3 device-to-device copies of this size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic record from two rocprofv3 counter CSVs and exit")
    ap.add_argument("--trace-from", metavar="KERNEL_TRACE_CSV",
                    help="summarize the timed dispatches of a rocprofv3 --kernel-trace CSV of a run with the same "
                         "--steps and --warmup, and exit")
    ap.add_argument("--pmc-from", nargs="+", metavar="COUNTER_CSV",
                    help="summarize rocprofv3 --pmc CSVs (one pass each) for the decode kernel, and exit")
    args = ap.parse_args()
    if args.trace_from:
        print(trace_summary(args.trace_from, args.steps, args.warmup))
        return
    if args.pmc_from:
        print(pmc_summary(args.pmc_from))
        return
    if args.traffic_from:
        import synth
        w = synth.workload(args.workload)
        rec = traffic_from(args.traffic_from[0], args.traffic_from[1], args.calibration_copy_mib or 1024, w.name)
        path = os.path.join(ROOT, "profiles", f"decode_{w.name}_hbm_traffic.json")
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return
    if args.uniform and (args.gqa or args.hetero or args.append or args.epilogue or args.depth != "shared"):
        print("--uniform times the decode step of one uniform table", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (the decode path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import compressed_decode_attention_kk_amd as kk
    import synth
    from synth.device import build_caches

    kk.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    t_setup = time.perf_counter()
    if args.depth != "shared" and (args.gqa or args.hetero or args.append or args.epilogue):
        print("--depth applies to the decode step of one table", file=sys.stderr)
        sys.exit(2)
    if args.gqa and (args.hetero or args.append or args.epilogue):
        print("--gqa times the grouped-query decode step alone", file=sys.stderr)
        sys.exit(2)
    if args.gqa:
        from synth.device import build_gqa_caches
        w = synth.gqa_workload()
        runs_w = []
        gm = kk.GqaModel(w.layers, w.n_q_heads, w.n_kv_heads, w.d_head)
        gcaches = build_gqa_caches(kk, gm, w)
        gq = synth.gqa_queries(w, "cuda")
        seq_lens = torch.full((w.batch,), w.seq_len, dtype=torch.int32, device="cuda")
        dec = kk.GqaDecoder(gm, gcaches, w.batch, w.seq_len, w.seq_len, split_tokens=args.split_tokens)
        step = lambda: dec(gq, seq_lens)
    elif args.hetero:
        if args.append or args.epilogue:
            print("--hetero times the decode step alone", file=sys.stderr)
            sys.exit(2)
        runs_w = synth.hetero_workloads()
        w = runs_w[0]
        runs, qls, qrs = [], [], []
        for rw in runs_w:
            m = kk.Model(rw.layers, rw.n_heads, rw.r, rw.d_rope)
            runs.append((m, build_caches(kk, m, rw), rw.batch))
            q = synth.queries(rw, "cuda")
            qls.append(q[0])
            qrs.append(q[1])
        ql = torch.cat(qls, 1).contiguous()
        qr = torch.cat(qrs, 1).contiguous()
        del qls, qrs
        batch = sum(rw.batch for rw in runs_w)
        seq_lens = torch.full((batch,), w.seq_len, dtype=torch.int32, device="cuda")
        dec = kk.MultiDecoder(runs, w.seq_len, w.seq_len, split_tokens=args.split_tokens)
        step = lambda: dec(ql, qr, seq_lens)
    else:
        if args.uniform:
            ud, ub = (int(x) for x in args.uniform.split(","))
            w = synth.uniform_workload(ud, ub)
        else:
            w = synth.depth_variant(synth.workload(args.workload), args.depth)
        runs_w = [w]
        model = kk.Model(w.layers, w.n_heads, w.r, w.d_rope)
        caches = build_caches(kk, model, w)
        ql, qr = synth.queries(w, "cuda")
        seq_lens = torch.full((w.batch,), w.seq_len, dtype=torch.int32, device="cuda")
        dec = kk.Decoder(model, caches, w.batch, w.seq_len, w.seq_len, split_tokens=args.split_tokens)
        step = lambda: dec(ql, qr, seq_lens)
    if args.epilogue and args.append:
        print("--epilogue and --append are separate steps", file=sys.stderr)
        sys.exit(2)
    if args.epilogue:
        d_v, d_model = 128, 5120
        dec(ql, qr, seq_lens)
        wts = [synth.gen_epilogue_weights(w.wid, l, w.n_heads, d_v, w.r, d_model, "cuda") for l in range(w.n_layers)]
        w_uv, w_o = [a for a, _ in wts], [b for _, b in wts]
        v_buf = torch.empty(w.n_layers, w.batch, w.n_heads * d_v, dtype=torch.float32, device="cuda")
        y_buf = torch.empty(w.n_layers, w.batch, d_model, dtype=torch.float32, device="cuda")
        step = lambda: kk.latent_epilogue(model, w.batch, dec.out, w_uv, w_o, v_buf, y_buf)
    if args.append:
        # the newest token of each sequence (row seq_len - 1) is rewritten from seeded rows every step
        g = torch.Generator(device="cuda").manual_seed(1234)
        new_lat = torch.randn(w.n_layers, w.batch, w.r, generator=g, device="cuda")
        new_rope = torch.randn(w.n_layers, w.batch, w.d_rope, generator=g, device="cuda")
        step = lambda: dec.append(new_lat, new_rope, ql, qr, seq_lens)
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    mean_dev_ms = sum(dev_ms) / len(dev_ms)
    ms_per_step = wall * 1000.0 / args.steps

    # (not in the counter runs, whose only large copies are the calibration ones)
    copy_gbps = copy_bandwidth(torch) if args.calibration_copy_mib == 0 else None
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    U = sum(algorithmic_bytes(kk, rw)[0] for rw in runs_w)
    flops = sum(useful_flops(rw) for rw in runs_w)
    if args.gqa:
        U = gqa_bytes(kk, w)
        flops = w.n_layers * w.batch * w.seq_len * w.n_q_heads * 4 * w.d_head
    if args.epilogue:
        U = epilogue_bytes(w, d_v, d_model)
        flops = sum(2 * w.batch * w.n_heads * d_v * w.d_eff(l) + 2 * w.batch * d_model * w.n_heads * d_v
                    for l in range(w.n_layers))
    achieved = U / (mean_dev_ms * 1e-3) / 1e9
    name = "14b_hetero_4tables" if args.hetero else (w.name + "_epilogue" if args.epilogue else w.name)
    batch = w.batch if args.gqa else sum(rw.batch for rw in runs_w)
    traffic = stored_traffic(name)
    print(f"[bench] device ms/step mean {mean_dev_ms:.4f} p10 {dev_ms[len(dev_ms) // 10]:.4f} "
          f"p90 {dev_ms[(9 * len(dev_ms)) // 10]:.4f}; wall ms/step {ms_per_step:.4f}; U {U / 1e9:.3f} GB; "
          f"{achieved:.0f} GB/s; MFMA-useful {flops / (mean_dev_ms * 1e-3) / 1e12:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline and not args.hetero and not args.epilogue and not args.gqa:
        cpu = cpu_baseline(w, args.cpu_budget)

    if args.gqa:
        anchors = [len(w.anchors())]
        bits_tok = [sum(2 * w.n_kv_heads * w.d_head * w.layers[a].bits + 32 for a in w.anchors())]
    else:
        anchors = [len(rw.anchors()) for rw in runs_w]
        bits_tok = [sum((rw.layers[a].d + rw.d_rope) * rw.layers[a].bits + 32 for a in rw.anchors()) for rw in runs_w]
    line = {
        "metric": "compressed decode-attn layer*tokens/s",
        "value": w.n_layers * batch / (ms_per_step * 1e-3),
        "unit": "layer*tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic of the step: fp16 P.V (the Q.K products are exact int8 x int8), bf16 epilogue
        "dtype": "bf16" if args.epilogue else "f16",
        "data": "synthetic",
        "config": {"workload": name, "layers": w.n_layers, "heads": w.n_q_heads if args.gqa else w.n_heads,
                   "batch": batch, "cached_tokens": w.seq_len,
                   **({"kv_heads": w.n_kv_heads, "d_head": w.d_head} if args.gqa else {"r": w.r, "d_rope": w.d_rope}),
                   "anchors": anchors if args.hetero else anchors[0],
                   "bits_per_token": bits_tok if args.hetero else bits_tok[0],
                   "q_dtype": str(w.q_dtype).replace("torch.", ""),
                   "split_tokens": args.split_tokens or "auto", "parallelism": "none (one GPU)",
                   "step": ("grouped-query decode (precision + depth)" if args.gqa else
                            "latent epilogue (W_UV per head, W_O; d_v 128, d_model 5120)" if args.epilogue else
                            "append + decode" if args.append else
                            "heterogeneous decode (4 tables x 8 sequences)" if args.hetero else "decode")},
        "roofline": {"bound": "hbm", "kernel": "epilogue: gemm_kernel (W_UV) + gemm_lds_kernel (W_O)" if args.epilogue else
                     ("append_kernel + " if args.append else
                                                "store_kernel (plan upload) + " if args.hetero else "") +
                     "decode step: decode_kernel + merge_kernel",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_step": U, "device_ms_per_step": mean_dev_ms,
                     "device_ms_p10_p50_p90": [dev_ms[len(dev_ms) // 10], dev_ms[len(dev_ms) // 2],
                                               dev_ms[(9 * len(dev_ms)) // 10]],
                     "copy_gbps_measured": copy_gbps, "frac_of_copy": achieved / copy_gbps if copy_gbps else None,
                     "useful_tflops": flops / (mean_dev_ms * 1e-3) / 1e12,
                     "mfma_util_vs_2500_tflops": flops / (mean_dev_ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
