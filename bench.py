#!/usr/bin/env python3
"""Benchmark of the fused LoRA-MLP forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1|2|3|4|5|6]

A step is one forward and one backward of the whole path on one batch of
synthetic, seeded inputs already resident in HBM: for the MLP shapes
lora_mlp_fwd + lora_mlp_bwd, for the attention shape lora_qkv_fwd/bwd +
lora_o_fwd/bwd.  The default workload is the Llama-3-8B-shaped SwiGLU LoRA
MLP (8192 tokens, 4096 -> 14336 -> 4096, r = 16, alpha = 32, bf16 with fp32
accumulation).

Prints one JSON line with the throughput (tokens/s over the timed steps),
the roofline of the dominant kernel (timed live with HIP events on the
library's launch stream) and the CPU oracle timed on a bounded token sample
on this host ("cpu_baseline").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
PEAK_F32_VALU_TFLOPS = 157.3  # 256 CU x 4 SIMD x 64 lanes x 2 flop (FMA) x 2.4 GHz
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_flops(cfg, name):
    """Algorithmic flops of one launch of a GEMM family for this workload."""
    T, r = cfg.T, cfg.r
    if cfg.kind == "mlp":
        H, I = cfg.H, cfg.I
        table = {
            "gemm_nn_act_fwd": 2 * T * H * (2 * I) + 2 * T * r * (2 * I),  # gate+up, incl. U B
            "gemm_nn_store": 2 * T * I * H + 2 * T * r * H,                  # down
            "gemm_nt_act_bwd": 2 * T * H * I + 2 * T * r * I,                # dh
            "gemm_nt_store": 2 * T * (2 * I) * H + 2 * T * (2 * r) * H,      # dX
        }
    elif cfg.kind == "relu2":
        H, I = cfg.H, cfg.I
        table = {
            "gemm_nn_relu2_fwd": 2 * T * H * I + 2 * T * r * I,             # up, incl. U B
            "gemm_nn_store": 2 * T * I * H + 2 * T * r * H,                  # down
            "gemm_nt_relu2_bwd": 2 * T * H * I + 2 * T * r * I,              # dh
            "gemm_nt_store": 2 * T * I * H + 2 * T * r * H,                  # dX
        }
    else:
        H, N = cfg.H, cfg.Nq + cfg.Nk + cfg.Nv
        table = {
            "gemm_nn_store": None,  # QKV and O share the family; averaged below
            "gemm_nt_store": None,
        }
        qkv_f = 2 * T * H * N + 2 * T * r * N
        o_f = 2 * T * cfg.Nq * H + 2 * T * r * H
        table["gemm_nn_store"] = (qkv_f + o_f) / 2
        qkv_b = 2 * T * N * H + 2 * T * (3 * r) * H
        o_b = 2 * T * H * cfg.Nq + 2 * T * r * cfg.Nq
        table["gemm_nt_store"] = (qkv_b + o_b) / 2
    base = name.replace("_nf4", "").replace("_f32", "")
    return table.get(base)


# Kernel names (as rocprofv3 prints them) of each GEMM family: the kernel's
# template arguments are <B orientation, gate/up tiles, epilogue, NF4 weights,
# activation>; a family covers both activations.
FAMILY_KERNEL = {
    "gemm_nn_act_fwd": "gemm_kernel<0, true, 1, false, ",
    "gemm_nn_act_fwd_nf4": "gemm_kernel<0, true, 1, true, ",
    "gemm_nn_store": "gemm_kernel<0, false, 0, false, ",
    "gemm_nn_store_nf4": "gemm_kernel<0, false, 0, true, ",
    "gemm_nt_act_bwd": "gemm_kernel<1, false, 2, false, ",
    "gemm_nt_act_bwd_nf4": "gemm_kernel<1, false, 2, true, ",
    "gemm_nt_store": "gemm_kernel<1, false, 0, false, ",
    "gemm_nt_store_nf4": "gemm_kernel<1, false, 0, true, ",
    "gemm_nn_relu2_fwd": "gemm_kernel<0, false, 3, false, ",
    "gemm_nn_relu2_fwd_nf4": "gemm_kernel<0, false, 3, true, ",
    "gemm_nt_relu2_bwd": "gemm_kernel<1, false, 4, false, ",
    "gemm_nt_relu2_bwd_nf4": "gemm_kernel<1, false, 4, true, ",
}
COPY_KERNEL = "neg_kernel"  # the --copy-calibration kernel


def pmc_summary(fetch_csv, write_csv, config_id):
    """Per-launch HBM bytes of every GEMM family from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for the known-size copy of --copy-calibration.  Writes
    profiles/<family>_<workload>_traffic.txt and prints the table."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return acc

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")

    def find(acc, key):
        vals = [v for k, vs in acc.items() if key in k for v in vs]
        return sum(vals) / len(vals) if vals else None

    from workload import CONFIGS
    cfg = CONFIGS[config_id]
    # the calibration copy moves the same number of bytes each way
    cf, cw = find(f, COPY_KERNEL), find(w, COPY_KERNEL)
    if cf is None or cw is None:
        raise SystemExit("no calibration copy kernel in the counter files (run with --copy-calibration)")
    # the copy's true size is logged by bench.py; the counter files only hold KiB:
    # WRITE_SIZE of the copy is taken as exact when it equals a whole MiB count
    true_kib = round(cw / 1024) * 1024
    kf, kw = true_kib / cf, true_kib / cw
    tag = workload_tag(cfg)
    out = []
    for fam, kname in FAMILY_KERNEL.items():
        a, b = find(f, kname), find(w, kname)
        if a is None or b is None:
            continue
        hbm = (a * kf + b * kw) * 1024
        path = os.path.join(ROOT, "profiles", f"{fam}_{tag}_traffic.txt")
        with open(path, "w") as fh:
            fh.write(f"# HBM traffic per launch of {kname} ({fam}), workload {cfg.note}\n")
            fh.write("# from two rocprofv3 --pmc runs over bench.py (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),\n")
            fh.write(f"# each scaled by the same counter on a {true_kib // 1024} MiB fp32 copy kernel of known size\n")
            fh.write("#   cd /tmp && export TMPDIR=/tmp\n")
            fh.write(f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o pf -- python3 <repo>/bench.py "
                     f"--config {config_id} --steps 2 --warmup 1 --no-cpu-baseline --no-family-times --copy-calibration {true_kib // 1024}\n")
            fh.write("#   rocprofv3 --pmc WRITE_SIZE ... (same)\n")
            fh.write(f"#   python3 bench.py --config {config_id} --pmc-summary pf_counter_collection.csv pw_counter_collection.csv\n")
            fh.write(f"source_digest = {source_digest()}\n")
            fh.write(f"fetch_kib_raw = {a:.1f}\nwrite_kib_raw = {b:.1f}\n")
            fh.write(f"copy_fetch_kib_raw = {cf:.1f}\ncopy_write_kib_raw = {cw:.1f}\ncopy_true_kib = {true_kib}\n")
            fh.write(f"fetch_scale = {kf:.4f}\nwrite_scale = {kw:.4f}\n")
            fh.write(f"hbm_read_bytes_per_launch = {a * kf * 1024:.0f}\nhbm_write_bytes_per_launch = {b * kw * 1024:.0f}\n")
            fh.write(f"hbm_bytes_per_launch = {hbm:.0f}\n")
        out.append((fam, a * kf * 1024, b * kw * 1024))
    for fam, rd, wr in out:
        print(f"{fam:22s} read {rd / 1e9:8.3f} GB  write {wr / 1e9:8.3f} GB per launch")
    print(f"calibration: FETCH x{kf:.4f}, WRITE x{kw:.4f}")


# Counter passes of --counter-summary (each within one rocprofv3 --pmc run's
# limits: at most 8 SQ and 2 GRBM counters).
PMC_PASSES = {
    "mfma": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
             "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_LDS_ADDR_CONFLICT",
            "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"],
    "cx": ["SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VALU2",
           "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"],
}
N_SIMD, N_CU, N_XCD = 1024, 256, 8  # MI355X: 256 CUs x 4 SIMDs in 8 XCDs


def counter_summary(csvs, config_id):
    """MFMA and LDS counters of every GEMM family from rocprofv3 --pmc runs of
    the PMC_PASSES sets over bench.py.  Per family: the MFMA pipe's busy share
    of the SIMD cycles, the executed bf16 MFMA flops against the algorithmic
    flops, VALU instructions per MFMA, LDS bank-conflict cycles against LDS
    active cycles, and the shader clock (GRBM_GUI_ACTIVE over the dispatch
    time).  Writes profiles/<family>_<workload>_counters.txt."""
    import csv

    from workload import CONFIGS
    cfg = CONFIGS[config_id]
    vals, dur = {}, {}
    for path in csvs:
        for row in csv.DictReader(open(path)):
            k = row["Kernel_Name"]
            vals.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
            d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
            dur.setdefault(k, {}).setdefault(row["Dispatch_Id"] + path, d)
    tag = workload_tag(cfg)
    lines = []
    for fam, kname in FAMILY_KERNEL.items():
        keys = [k for k in vals if kname in k]
        if not keys:
            continue
        avg = {}
        for k in keys:
            for cn, v in vals[k].items():
                avg.setdefault(cn, []).extend(v)
        avg = {cn: sum(v) / len(v) for cn, v in avg.items()}
        ds = [d for k in keys for d in dur[k].values()]
        t = sum(ds) / len(ds)
        fl = kernel_flops(cfg, fam)
        # rocprofv3 sums GRBM_GUI_ACTIVE over the 8 XCDs' GRBM instances
        gui = avg["GRBM_GUI_ACTIVE"] / N_XCD if "GRBM_GUI_ACTIVE" in avg else None
        m = {"dispatch_s": t}
        if gui:
            m["clock_GHz"] = gui / t / 1e9
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and gui:
            m["mfma_busy_frac"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * N_SIMD)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
            ex = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            m["mfma_flops_executed"] = ex
            if fl:
                m["mfma_flops_algorithmic"] = fl
                m["executed_over_algorithmic"] = ex / fl
        if "SQ_INSTS_MFMA" in avg and "SQ_INSTS_VALU" in avg and avg["SQ_INSTS_MFMA"]:
            m["valu_non_mfma_per_mfma"] = (avg["SQ_INSTS_VALU"] - avg["SQ_INSTS_MFMA"]) / avg["SQ_INSTS_MFMA"]
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and avg.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            m["coexec_over_mfma_busy"] = avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"]
        if "SQ_ACTIVE_INST_VALU" in avg and gui:  # quad-cycles summed over the SIMDs
            m["valu_active_frac"] = 4 * avg["SQ_ACTIVE_INST_VALU"] / (gui * N_SIMD)
        if "SQ_LDS_IDX_ACTIVE" in avg and gui:
            m["lds_active_frac"] = avg["SQ_LDS_IDX_ACTIVE"] / (gui * N_CU)
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            m["lds_bank_conflict_over_active"] = avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"]
        if fl:
            m["tflops_under_profiler"] = fl / t / 1e12
            m["frac_of_nominal_peak"] = fl / t / 1e12 / PEAK_BF16_TFLOPS
            if gui:
                m["frac_of_peak_at_measured_clock"] = fl / (gui * N_CU * 4096)
        path = os.path.join(ROOT, "profiles", f"{fam}_{tag}_counters.txt")
        with open(path, "w") as fh:
            fh.write(f"# MFMA and LDS counters per launch of {kname} ({fam}), workload {cfg.note}\n")
            fh.write("# from rocprofv3 --pmc runs over bench.py, one per counter set (averages over the dispatches):\n")
            fh.write("#   cd /tmp && export TMPDIR=/tmp\n")
            for name, cs in PMC_PASSES.items():
                fh.write(f"#   rocprofv3 --pmc {' '.join(cs)} --output-format csv -d <dir> -o {name} -- python3 "
                         f"<repo>/bench.py --config {config_id} --steps 2 --warmup 1 --no-cpu-baseline --no-family-times\n")
            fh.write(f"#   python3 bench.py --config {config_id} --counter-summary "
                     f"{' '.join(n + '_counter_collection.csv' for n in PMC_PASSES)}   (the sets that were run)\n")
            fh.write("# coexec_over_mfma_busy = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (a VALU issued while\n")
            fh.write("# the matrix core works); valu_active_frac = 4 SQ_ACTIVE_INST_VALU (quad-cycles) / (GRBM_GUI_ACTIVE x 1024)\n")
            fh.write("# GRBM_GUI_ACTIVE below is per XCD (the counter's sum over the 8 XCDs / 8);\n")
            fh.write("# mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs);\n")
            fh.write("# mfma_flops_executed = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; clock = GRBM_GUI_ACTIVE / dispatch time;\n")
            fh.write("# frac_of_peak_at_measured_clock = algorithmic flops / (GRBM_GUI_ACTIVE x 256 CU x 4096 flop/clk)\n")
            fh.write(f"source_digest = {source_digest()}\n")
            for cn in sorted(avg):
                fh.write(f"raw.{cn} = {avg[cn]:.6g}\n")
            for k2, v in m.items():
                fh.write(f"{k2} = {v:.6g}\n")
        lines.append((fam, m))
    for fam, m in lines:
        print(f"{fam:24s} " + "  ".join(f"{k}={v:.4g}" for k, v in m.items() if k in (
            "clock_GHz", "mfma_busy_frac", "executed_over_algorithmic", "valu_non_mfma_per_mfma",
            "lds_active_frac", "lds_bank_conflict_over_active", "coexec_over_mfma_busy", "valu_active_frac",
            "frac_of_nominal_peak")))


def trace_summary(stats_csv, bench_log, config_id):
    """Per-kernel durations from a rocprofv3 --kernel-trace --stats run over
    bench.py (its *_kernel_stats.csv) next to the bench line the same run
    printed.  Writes profiles/<dominant family>_<workload>_kernel_trace.txt."""
    import csv
    import json
    import re

    from workload import CONFIGS
    cfg = CONFIGS[config_id]
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [l for l in open(bench_log) if l.startswith("{")]
    d = json.loads(lines[-1]) if lines else None

    def short(n):
        n = n.replace("lora::(anonymous namespace)::", "").replace("void ", "")
        return re.sub(r"\(lora::\w+(, \w+)*\)$", "", n)[:70]

    fam = d["roofline"]["kernel"] if d else "gemm"
    path = os.path.join(ROOT, "profiles", f"{fam}_{workload_tag(cfg)}_kernel_trace.txt")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel trace summary, workload {cfg.note}\n")
        f.write("# command (repository root on the GPU host; 3 warm-up + 10 timed steps):\n")
        f.write("#   cd /tmp && export TMPDIR=/tmp\n")
        f.write(f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o kt -- python3 <repo>/bench.py "
                f"--config {config_id} --steps 10 --warmup 3 --no-cpu-baseline --no-family-times > kt.log\n")
        f.write(f"#   python3 bench.py --config {config_id} --trace-summary <dir>/kt_kernel_stats.csv kt.log\n")
        f.write(f"source_digest = {source_digest()}\n")
        f.write("# durations in microseconds\n\n")
        f.write(f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}\n")
        for r in rows:
            f.write(f"{short(r['Name']):70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                    f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f} {float(r['Percentage']):6.2f}\n")
        if d:
            f.write("\n# bench.py line of the same run (live HIP-event timing of the dominant kernel):\n")
            f.write(f"#   ms_per_step = {d['ms_per_step']:.4f}, tokens/s = {d['value']:.0f}, "
                    f"{fam} avg_launch_ms = {d['roofline']['avg_launch_ms']:.4f}, "
                    f"achieved = {d['roofline']['achieved']:.1f} {d['roofline']['unit']}\n")
    print(f"wrote {path}")


TIMING_LIB = os.path.join(ROOT, "adapter_mlp_amd", "liblora_mi355x_timing.so")
PHASES_LIB = os.path.join(ROOT, "adapter_mlp_amd", "liblora_mi355x_phases.so")
TIMED_BLOCKS = 8192  # block_times' second dimension in the timing build


def timing_family_names(cfg):
    """Family names of the timing build's 8 record slots for this workload."""
    act = "relu2" if cfg.kind == "relu2" else "act"
    base = [f"gemm_nn_{act}_fwd", f"gemm_nt_{act}_bwd", "gemm_nt_store", "gemm_nn_store"]
    return base + [n + "_nf4" for n in base]


def block_timing_report(rec, name, tile_mfma_cycles=2048):
    """Per-launch summary of one family's block records (the latest launch).

    rec: [blocks, 8] uint64 rows (real-time stamps at entry, K-loop start,
    K-loop end and epilogue end in 10 ns units; shader clock at entry and
    exit; hardware ids; grid size | K steps << 32).  The K loop's MFMA issue
    fraction is the ideal cycles of one 256 x 256 x 64 step per SIMD (two
    wavefronts x 64 MFMAs x 16 cycles in the dense kernels, 32 x 32 cycles in
    the NF4 kernels) over the measured cycles per step."""
    import numpy as np

    rec = rec.astype(np.int64)
    written = rec[:, 0] != 0
    if not written.any():
        return None
    # every block of the latest launch (the one that started last) rewrote its slot
    last = rec[written][np.argmax(rec[written, 0])]
    grid = min(int(last[7] & 0xFFFFFFFF), len(rec))
    rec = rec[:grid]
    kt = (rec[:, 7] >> 32).astype(np.int64)
    pro = (rec[:, 1] - rec[:, 0]) / 100.0
    loop = (rec[:, 2] - rec[:, 1]) / 100.0
    epi = (rec[:, 3] - rec[:, 2]) / 100.0
    life = (rec[:, 3] - rec[:, 0]) / 100.0
    ghz = (rec[:, 5] - rec[:, 4]) / np.maximum(life, 1e-3) / 1e3
    cyc_step = loop * ghz * 1e3 / np.maximum(kt, 1)
    hw = rec[:, 6] & 0xFFFFFFFF
    xcc = rec[:, 6] >> 32
    cu = xcc * 4096 + (hw >> 8)  # XCC, then cu/sh/se bits of HW_ID
    gaps = []
    per_cu = {}
    for k in np.unique(cu):
        idx = np.where(cu == k)[0]
        idx = idx[np.argsort(rec[idx, 0])]
        per_cu[int(k)] = len(idx)
        gaps += [(rec[b, 0] - rec[a, 3]) / 100.0 for a, b in zip(idx[:-1], idx[1:])]
    span = (rec[:, 3].max() - rec[:, 0].min()) / 100.0
    tiles = float(np.median(list(per_cu.values())))
    gap = float(np.mean(gaps)) if gaps else 0.0
    return {
        "family": name, "blocks": int(len(rec)), "grid": grid, "k_steps": int(np.median(kt)),
        "span_us": float(span), "cus": len(per_cu), "tiles_per_cu": tiles,
        "prologue_us": float(pro.mean()), "k_loop_us": float(loop.mean()), "epilogue_us": float(epi.mean()),
        "gap_between_blocks_us": gap, "clock_GHz": float(ghz.mean()),
        "cycles_per_k_step": float(cyc_step.mean()),
        "k_loop_mfma_issue_frac": float(tile_mfma_cycles / cyc_step.mean()),
        "k_loop_share_of_cu_time": float(loop.sum() / (pro.sum() + loop.sum() + epi.sum() + max(sum(gaps), 0.0))),
    }


def block_timing(args):
    """Run the workload on the per-block timing build and summarise where each
    GEMM family's time goes: prologue (entry to the first MFMA phase), K loop,
    epilogue, the gap before the next block on the same CU, and the K loop's
    cycles per step at the clock the blocks measured.  Writes
    profiles/<family>_<workload>_block_timing.txt."""
    import ctypes

    import numpy as np
    import torch

    import adapter_mlp_amd as lm
    from workload import CONFIGS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if not os.path.exists(TIMING_LIB):
        raise SystemExit(f"{TIMING_LIB} is missing: build it with `python -m adapter_mlp_amd.build --timing`")
    lib = lm.load(TIMING_LIB)
    cfg = CONFIGS[args.config]
    inp = make_inputs(cfg)
    step = {"mlp": MlpStep, "relu2": Relu2Step, "attn": AttnStep}[cfg.kind](cfg, inp, lm, torch)
    for _ in range(max(args.warmup, 1) + max(args.steps, 1)):
        step()
    torch.cuda.synchronize()
    buf = np.zeros((8, TIMED_BLOCKS, 8), dtype=np.uint64)
    fetch = lib.lora_block_times
    fetch.restype = ctypes.c_int
    fetch.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    rc = fetch(buf.ctypes.data, buf.nbytes)
    if rc != 0:
        raise SystemExit(f"lora_block_times returned HIP error {rc}")
    names = timing_family_names(cfg)
    cmd = (f"python3 bench.py --config {cfg.cid} --block-timing --steps {args.steps} --warmup {args.warmup}")
    for f in range(8):
        r = block_timing_report(buf[f], names[f])
        if r is None:
            continue
        lines = [f"# per-block timing of {names[f]}, workload {cfg.note}, latest launch after "
                 f"{max(args.warmup, 1) + max(args.steps, 1)} steps",
                 "# timing build of the library (-DLORA_BLOCK_TIMING): wavefront 0 of each block records the",
                 "# 100 MHz real-time clock at entry, at the start and the end of its K loop and after the",
                 "# epilogue, and the shader clock (s_memtime) at entry and exit",
                 f"#   python -m adapter_mlp_amd.build --timing && {cmd}",
                 "# k_loop_mfma_issue_frac = 2048 (two wavefronts x one K step's MFMAs per SIMD: 64 x 16 cycles",
                 "#   (16x16x32, dense kernels) or 32 x 32 cycles (32x32x16, NF4 kernels))",
                 "#   / measured shader cycles per K step",
                 f"source_digest = {source_digest()}"]
        if names[f].endswith("_nf4"):
            lines.insert(-1, "# NF4 kernels spill 2-5 scalar registers in the timing build (held stamps), so these figures "
                             "run slower than the normal build's kernel trace")
        lines += [f"{k} = {v:.4g}" if isinstance(v, float) else f"{k} = {v}" for k, v in r.items()]
        text = "\n".join(lines) + "\n"
        path = os.path.join(ROOT, "profiles", f"{names[f]}_{workload_tag(cfg)}_block_timing.txt")
        with open(path, "w") as fh:
            fh.write(text)
        print(f"{names[f]:24s} span {r['span_us']:8.1f} us  tiles/CU {r['tiles_per_cu']:4.1f}  "
              f"prologue {r['prologue_us']:6.2f}  K loop {r['k_loop_us']:8.2f}  epilogue {r['epilogue_us']:6.2f}  "
              f"gap {r['gap_between_blocks_us']:5.2f} us  clock {r['clock_GHz']:.3f} GHz  "
              f"{r['cycles_per_k_step']:.0f} cycles/step ({100 * r['k_loop_mfma_issue_frac']:.1f}% MFMA issue)",
              flush=True)


def phase_timing_report(rec, name):
    """Summary of one family's phase records ([64 blocks, 2 groups, 8] uint64,
    shader-clock stamps of one K step: group 0 = MFMA start, MFMA end, after its
    load wait, read start, read end; group 1 = read start, read end, MFMA
    start, MFMA end; word 5 = the next step's start, 6 = K steps)."""
    import numpy as np

    rec = rec.astype(np.int64)
    ok = (rec[:, 0, 0] != 0) & (rec[:, 1, 0] != 0) & (rec[:, 0, 5] > rec[:, 0, 0]) & (rec[:, 1, 5] > rec[:, 1, 0])
    if not ok.any():
        return None
    g0, g1 = rec[ok, 0], rec[ok, 1]
    m = lambda a: float(np.mean(a))  # noqa: E731
    return {
        "family": name, "blocks": int(ok.sum()), "k_steps": int(np.median(g0[:, 6])),
        "cycles_per_k_step": m(g0[:, 5] - g0[:, 0]),
        "g0_mfma": m(g0[:, 1] - g0[:, 0]), "g0_load_wait": m(g0[:, 2] - g0[:, 1]),
        "g0_barrier_after_mfma": m(g0[:, 3] - g0[:, 2]), "g0_read": m(g0[:, 4] - g0[:, 3]),
        "g0_barrier_after_read": m(g0[:, 5] - g0[:, 4]),
        "g1_read": m(g1[:, 1] - g1[:, 0]), "g1_barrier_after_read": m(g1[:, 2] - g1[:, 1]),
        "g1_mfma": m(g1[:, 3] - g1[:, 2]), "g1_barrier_after_mfma": m(g1[:, 5] - g1[:, 3]),
    }


def phase_timing(args):
    """Run the workload on the phase-timing build and summarise one K step of
    the first 64 blocks of each GEMM family: how long each group's MFMA
    cluster and read phase take and how long each waits at the barriers, in
    shader cycles.  Writes profiles/<family>_<workload>_phase_timing.txt."""
    import ctypes

    import numpy as np
    import torch

    import adapter_mlp_amd as lm
    from workload import CONFIGS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if not os.path.exists(PHASES_LIB):
        raise SystemExit(f"{PHASES_LIB} is missing: build it with `python -m adapter_mlp_amd.build --phases`")
    lib = lm.load(PHASES_LIB)
    cfg = CONFIGS[args.config]
    step = {"mlp": MlpStep, "relu2": Relu2Step, "attn": AttnStep}[cfg.kind](cfg, make_inputs(cfg), lm, torch)
    for _ in range(max(args.warmup, 1) + max(args.steps, 1)):
        step()
    torch.cuda.synchronize()
    buf = np.zeros((8, 64, 2, 8), dtype=np.uint64)
    fetch = lib.lora_phase_times
    fetch.restype = ctypes.c_int
    fetch.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    rc = fetch(buf.ctypes.data, buf.nbytes)
    if rc != 0:
        raise SystemExit(f"lora_phase_times returned HIP error {rc}")
    names = timing_family_names(cfg)
    cmd = f"python3 bench.py --config {cfg.cid} --phase-timing --steps {args.steps} --warmup {args.warmup}"
    for f in range(8):
        r = phase_timing_report(buf[f], names[f])
        if r is None:
            continue
        lines = [f"# per-phase timing of {names[f]}, workload {cfg.note}: K step 21 of blocks 0-63 of the latest launch",
                 "# phase-timing build of the library (-DLORA_PHASE_TIMING): lane 0 of the first wavefront of each",
                 "# group reads the shader clock (s_memtime) at every phase boundary; its stamps change that build's",
                 "# register allocation (scratch and spilled registers), so its K steps run a little slower",
                 f"#   python -m adapter_mlp_amd.build --phases && {cmd}",
                 "# cycles; an MFMA cluster issues one K step's MFMAs (64 of 16x16x32 in the dense kernels,",
                 "#   32 of 32x32x16 in the NF4 kernels; 1024 cycles at full rate)",
                 f"source_digest = {source_digest()}"]
        lines += [f"{k} = {v:.1f}" if isinstance(v, float) else f"{k} = {v}" for k, v in r.items()]
        with open(os.path.join(ROOT, "profiles", f"{names[f]}_{workload_tag(cfg)}_phase_timing.txt"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"{names[f]:24s} {r['cycles_per_k_step']:6.0f} cycles/step  g0: MFMA {r['g0_mfma']:5.0f} "
              f"wait {r['g0_load_wait']:4.0f} barrier {r['g0_barrier_after_mfma']:4.0f} read {r['g0_read']:5.0f} "
              f"barrier {r['g0_barrier_after_read']:4.0f} | g1: read {r['g1_read']:5.0f} barrier "
              f"{r['g1_barrier_after_read']:4.0f} MFMA {r['g1_mfma']:5.0f} barrier {r['g1_barrier_after_mfma']:4.0f}",
              flush=True)


def workload_tag(cfg):
    return {1: "tiny_fp32_mlp", 2: "llama3_8b_mlp", 3: "gemma_geglu_mlp", 4: "llama3_8b_qlora_mlp", 5: "llama3_8b_qkvo",
            6: "nemotron_h_relu2_mlp"}[cfg.cid]


def source_digest():
    h = hashlib.sha256()
    for f in ("gemm_bf16.hip", "common.hpp"):
        with open(os.path.join(ROOT, "adapter_mlp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, tag):
    """HBM bytes per launch from the committed PMC summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def nf4_bytes(rows, cols):
    """Bytes of one NF4 weight: codes (2 per byte), int8 scale codes per 64
    elements, fp32 second-level scales per 64 x 256 elements, the fp32 mean."""
    n = rows * cols
    return n // 2 + n // 64 + 4 * (n // (64 * 256)) + 4


def nf4_report(cfg, step, lm, torch, reps=5):
    """QLoRA extras: per NF4 GEMM family, the packed weight bytes it reads
    once per launch over its average launch time (the weight stream rate),
    and the standalone dequant kernel (codes + scales in, bf16 out) against
    HBM, timed on the gate weight."""
    H, I = cfg.H, cfg.I
    w = {"gemm_nn_act_fwd_nf4": 2 * nf4_bytes(H, I), "gemm_nn_store_nf4": nf4_bytes(I, H),
         "gemm_nt_act_bwd_nf4": nf4_bytes(I, H), "gemm_nt_store_nf4": 2 * nf4_bytes(H, I)}
    lm.trace_begin("gemm")
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    fams = lm.trace_end()
    stream = {}
    for fam, b in w.items():
        if fam in fams:
            ms = fams[fam][1] / fams[fam][0]
            stream[fam] = {"weight_bytes": b, "avg_launch_ms": ms, "GB_s": b / (ms / 1e3) / 1e9}
    q = step.p["gate"].nf4
    out = torch.empty((H, I), dtype=torch.bfloat16, device="cuda:0")
    lm.nf4_dequant(q, torch.bfloat16, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        lm.nf4_dequant(q, torch.bfloat16, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    moved = nf4_bytes(H, I) + 2 * H * I
    return {"weight_stream": stream,
            "dequant": {"shape": [H, I], "bytes": moved, "ms": ms, "GB_s": moved / (ms / 1e3) / 1e9,
                        "hbm_frac": moved / (ms / 1e3) / (PEAK_HBM_GBS * 1e9)}}


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def with_wt(step):
    """Give every dense bf16 projection of a step the K-contiguous copy of its
    frozen weight, Wt = W^T ([n_out, n_in]); the library's forward GEMMs then
    read Wt, the backward ones W."""
    for p in step.p.values():
        if p.W is not None and p.nf4 is None and p.W.element_size() == 2:
            p.Wt = p.W.t().contiguous()
    return step


class MlpStep:
    def __init__(self, cfg, inp, lm, torch):
        self.cfg, self.lm = cfg, lm
        cdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        dev = lambda a: torch.from_numpy(a).to("cuda:0").to(cdt)  # noqa: E731
        adt = torch.float32 if cfg.lora_dtype == "f32" else cdt
        adev = lambda a: torch.from_numpy(a).to("cuda:0").to(adt)  # noqa: E731
        self.X, self.dY = dev(inp["X"]), dev(inp["dY"])
        self.p = {}
        for k in ("gate", "up", "down"):
            nf4 = None
            if cfg.nf4:
                nf4 = lm.nf4_quantize(dev(inp[k]["W"]))
            self.p[k] = lm.Proj(A=adev(inp[k]["A"]), B=adev(inp[k]["B"]), scale=inp[k]["s"],
                                W=None if cfg.nf4 else dev(inp[k]["W"]), nf4=nf4)
        T, H, I, r = cfg.T, cfg.H, cfg.I, cfg.r
        fb, bb = lm.mlp_workspace_size(T, H, I, r, cfg.act, lm._call_dtype(self.X, list(self.p.values())))
        bf = cdt
        self.Y = torch.empty((T, H), dtype=bf, device="cuda:0")
        self.saved = dict(e=torch.empty((T, I), dtype=bf, device="cuda:0"),
                          g=torch.empty((T, I), dtype=bf, device="cuda:0"),
                          U=torch.empty((T, 3 * r), dtype=bf, device="cuda:0"))
        self.dX = torch.empty_like(self.X)
        self.grads = {n: torch.empty_like(getattr(self.p[k], m)) for n, k, m in
                      (("dA_gate", "gate", "A"), ("dB_gate", "gate", "B"), ("dA_up", "up", "A"),
                       ("dB_up", "up", "B"), ("dA_down", "down", "A"), ("dB_down", "down", "B"))}
        self.wsf = torch.empty(fb, dtype=torch.uint8, device="cuda:0")
        self.wsb = torch.empty(bb, dtype=torch.uint8, device="cuda:0")

    def __call__(self):
        lm, p = self.lm, self.p
        lm.mlp_fwd(self.X, p["gate"], p["up"], p["down"], self.cfg.act, Y=self.Y, saved=self.saved, ws=self.wsf)
        lm.mlp_bwd(self.dY, self.X, self.saved, p["gate"], p["up"], p["down"], self.cfg.act, dX=self.dX,
                   grads=self.grads, ws=self.wsb)


class Relu2Step:
    def __init__(self, cfg, inp, lm, torch):
        self.cfg, self.lm = cfg, lm
        dev = lambda a: torch.from_numpy(a).to("cuda:0").to(torch.bfloat16)  # noqa: E731
        adt = torch.float32 if cfg.lora_dtype == "f32" else torch.bfloat16
        adev = lambda a: torch.from_numpy(a).to("cuda:0").to(adt)  # noqa: E731
        self.X, self.dY = dev(inp["X"]), dev(inp["dY"])
        self.p = {k: lm.Proj(A=adev(inp[k]["A"]), B=adev(inp[k]["B"]), scale=inp[k]["s"], W=dev(inp[k]["W"]))
                  for k in ("up", "down")}
        T, H, I, r = cfg.T, cfg.H, cfg.I, cfg.r
        fb, bb = lm.relu2_mlp_workspace_size(T, H, I, r, lm._call_dtype(self.X, list(self.p.values())))
        bf = torch.bfloat16
        self.Y = torch.empty((T, H), dtype=bf, device="cuda:0")
        self.saved = dict(u=torch.empty((T, I), dtype=bf, device="cuda:0"),
                          U=torch.empty((T, 2 * r), dtype=bf, device="cuda:0"))
        self.dX = torch.empty_like(self.X)
        self.grads = {n: torch.empty_like(getattr(self.p[k], m)) for n, k, m in
                      (("dA_up", "up", "A"), ("dB_up", "up", "B"), ("dA_down", "down", "A"),
                       ("dB_down", "down", "B"))}
        self.wsf = torch.empty(fb, dtype=torch.uint8, device="cuda:0")
        self.wsb = torch.empty(bb, dtype=torch.uint8, device="cuda:0")

    def __call__(self):
        lm, p = self.lm, self.p
        lm.relu2_mlp_fwd(self.X, p["up"], p["down"], Y=self.Y, saved=self.saved, ws=self.wsf)
        lm.relu2_mlp_bwd(self.dY, self.X, self.saved, p["up"], p["down"], dX=self.dX, grads=self.grads,
                         ws=self.wsb)


class AttnStep:
    def __init__(self, cfg, inp, lm, torch):
        self.cfg, self.lm = cfg, lm
        dev = lambda a: torch.from_numpy(a).to("cuda:0").to(torch.bfloat16)  # noqa: E731
        adt = torch.float32 if cfg.lora_dtype == "f32" else torch.bfloat16
        adev = lambda a: torch.from_numpy(a).to("cuda:0").to(adt)  # noqa: E731
        self.t = {k: dev(inp[k]) for k in ("X", "Xo", "dQ", "dK", "dV", "dO")}
        self.p = {k: lm.Proj(A=adev(inp[k]["A"]), B=adev(inp[k]["B"]), scale=inp[k]["s"], W=dev(inp[k]["W"]))
                  for k in ("q", "k", "v", "o")}
        T, H, r = cfg.T, cfg.H, cfg.r
        bf = torch.bfloat16
        self.qkv = [torch.empty((T, n), dtype=bf, device="cuda:0") for n in (cfg.Nq, cfg.Nk, cfg.Nv)]
        self.U = torch.empty((T, 3 * r), dtype=bf, device="cuda:0")
        self.Yo = torch.empty((T, H), dtype=bf, device="cuda:0")
        self.Uo = torch.empty((T, r), dtype=bf, device="cuda:0")
        self.dX = torch.empty_like(self.t["X"])
        self.dXo = torch.empty_like(self.t["Xo"])
        self.g = {n: torch.empty_like(getattr(self.p[k], m)) for n, k, m in
                  (("dA_q", "q", "A"), ("dB_q", "q", "B"), ("dA_k", "k", "A"), ("dB_k", "k", "B"),
                   ("dA_v", "v", "A"), ("dB_v", "v", "B"))}
        self.dAo = torch.empty_like(self.p["o"].A)
        self.dBo = torch.empty_like(self.p["o"].B)

    def __call__(self):
        lm, p, t = self.lm, self.p, self.t
        lm.qkv_fwd(t["X"], p["q"], p["k"], p["v"], out=self.qkv, U=self.U)
        lm.o_fwd(t["Xo"], p["o"], Y=self.Yo, U=self.Uo)
        lm.o_bwd(t["dO"], t["Xo"], self.Uo, p["o"], dX=self.dXo, dA=self.dAo, dB=self.dBo)
        lm.qkv_bwd(t["dQ"], t["dK"], t["dV"], t["X"], self.U, p["q"], p["k"], p["v"], dX=self.dX, grads=self.g)


def cpu_baseline(cfg, inp, seconds):
    """The oracle as it stands, on the first Ts tokens of the same inputs."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import lora as OL
    from oracle import nf4 as ON

    if cfg.kind == "mlp":
        projs = {k: inp[k] for k in ("gate", "up", "down")}
        if cfg.nf4:  # the QLoRA oracle: the dense oracle on the dequantized base
            projs = {k: dict(v, W=ON.dequantize(ON.quantize(v["W"]), "bf16")) for k, v in projs.items()}

        def run(ts):
            X, dY = inp["X"][:ts], inp["dY"][:ts]
            Y, s = OL.mlp_fwd(X, projs["gate"], projs["up"], projs["down"], cfg.act)
            OL.mlp_bwd(dY, X, s, projs["gate"], projs["up"], projs["down"], cfg.act)
    elif cfg.kind == "relu2":
        def run(ts):
            X, dY = inp["X"][:ts], inp["dY"][:ts]
            Y, s = OL.relu2_mlp_fwd(X, inp["up"], inp["down"])
            OL.relu2_mlp_bwd(dY, X, s, inp["up"], inp["down"])
    else:
        def run(ts):
            X, Xo = inp["X"][:ts], inp["Xo"][:ts]
            (_, _, _), s = OL.qkv_fwd(X, inp["q"], inp["k"], inp["v"])
            _, so = OL.o_fwd(Xo, inp["o"])
            OL.o_bwd(inp["dO"][:ts], Xo, so, inp["o"])
            OL.qkv_bwd(inp["dQ"][:ts], inp["dK"][:ts], inp["dV"][:ts], X, s, inp["q"], inp["k"], inp["v"])

    ts = min(128, cfg.T)
    t0 = time.perf_counter()
    run(ts)
    probe = time.perf_counter() - t0
    ts = int(max(128, min(cfg.T, (seconds / max(probe, 1e-3)) * ts)) // 128 * 128)
    t0 = time.perf_counter()
    run(ts)
    dt = time.perf_counter() - t0
    reps = 1
    # when the whole workload takes less than the target, pass over it again
    # (at most 10 passes) so the timed CPU work still lasts about `seconds`
    if ts >= cfg.T and dt < 0.75 * seconds:
        extra = min(9, int(round(seconds / max(dt, 1e-3))) - 1)
        t1 = time.perf_counter()
        for _ in range(extra):
            run(ts)
        dt += time.perf_counter() - t1
        reps += extra
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("internal_api") == "openblas"]
                  or [1])
    what = f"{reps} passes over all {cfg.T} tokens" if reps > 1 else f"first {ts} of {cfg.T} tokens"
    return {"value": reps * ts / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what}, full-size weights, fp32 numpy oracle fwd+bwd ({dt:.1f} s)",
            "seconds": round(dt, 2), "cpu_count": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def cpu_model():
    """The host CPU's model name as /proc/cpuinfo gives it."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--lora-dtype", default="bf16", choices=["bf16", "f32"],
                    help="f32: fp32 adapters and adapter gradients with bf16 inputs (fp32 LoRA-gradient mode)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-family-times", action="store_true",
                    help="skip the 5 extra traced steps that time every kernel family")
    ap.add_argument("--wt", action="store_true",
                    help="also pass each dense bf16 base weight as W^T, so the forward GEMMs read it K-contiguous")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter files into profiles/*_traffic.txt")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="no GPU run: turn rocprofv3 --pmc runs of the MFMA and LDS counter sets into "
                         "profiles/*_counters.txt")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="no GPU run: turn a rocprofv3 --kernel-trace --stats run into profiles/*_kernel_trace.txt")
    ap.add_argument("--block-timing", action="store_true",
                    help="run on the per-block timing build (liblora_mi355x_timing.so) and write "
                         "profiles/*_block_timing.txt: prologue, K loop, epilogue and clock per GEMM family")
    ap.add_argument("--phase-timing", action="store_true",
                    help="run on the per-phase timing build (liblora_mi355x_phases.so) and write "
                         "profiles/*_phase_timing.txt: MFMA cluster, read phase and barrier waits of one K step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run a plain fp32 elementwise copy (negation) of MIB MiB "
                         "three times, the known-size kernel that scales HBM byte counters")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.config)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary[0], args.trace_summary[1], args.config)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.config)
        return
    if args.block_timing:
        block_timing(args)
        return
    if args.phase_timing:
        phase_timing(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused LoRA path runs on a single MI355X here and "
              "--gpus N with N > 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    import adapter_mlp_amd as lm
    from workload import CONFIGS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lm.load()
    cfg = CONFIGS[args.config]
    if args.lora_dtype == "f32":
        cfg = cfg.with_(lora_dtype="f32")
    log(f"[bench] config {cfg.cid}: {cfg.note}; adapters {args.lora_dtype}; generating seeded inputs")
    t0 = time.time()
    inp = make_inputs(cfg)
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    step = {"mlp": MlpStep, "relu2": Relu2Step, "attn": AttnStep}[cfg.kind](cfg, inp, lm, torch)
    if args.wt:
        with_wt(step)
    torch.cuda.synchronize()

    # W warm-up steps; the second one (the first is cold: code loading and
    # first-touch costs can outweigh a whole small GEMM), or the only one,
    # finds the dominant GEMM family
    if args.warmup >= 2:
        step()
        torch.cuda.synchronize()
    lm.trace_begin("")
    step()
    torch.cuda.synchronize()
    fams = lm.trace_end()
    for _ in range(max(args.warmup - 2, 0)):
        step()
    torch.cuda.synchronize()
    gemms = {k: v for k, v in fams.items() if k.startswith("gemm")}
    dominant = max(gemms, key=lambda k: gemms[k][1])
    log("[bench] warm-up per-family ms: " + ", ".join(f"{k}={v[1]:.3f}" for k, v in fams.items()))

    # timed region: only the dominant family carries event pairs
    lm.trace_begin(dominant)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    traced = lm.trace_end()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    tokens_s = cfg.T / (ms_step / 1e3)
    tflops = cfg.flops() / (ms_step / 1e3) / 1e12
    launches, kms = traced.get(dominant, (0, 0.0))
    avg_ms = kms / max(launches, 1)
    fl = kernel_flops(cfg, dominant)
    achieved = fl / (avg_ms / 1e3) / 1e12 if fl and avg_ms > 0 else None
    # the committed traffic profiles were taken with W only
    traffic = None if args.wt else read_traffic(dominant, workload_tag(cfg))
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step ({wall / args.steps * 1e3:.3f} ms wall), "
        f"{tokens_s:,.0f} tokens/s, {tflops:.1f} TFLOP/s; {dominant}: {avg_ms:.3f} ms/launch")

    # every kernel family's launch time, from 5 more steps with all families
    # traced (after the timed region, which they do not touch)
    per_family = {}
    if not args.no_family_times:
        n_fam = 5
        lm.trace_begin("")
        for _ in range(n_fam):
            step()
        torch.cuda.synchronize()
        for k, (n, t) in lm.trace_end().items():
            per_family[k] = {"launches_per_step": n / n_fam, "avg_ms": t / max(n, 1)}

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x neg over {args.copy_calibration} MiB fp32 "
            f"(reads {n * 4} B, writes {n * 4} B per launch)")
        del src, dst

    nf4 = nf4_report(cfg, step, lm, torch) if cfg.nf4 else None
    f32 = cfg.dtype == "f32"
    peak = PEAK_F32_VALU_TFLOPS if f32 else PEAK_BF16_TFLOPS

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a token sample")
        cpu = cpu_baseline(cfg, inp, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads ({cpu['sample']})")

    out = {
        "metric": {"mlp": "LoRA-MLP fwd+bwd tokens/s at Llama-3-8B MLP shape; % bf16 MFMA peak",
                   "relu2": "ReLU^2 LoRA-MLP fwd+bwd tokens/s at a Nemotron-H-8B-like MLP shape",
                   "attn": "LoRA QKV+O fwd+bwd tokens/s at Llama-3-8B attention shapes"}[cfg.kind],
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic (seeded; random-init weights and adapters of the named shapes)",
        "config": {"workload": cfg.note, "tokens": cfg.T, "hidden": cfg.H,
                   **({"intermediate": cfg.I, "activation": cfg.act} if cfg.kind == "mlp"
                      else {"intermediate": cfg.I, "activation": "relu2"} if cfg.kind == "relu2"
                      else {"q": cfg.Nq, "k": cfg.Nk, "v": cfg.Nv, "o": [cfg.Nq, cfg.H]}),
                   "rank": cfg.r, "alpha": cfg.alpha, "base": "nf4" if cfg.nf4 else "bf16",
                   **({"base_layout": "W [in, out] and W^T [out, in] (forward GEMMs read W^T)"} if args.wt
                      else {}),
                   "adapters": args.lora_dtype,
                   "parallelism": "single GPU"},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        # the fp32 path runs on fp32 FMAs (no MFMA): its bound is the vector ALU peak
        "roofline": {"bound": "alu" if f32 else "mfma", "kernel": dominant, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": (achieved / peak) if achieved else None,
                     "traffic": traffic, "flops_per_launch": fl, "avg_launch_ms": avg_ms,
                     "launches_timed": launches},
        "cpu_baseline": cpu,
        "kernel_families": per_family,
    }
    if nf4:
        out["nf4"] = nf4
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
