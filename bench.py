"""Throughput of one training step (forward, backward, clip + AdamW) on one GPU.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4] [--no-cpu]

Default workload: the GPT-2-small-shaped step (vocab 50257, d_model 768,
12 heads of 64, MLP 3072, 12 pre-LN blocks, seq 1024, batch 8, causal mask,
bf16 operands with fp32 master weights), on seeded synthetic tokens with a
Zipf(1.1) id law and random-init weights (no dataset or checkpoint exists
here). Inputs are resident in HBM before timing starts.

Prints one JSON line: tokens/s over K timed steps (W untimed warm-up steps
first; each timed region is bracketed by a device synchronisation), MFMA
utilisation of the GEMM + attention kernels, the roofline of the dominant
kernel from per-launch HIP events recorded on the step's stream in a second
pass of K steps, and the CPU oracle timed on a bounded sample of the same
workload as a baseline.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "training tokens/sec (fwd+bwd+AdamW) on 1 MI355X; MFMA util % of peak"
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    "C1": "tiny byte-level GPT, fp32: V=257, d=128, 4x32 heads, MLP 256, 3 blocks, seq 80, batch 4",
    "C2": "small byte-level GPT, bf16: V=257, d=256, 8x32 heads, MLP 1024, 4 blocks, seq 256, batch 16",
    "C3": "packed-SFT GPT (~1.9M params), bf16: V=8000, d=128, 4x32, MLP 512, 4 blocks, seq 512, batch 32, "
          "packed docs 20..200, block-diagonal mask",
    "C4": "GPT-2-small-shaped step, bf16/fp32 master: V=50257, d=768, 12x64 heads, MLP 3072, 12 blocks, "
          "seq 1024, batch 8, causal",
    "C5": "~30M-param subword GPT, bf16: V=16384, d=512, 8x64, MLP 2048, 8 blocks, seq 2048, batch 16, "
          "packed docs log-uniform 64..2048",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(shape, doc_ids, B, T):
    """Algorithmic attention flops per step: 12 * D * H * L * pairs, pairs =
    allowed (query, key) pairs over non-pad queries (forward 4 D per pair,
    backward 8 D per pair)."""
    pairs = 0
    for b in range(B):
        if doc_ids is None:
            pairs += T * (T + 1) // 2
        else:
            _, counts = np.unique(doc_ids[b], return_counts=True)
            pairs += int(sum(c * (c + 1) // 2 for c in counts))
    return 12.0 * shape.head_dim * shape.n_heads * shape.n_layers * pairs


# Kernel symbol of each timing class whose HBM traffic is taken from counters:
# a class maps to one kernel instantiation used by nothing else, or to
# (symbol, period, phase) when several classes share an instantiation in a
# fixed order: the class takes that kernel's dispatches whose index, in
# dispatch order, is phase modulo period (the attention-output and MLP-out
# forward GEMMs share the residual-epilogue kernel and alternate, attention
# output first, in every block). The blocks' weight gradients run as one
# grouped launch after the backward (gemm_dw_group).
TRAFFIC_SYMBOLS = {
    "gemm_head_bwd_dw": "gemm16_pipe_kernel<256, 256, 2, 4, 64, 2, 2, false, false, 4, float,",
    "gemm_head_fwd": "gemm16_pipe_kernel<256, 256, 2, 4, 64, 2, 2, true, true, 0,",
    "gemm_fc1_fwd": "gemm16_pipe_kernel<128, 128, 2, 2, 64, 2, 2, true, true, 2,",
    "gemm_fc2_bwd_dx": "gemm16_pipe_kernel<128, 128, 2, 2, 64, 2, 2, true, false, 3,",
    "gemm_qkv_fwd": "gemm16_pipe_kernel<192, 128, 2, 2, 64, 2, 2, true, true, 0,",
    "adamw": "adamw_kernel(",
    "gemm_attnout_fwd": ("gemm16_ksplit_kernel<3, 4, true, true, 1, float,", 2, 0),
    "gemm_fc2_fwd": ("gemm16_ksplit_kernel<3, 4, true, true, 1, float,", 2, 1),
    "gemm_dw_group": "gemm16_ksplit_kernel<3, 4, false, false, 4, float, unsigned short, true>",
    "attn_bwd_dkv": "attn_dkv_kernel<64, unsigned short>",
    "attn_bwd_dq": "attn_dq_kernel<64, unsigned short>",
    "attn_fwd": "attn_fwd_kernel<64, unsigned short>",
    "layernorm_fwd": "ln_fwd_kernel<6, unsigned short>",
    "layernorm_bwd": "ln_bwd_kernel<6, unsigned short>",
    "xent": "xent_reg_kernel<unsigned short,",
}
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters_c4_step.md")
SIMDS = 1024  # 256 compute units x 4 SIMDs
XCDS = 8  # accelerator complex dies (32 compute units each)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_c4_step.md")
CALIB_BYTES = 1 << 30  # plain device copy used to scale the counters


def source_digest():
    """Hash of the kernel sources; counters taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "scratch_decoder_only_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def pmc_summary(fetch_dir, write_dir, out=TRAFFIC_FILE, cmd=""):
    """Per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch) from two rocprofv3
    --pmc runs, scaled by what the same counters read for the calibration copy
    of CALIB_BYTES bytes; writes the summary with its machine-readable record."""
    import csv
    import glob

    def read(d, counter):
        """kernel name -> [(dispatch id, value)] in dispatch order"""
        acc = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                acc.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        return {k: [v for _, v in sorted(x)] for k, x in acc.items()}

    fetch_all, write_all = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")

    def mean_of(vals, period, phase):
        sel = vals[phase::period]
        return (sum(sel) / len(sel), len(sel)) if sel else (0.0, 0)
    # the calibration copy: the largest dispatch of a copy kernel (it moves
    # more bytes than any other copy of the run)
    cal = [(max(v), k) for k, v in fetch_all.items() if "copy" in k.lower()]
    if not cal:
        raise SystemExit("no calibration copy in the counter data")
    cf, ck = max(cal)
    cw = max(write_all.get(ck, [0.0]))
    f_scale = CALIB_BYTES / (cf * 1024)
    w_scale = CALIB_BYTES / (cw * 1024) if cw > 0 else 1.0
    rec = {"source_digest": source_digest(), "calib_kernel": ck, "calib_bytes": CALIB_BYTES,
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "classes": {}}
    lines = []
    for cls, spec in TRAFFIC_SYMBOLS.items():
        sym, period, phase = (spec, 1, 0) if isinstance(spec, str) else spec
        ks = [k for k in fetch_all if sym in k]
        if not ks:
            continue
        k = ks[0]
        fm, fn = mean_of(fetch_all[k], period, phase)
        wm, _ = mean_of(write_all.get(k, []), period, phase)
        fb = fm * 1024 * f_scale
        wb = wm * 1024 * w_scale
        rec["classes"][cls] = {"kernel": k, "dispatches": fn, "fetch_kib": round(fm, 1), "write_kib": round(wm, 1),
                               "bytes_per_launch": round(fb + wb)}
        lines.append(f"| {cls} | `{k[:90]}` | {fn} | {fm:.1f} | {wm:.1f} | {(fb + wb) / 1e6:.2f} |")
    with open(out, "w") as fh:
        fh.write("# HBM traffic per launch from hardware counters (GPT-2-small-shaped step, C4)\n\n")
        fh.write("Commands (run from the repository root on one MI355X):\n\n```\n" + cmd + "\n```\n\n")
        fh.write(f"Calibration: `{ck[:80]}` copying {CALIB_BYTES} bytes read FETCH_SIZE {cf:.1f} KiB "
                 f"and WRITE_SIZE {cw:.1f} KiB; scale factors {f_scale:.4f} (fetch) and "
                 f"{w_scale:.4f} (write) turn counter KiB into bytes.\n\n")
        fh.write("| class | kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | "
                 "scaled MB/launch |\n|---|---|---|---|---|---|\n")
        fh.write("\n".join(lines) + "\n\n")
        fh.write("Record read by bench.py (null traffic once the kernel sources differ from source_digest):\n\n")
        fh.write("```json\n" + json.dumps(rec, indent=1) + "\n```\n")
    print(out)


def mfma_summary(pmc_dir, out=MFMA_FILE, cmd=""):
    """MFMA utilisation of the GEMM and attention kernels from one rocprofv3
    --pmc run with SQ_INSTS_VALU_MFMA_MOPS_BF16 (MFMA operations / 512),
    SQ_VALU_MFMA_BUSY_CYCLES (matrix-core busy cycles summed over the SIMDs)
    and GRBM_GUI_ACTIVE (GPU busy cycles per XCD): per kernel, the busy
    fraction = MFMA busy cycles / (GPU cycles x SIMDs), which does not depend
    on the clock, and the matrix flops the hardware executed (attention score
    recomputation included)."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            d = per.setdefault(k, {})
            c = r["Counter_Name"]
            v = float(r["Counter_Value"])
            if c == "GRBM_GUI_ACTIVE":
                d.setdefault("grbm_rows", []).append(v)
            else:
                d[c] = d.get(c, 0.0) + v
    for d in per.values():
        rows = d.pop("grbm_rows", None)
        if rows:
            # one row per XCD: the longest; one row: rocprofv3's sum over the XCDs
            d["GRBM_GUI_ACTIVE"] = max(rows) if len(rows) > 1 else rows[0] / XCDS
    by = {}
    for (_, name), d in per.items():
        if not ("gemm16" in name or "attn_" in name) or "GRBM_GUI_ACTIVE" not in d:
            continue
        e = by.setdefault(name, {"n": 0, "busy": 0.0, "gpu": 0.0, "mops": 0.0})
        e["n"] += 1
        e["busy"] += d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        e["gpu"] += d["GRBM_GUI_ACTIVE"]
        e["mops"] += d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
    if not by:
        raise SystemExit("no GEMM or attention dispatches with MFMA counters in " + pmc_dir)
    tot_busy = sum(e["busy"] for e in by.values())
    tot_gpu = sum(e["gpu"] for e in by.values())
    rec = {"source_digest": source_digest(), "busy_frac": round(tot_busy / (tot_gpu * SIMDS), 4),
           "mfma_flops": sum(e["mops"] for e in by.values()) * 512, "kernels": {}}
    lines = []
    for name, e in sorted(by.items(), key=lambda kv: -kv[1]["gpu"]):
        frac = e["busy"] / (e["gpu"] * SIMDS)
        rec["kernels"][name] = {"dispatches": e["n"], "busy_frac": round(frac, 4),
                                "mfma_flops_per_dispatch": e["mops"] * 512 / e["n"]}
        lines.append(f"| `{name[:100]}` | {e['n']} | {e['gpu'] / e['n']:.0f} | {frac:.3f} | "
                     f"{e['mops'] * 512 / e['n'] / 1e9:.2f} |")
    with open(out, "w") as fh:
        fh.write("# MFMA utilisation from hardware counters (GPT-2-small-shaped step, C4)\n\n")
        fh.write("Command (repository root, on one MI355X):\n\n```\n" + cmd + "\n```\n\n")
        fh.write("Busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GPU cycles per XCD x "
                 f"{SIMDS} SIMDs), GPU cycles per XCD = GRBM_GUI_ACTIVE / {XCDS} (rocprofv3 reports it summed "
                 "over the XCDs): the share of the kernel's GPU cycles in which the matrix cores were "
                 "busy, whatever the clock ran at. MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the "
                 "attention kernels' score recomputation included).\n\n")
        fh.write(f"All GEMM and attention dispatches: busy fraction **{rec['busy_frac']:.3f}** "
                 "(cycle-weighted).\n\n")
        fh.write("| kernel | dispatches | GPU cycles / dispatch | MFMA busy | MFMA GFLOP / dispatch |\n"
                 "|---|---:|---:|---:|---:|\n")
        fh.write("\n".join(lines) + "\n\n")
        fh.write("Record read by bench.py (ignored once the kernel sources differ from source_digest):\n\n")
        fh.write("```json\n" + json.dumps(rec, indent=1) + "\n```\n")
    print(out)


GAP_FILE = os.path.join(ROOT, "profiles", "gemm_attn_gap_c4_step.md")
GAP_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
                "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE")


def gap_summary(pmc_dir, out=GAP_FILE, cmd=""):
    """Where the GEMM and attention kernels' cycles go, from one rocprofv3
    --pmc run with GAP_COUNTERS: per kernel (summed over its dispatches), the
    matrix cores' busy share of the SIMD cycles, the vector ALU's and the LDS
    instructions' active shares (SQ_ACTIVE_INST_*, in 4-cycle units, summed
    over the SIMDs), and the share of the wavefronts' lifetime spent waiting
    for an operand (SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES, both in 4-cycle
    units). SIMD cycles = GRBM_GUI_ACTIVE / XCDS x SIMDS."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            d = per.setdefault(k, {})
            c, v = r["Counter_Name"], float(r["Counter_Value"])
            if c == "GRBM_GUI_ACTIVE":
                d.setdefault("grbm_rows", []).append(v)
            else:
                d[c] = d.get(c, 0.0) + v
    by = {}
    for (_, name), d in per.items():
        rows = d.pop("grbm_rows", None)
        if not rows or not ("gemm16" in name or "attn_" in name):
            continue
        gpu = max(rows) if len(rows) > 1 else rows[0] / XCDS
        e = by.setdefault(name, {"n": 0, "gpu": 0.0})
        e["n"] += 1
        e["gpu"] += gpu
        for c in GAP_COUNTERS[:-1]:
            e[c] = e.get(c, 0.0) + d.get(c, 0.0)
    if not by:
        raise SystemExit("no GEMM or attention dispatches with the counters in " + pmc_dir)
    lines = []
    rec = {"source_digest": source_digest(), "kernels": {}}
    for name, e in sorted(by.items(), key=lambda kv: -kv[1]["gpu"]):
        simd = e["gpu"] * SIMDS
        mfma = e["SQ_VALU_MFMA_BUSY_CYCLES"] / simd
        valu = e["SQ_ACTIVE_INST_VALU"] * 4 / simd
        lds = e["SQ_ACTIVE_INST_LDS"] * 4 / simd
        wait = e["SQ_WAIT_INST_ANY"] / e["SQ_WAVE_CYCLES"] if e["SQ_WAVE_CYCLES"] else 0.0
        vpm = (e["SQ_INSTS_VALU"] / (e["SQ_VALU_MFMA_BUSY_CYCLES"] / 32) if e["SQ_VALU_MFMA_BUSY_CYCLES"] else 0.0)
        rec["kernels"][name] = {"dispatches": e["n"], "mfma_busy": round(mfma, 3), "valu_active": round(valu, 3),
                                "lds_active": round(lds, 3), "wave_wait": round(wait, 3),
                                "valu_insts_per_mfma": round(vpm, 2)}
        lines.append(f"| `{name[:96]}` | {e['n']} | {mfma:.3f} | {valu:.3f} | {lds:.3f} | {wait:.3f} | {vpm:.1f} |")
    with open(out, "w") as fh:
        fh.write("# Where the GEMM and attention cycles go (hardware counters, GPT-2-small-shaped step, C4)\n\n")
        fh.write("Command (repository root, on one MI355X):\n\n```\n" + cmd + "\n```\n\n")
        fh.write("Per kernel, over all its dispatches of the run. SIMD cycles = GRBM_GUI_ACTIVE / "
                 f"{XCDS} XCDs (rocprofv3 sums it over them) x {SIMDS} SIMDs. *MFMA busy* = "
                 "SQ_VALU_MFMA_BUSY_CYCLES / SIMD cycles; *VALU active* and *LDS active* = SQ_ACTIVE_INST_VALU "
                 "and SQ_ACTIVE_INST_LDS (4-cycle units, summed over the SIMDs) x 4 / SIMD cycles (the VALU "
                 "share includes issuing the MFMAs); *wave wait* = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, the share "
                 "of the wavefronts' lifetime spent waiting for an operand (memory, LDS or a dependency); "
                 "*VALU / MFMA* = vector instructions (MFMAs included) per 32x32x16 MFMA.\n\n")
        fh.write("| kernel | dispatches | MFMA busy | VALU active | LDS active | wave wait | VALU / MFMA |\n"
                 "|---|---:|---:|---:|---:|---:|---:|\n")
        fh.write("\n".join(lines) + "\n\n")
        fh.write("Record (taken on the sources with this digest):\n\n```json\n" + json.dumps(rec, indent=1) +
                 "\n```\n")
    print(out)


def mfma_record():
    try:
        txt = open(MFMA_FILE).read()
        rec = json.loads(txt[txt.index("```json") + 7: txt.rindex("```")])
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    return rec


def stats_summary(stats_csv, out, cmd="", steps=7):
    """Kernel table from a rocprofv3 --stats kernel_stats.csv (Name, Calls,
    TotalDurationNs, AverageNs), sorted by total time."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    with open(out, "w") as fh:
        fh.write("# C4 training step: rocprofv3 kernel statistics\n\n")
        fh.write("Workload: " + WORKLOADS["C4"] + ", one MI355X.\n\n")
        fh.write("Command (repository root, on the GPU host):\n\n```\n" + cmd + "\n```\n\n")
        fh.write(f"The run covers {steps} training steps (warm-up + timed) plus the parameter upload; totals are "
                 f"over all of them (per-step time = total / {steps}). Source: the run's kernel_stats.csv.\n\n")
        fh.write("| kernel | calls | total ms | avg us | share |\n|---|---:|---:|---:|---:|\n")
        for r in rows:
            t = float(r["TotalDurationNs"])
            if t < 0.002 * total:
                continue
            fh.write(f"| `{r['Name'][:110]}` | {r['Calls']} | {t / 1e6:.2f} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{100 * t / total:.1f}% |\n")
        fh.write(f"\nAll kernels: {total / 1e6:.2f} ms, {total / 1e6 / steps:.3f} ms per step.\n")
        # per timing class, for the classes with hardware-counter records:
        # average dispatch duration from the run's kernel trace (a kernel
        # shared by two alternating classes is split the same way as the
        # counters)
        trace = os.path.join(os.path.dirname(stats_csv), os.path.basename(stats_csv).replace("kernel_stats",
                                                                                               "kernel_trace"))
        if os.path.exists(trace):
            durs = {}
            for r in csv.DictReader(open(trace)):
                durs.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            fh.write("\nPer timing class (dispatches of its kernel, from the kernel trace):\n\n"
                     "| class | dispatches | avg us |\n|---|---:|---:|\n")
            for cls, spec in TRAFFIC_SYMBOLS.items():
                sym, period, phase = (spec, 1, 0) if isinstance(spec, str) else spec
                ks = [k for k in durs if sym in k]
                if not ks:
                    continue
                sel = [d for _, d in sorted(durs[ks[0]])][phase::period]
                if sel:
                    fh.write(f"| {cls} | {len(sel)} | {sum(sel) / len(sel) / 1e3:.1f} |\n")
    print(out)


def traffic_of(cls):
    """Counter-based HBM bytes per launch of a timing class, or None (no record,
    or taken on different kernel sources)."""
    try:
        txt = open(TRAFFIC_FILE).read()
        rec = json.loads(txt[txt.index("```json") + 7: txt.rindex("```")])
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest() or cls not in rec.get("classes", {}):
        return None
    return rec["classes"][cls]["bytes_per_launch"]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    """Threads numpy's BLAS runs its products on (what the oracle's matmuls use)."""
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return int(os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or os.cpu_count())


def cpu_baseline(shape, batch=1):
    """The oracle (float64 numpy, untuned) on a bounded sample of the workload:
    one full step at `batch` rows (default 1; same width, depth, vocabulary and
    sequence). A full GPT-2-small-shaped batch of 8 rows takes about a minute
    on 16 host threads, beyond what the default run should spend on the
    baseline; --cpu-batch 8 times it."""
    import oracle
    import synth
    sample = shape.with_batch(batch)
    b = synth.make_batch(sample)
    params = synth.init_params(sample)
    zeros = {k: np.zeros_like(v, dtype=np.float64) for k, v in params.items()}
    t0 = time.perf_counter()
    oracle.train_step(params, zeros, zeros, sample, b.tokens, b.targets, b.doc_ids, step=1, lr=sample.lr,
                      weight_decay=sample.weight_decay, clip=sample.clip)
    dt = time.perf_counter() - t0
    threads = blas_threads()
    return {"value": batch * sample.seq / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one full fp64 step at batch {batch} x seq {sample.seq} of the same model ({dt:.1f} s)",
            "cpu_model": cpu_model(), "blas_threads": threads}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C4")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prof", action="store_true")
    ap.add_argument("--ckpt", metavar="DIR", help="also time a checkpoint save and load of the model in DIR")
    ap.add_argument("--fp16", action="store_true",
                    help="also time the step with fp16 operands and dynamic loss scaling")
    ap.add_argument("--untied-head", action="store_true",
                    help="also time the step of the same model with a separate vocabulary projection and bias")
    ap.add_argument("--gen", type=int, default=0, metavar="N",
                    help="also time greedy generation of N tokens per row after a 128-token prompt")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain device copy of a known size (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--pmc-cmd", default="", help="command line recorded in the summary")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "OUT_MD"),
                    help="write the kernel table of a rocprofv3 --stats run and exit")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="summarise a rocprofv3 --pmc run of the MFMA counters and exit")
    ap.add_argument("--cpu-batch", type=int, default=1, help="rows of the CPU oracle's timed step")
    ap.add_argument("--gap-summary", metavar="PMC_DIR",
                    help="write the cycle-attribution table of the GEMM and attention kernels from a --pmc run")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, cmd=args.pmc_cmd)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary, cmd=args.pmc_cmd)
        return
    if args.gap_summary:
        gap_summary(args.gap_summary, cmd=args.pmc_cmd)
        return
    if args.stats_summary:
        stats_summary(*args.stats_summary, cmd=args.pmc_cmd, steps=args.steps + args.warmup)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import scratch_decoder_only_amd as sd
    import synth

    shape = synth.SHAPES[args.config]
    B, T = shape.batch, shape.seq
    torch.cuda.set_device(0)
    log(f"bench: {args.config} B={B} T={T} building inputs")
    batch = synth.make_batch(shape)
    params = synth.init_params(shape)
    model = sd.Model(shape, max_batch=B)
    model.set(sd.LM_PARAMS, params)
    tok = torch.from_numpy(batch.tokens).cuda()
    tgt = torch.from_numpy(batch.targets).cuda()
    doc = None if batch.doc_ids is None else torch.from_numpy(batch.doc_ids).cuda()
    stream = torch.cuda.current_stream()
    if args.calib_copy:
        src = torch.ones(CALIB_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    step_no = [0]

    def step():
        step_no[0] += 1
        model.train_step(tok, tgt, doc, lr=shape.lr, step=step_no[0], beta1=shape.beta1, beta2=shape.beta2,
                         eps=shape.eps, weight_decay=shape.weight_decay, clip=shape.clip)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: warm-up done ({args.warmup} steps), loss {float(model.stats[0]):.4f}")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = B * T / (ms / 1e3)
    stats = model.stats.cpu().numpy()
    log(f"bench: {args.steps} steps, {ms:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}), "
        f"{tokens_per_s:,.0f} tokens/s, loss {stats[0]:.4f}")

    attn_f = attention_flops(shape, batch.doc_ids, B, T)
    out = {"metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if shape.precision == "bf16" else "f32",
           "data": "synthetic (seeded Zipf token ids, random-init weights)",
           "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}", "global_batch": B, "seq_len": T}}
    n_valid = int((batch.targets >= 0).sum())
    if n_valid < B * T:
        # packed rows: positions that carry a loss target (padding excluded)
        out["valid_target_tokens_per_s"] = round(n_valid / (ms / 1e3), 1)
        out["valid_targets"] = n_valid

    if not args.no_prof:
        model.profile(True)
        model.profile_read(reset=True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        prof = model.profile_read(reset=True)
        model.profile(False)
        # algorithmic attention flops per allowed pair: forward 4 D (S, PV);
        # backward 8 D, attributed 6 D to the dK/dV pass (dP, dV, dK) and 2 D to
        # the dQ pass (dQ); score recomputation is not algorithmic work
        share = {"attn_fwd": 1.0 / 3.0, "attn_bwd_dq": 1.0 / 6.0, "attn_bwd_dkv": 1.0 / 2.0}
        for k, v in prof.items():
            if k in share:
                v["flops"] = attn_f * share[k] * v["launches"] / shape.n_layers
        total_ms = sum(v["ms"] for v in prof.values())
        mm = {k: v for k, v in prof.items() if k.startswith("gemm") or k.startswith("attn")}
        mm_flops = sum(v["flops"] for v in mm.values())
        mm_ms = sum(v["ms"] for v in mm.values())
        peak = PEAK_BF16_TFLOPS if shape.precision == "bf16" else PEAK_FP32_TFLOPS
        out["mfma_util"] = round(mm_flops / (mm_ms * 1e-3) / (peak * 1e12), 4) if mm_ms > 0 else None
        out["gemm_attn_ms_per_step"] = round(mm_ms / args.steps, 4)
        out["profiled_ms_per_step"] = round(total_ms / args.steps, 4)
        dom = max(prof.items(), key=lambda kv: kv[1]["ms"])
        name, v = dom
        per_launch_ms = v["ms"] / v["launches"]
        # (the counter tables cover the C4 step; other workloads report null)
        traffic = traffic_of(name) if args.config == "C4" else None
        if v["flops"] > 0:
            ach = v["flops"] / v["launches"] / (per_launch_ms * 1e-3) / 1e12
            out["roofline"] = {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                               "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                               "per_launch_ms": round(per_launch_ms, 5),
                               "algorithmic_per_launch": v["flops"] / v["launches"]}
        else:
            ach = v["bytes"] / v["launches"] / (per_launch_ms * 1e-3) / 1e9
            out["roofline"] = {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                               "per_launch_ms": round(per_launch_ms, 5),
                               "algorithmic_per_launch": v["bytes"] / v["launches"]}
        out["kernels"] = {k: {"ms_per_step": round(v["ms"] / args.steps, 4),
                              "launches_per_step": v["launches"] / args.steps,
                              "tflops": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["flops"] and v["ms"] else None,
                              "gbs": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1) if v["bytes"] and v["ms"] else None}
                          for k, v in sorted(prof.items(), key=lambda kv: -kv[1]["ms"])}
        rec = mfma_record() if args.config == "C4" else None
        if rec:
            out["mfma_counters"] = {"busy_frac": rec["busy_frac"],
                                    "source": os.path.relpath(MFMA_FILE, ROOT)}
        log(f"bench: profiled pass {total_ms / args.steps:.3f} ms/step; dominant {name} "
            f"{per_launch_ms:.4f} ms/launch; GEMM+attention MFMA util {out['mfma_util']}")

    if args.gen:
        # generation through forward_logits (no key/value cache) and the
        # next-token kernel; the sampler alone on the last position's logits
        T0 = min(128, T - args.gen)
        prompt = tok[:, :T0].contiguous()
        rates = {}
        for mode in ("recompute", "cache", "graph"):
            kw = dict(kv_cache=mode != "recompute", graph=mode == "graph")
            sd.generate(model, prompt, 3, **kw)  # warm-up
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            sd.generate(model, prompt, args.gen, **kw)
            torch.cuda.synchronize()
            rates[mode] = time.perf_counter() - t0
        logits = model.forward_logits(prompt)[:, T0 - 1, :]
        u = torch.rand(B, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            sd.sample_tokens(logits, 1.0, 50, u)
        e1.record(stream)
        torch.cuda.synchronize()
        out["generation"] = {"batch": B, "prompt": T0, "new_tokens": args.gen,
                             "tokens_per_s_recompute": round(B * args.gen / rates["recompute"], 1),
                             "tokens_per_s_kv_cache": round(B * args.gen / rates["cache"], 1),
                             "ms_per_token_step_kv_cache": round(rates["cache"] / args.gen * 1e3, 3),
                             "tokens_per_s_kv_cache_graph": round(B * args.gen / rates["graph"], 1),
                             "ms_per_token_step_kv_cache_graph": round(rates["graph"] / args.gen * 1e3, 3),
                             "sample_us_per_call": round(e0.elapsed_time(e1) / 10 * 1e3, 1)}
        log(f"bench: generation {B}x{args.gen} tokens: {rates['recompute']:.3f} s recomputing, "
            f"{rates['cache']:.3f} s with the cache, {rates['graph']:.3f} s with the cache and a decode graph")

    def time_variant(vshape):
        """ms per step of the same workload on a model of another variant."""
        vm = sd.Model(vshape, max_batch=B)
        vm.set(sd.LM_PARAMS, synth.init_params(vshape))
        kw = dict(lr=shape.lr, beta1=shape.beta1, beta2=shape.beta2, eps=shape.eps,
                  weight_decay=shape.weight_decay, clip=shape.clip)
        for i in range(args.warmup):
            vm.train_step(tok, tgt, doc, step=i + 1, **kw)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            vm.train_step(tok, tgt, doc, step=args.warmup + i + 1, **kw)
        ev1.record(stream)
        torch.cuda.synchronize()
        vms = ev0.elapsed_time(ev1) / args.steps
        return vm, vms

    if args.untied_head:
        # the same workload with head.w [V, C] and head.b [V] instead of the
        # projection tied to wte: one more weight-gradient-sized AdamW range
        # and the head bias gradient
        um, ums = time_variant(shape.replace(untied_head=True))
        out["untied_head"] = {"ms_per_step": round(ums, 4), "tokens_per_s": round(B * T / (ums / 1e3), 1),
                              "params": int(sum(r * c for _, _, r, c in um.table)),
                              "loss": round(float(um.stats[0]), 4)}
        log(f"bench: untied head {ums:.3f} ms/step, {B * T / (ums / 1e3):,.0f} tokens/s")
        del um

    if args.fp16:
        # fp16 operands with dynamic loss scaling instead of bf16
        fm, fms = time_variant(shape.replace(precision="fp16"))
        sc = fm.loss_scaler()
        out["fp16"] = {"ms_per_step": round(fms, 4), "tokens_per_s": round(B * T / (fms / 1e3), 1),
                       "loss": round(float(fm.stats[0]), 4), "loss_scale": sc["scale"],
                       "finite_steps_in_a_row": sc["good_steps"]}
        log(f"bench: fp16 {fms:.3f} ms/step, {B * T / (fms / 1e3):,.0f} tokens/s, loss scale {sc['scale']:g}")
        del fm

    if args.ckpt:
        # checkpoint file of the multi-step driver: parameters + both Adam moments
        os.makedirs(args.ckpt, exist_ok=True)
        path = os.path.join(args.ckpt, f"bench_{args.config}.safetensors")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        model.save(path, step_no[0])
        t_save = time.perf_counter() - t0
        size = os.path.getsize(path)
        t0 = time.perf_counter()
        got = model.load(path)
        t_load = time.perf_counter() - t0
        os.remove(path)
        out["checkpoint"] = {"bytes": size, "save_s": round(t_save, 3), "load_s": round(t_load, 3),
                             "save_gbs": round(size / t_save / 1e9, 2), "load_gbs": round(size / t_load / 1e9, 2),
                             "step": got}
        log(f"bench: checkpoint {size / 1e9:.2f} GB saved in {t_save:.2f} s, loaded in {t_load:.2f} s")

    if not args.no_cpu:
        log("bench: timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(shape, args.cpu_batch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
