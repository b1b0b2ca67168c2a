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


def cpu_baseline(shape, budget_s=30.0):
    """The oracle (float64 numpy, untuned) on a bounded sample of the workload:
    one full step at batch 1 (same width, depth, vocabulary and sequence)."""
    import oracle
    import synth
    sample = shape.with_batch(1)
    b = synth.make_batch(sample)
    params = synth.init_params(sample)
    zeros = {k: np.zeros_like(v, dtype=np.float64) for k, v in params.items()}
    t0 = time.perf_counter()
    oracle.train_step(params, zeros, zeros, sample, b.tokens, b.targets, b.doc_ids, step=1, lr=sample.lr,
                      weight_decay=sample.weight_decay, clip=sample.clip)
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get("OMP_NUM_THREADS") or cores)
    return {"value": sample.seq / dt, "unit": "tokens/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"one full fp64 step at batch 1 x seq {sample.seq} of the same model ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C4")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prof", action="store_true")
    args = ap.parse_args()
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
        if v["flops"] > 0:
            ach = v["flops"] / v["launches"] / (per_launch_ms * 1e-3) / 1e12
            out["roofline"] = {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                               "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": None,
                               "per_launch_ms": round(per_launch_ms, 5),
                               "algorithmic_per_launch": v["flops"] / v["launches"]}
        else:
            ach = v["bytes"] / v["launches"] / (per_launch_ms * 1e-3) / 1e9
            out["roofline"] = {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                               "per_launch_ms": round(per_launch_ms, 5),
                               "algorithmic_per_launch": v["bytes"] / v["launches"]}
        out["kernels"] = {k: {"ms_per_step": round(v["ms"] / args.steps, 4),
                              "launches_per_step": v["launches"] / args.steps,
                              "tflops": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["flops"] and v["ms"] else None,
                              "gbs": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1) if v["bytes"] and v["ms"] else None}
                          for k, v in sorted(prof.items(), key=lambda kv: -kv[1]["ms"])}
        log(f"bench: profiled pass {total_ms / args.steps:.3f} ms/step; dominant {name} "
            f"{per_launch_ms:.4f} ms/launch; GEMM+attention MFMA util {out['mfma_util']}")

    if not args.no_cpu:
        log("bench: timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(shape)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
