#!/usr/bin/env python3
"""Throughput of the MoE FFN block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c3|c4|c5|c1]

One step = one moe_block_forward call (router, top-k, permutation, grouped
gate/up + SwiGLU, grouped down, combine with the shared expert) over one batch
of synthetic tokens already resident in HBM.  The default workload is the
Klear-shaped decode layer (32 tokens, hidden 2048, 256 experts top-8, 4-bit
affine g64 experts, blended shared expert).  The weights are rotated over
several copies so that the 256 MB Infinity Cache cannot serve them.

Prints one JSON line: tokens/s for the whole step, the roofline of the dominant
kernel (the grouped gate/up GEMM, timed live with HIP events on the stream it
runs on, on every --gu-every'th step of the timed region: the events cost the
step ~2.5 us), and the float64 CPU oracle timed on the host cores over a bounded
sample of the same layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + HBM GB/s (decode) / MFMA TFLOP/s (4096-tok prefill)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

WORKLOADS = {
    "c2": "Klear-shaped decode: 32 tokens, hidden 2048, 256 experts top-8, sigmoid + selection bias, renormalised, "
          "SwiGLU intermediate 768 with 4-bit affine g64 weights, shared expert (768) blended",
    "c3": "Klear-shaped prefill: 4096 tokens, hidden 2048, 256 experts top-8, 4-bit affine g64, shared blended",
    "c4": "standard top-k: 2048 tokens, hidden 2816, 128 experts top-8 softmax, 4-bit affine g64, shared 2112 added",
    "c5": "latent MoE: 1024 tokens, hidden 7168 -> latent 3584, 384 experts top-8, MXFP4 clamped at 7, "
          "RMSNorm, bf16 shared 2048 added",
    "c1": "tiny fp32 layer: 4 tokens, hidden 64, 8 experts top-2, dense fp32, shared blended",
}
CPU_SAMPLE_TOKENS = {"c1": 4, "c2": 32, "c3": 96, "c4": 96, "c5": 12}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def work_model(b, hit):
    """Algorithmic bytes/FLOPs of one step and of one gate/up launch.
    hit: sorted distinct experts chosen by the batch."""
    import synth
    T, H, D, K, I, Is, E = b.T, b.H, (b.D or b.H), b.K, b.I, b.I_s, b.E
    ex = b.experts
    per_gu = ex.gate.nbytes_per_matrix() + ex.up.nbytes_per_matrix()
    per_dn = ex.down.nbytes_per_matrix()
    act = b.x.element_size()
    inter = 4 if act == 4 else 2
    sh_gu = sh_dn = 0
    if b.shared is not None:
        sh_gu = b.shared.gate.nbytes_per_matrix() + b.shared.up.nbytes_per_matrix()
        sh_dn = b.shared.down.nbytes_per_matrix()
    latent = 0
    if b.latent_down is not None:
        latent = b.latent_down.nbytes_per_matrix() + b.latent_up.nbytes_per_matrix()
    router = b.router_w.numel() * b.router_w.element_size()
    coef = 0 if b.coef_w is None else b.coef_w.numel() * b.coef_w.element_size()
    n = len(hit)
    step_bytes = router + coef + n * (per_gu + per_dn) + sh_gu + sh_dn + latent + T * H * act + T * H * 4
    step_flops = 2 * T * H * E + 6 * T * K * D * I + (6 * T * H * Is if b.shared is not None else 0)
    if b.coef_w is not None:
        step_flops += 4 * T * H
    if b.latent_down is not None:
        step_flops += 4 * T * H * D
    # the grouped gate/up launch: hit experts' gate+up planes (+ the shared expert's
    # when it runs inside that launch), its input rows, its output h
    latent_or_f32 = b.latent_down is not None or act == 4
    gu_bytes = n * per_gu + (0 if latent_or_f32 else sh_gu)
    gu_bytes += T * D * (inter if b.latent_down is not None else act)
    gu_bytes += (T * K * I + (0 if latent_or_f32 else T * Is)) * inter
    gu_flops = 4 * T * K * I * D + (0 if latent_or_f32 else 4 * T * Is * H)
    return {"step_bytes": step_bytes, "step_flops": step_flops, "gu_bytes": gu_bytes, "gu_flops": gu_flops,
            "experts_hit": n}


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("moe_gemm_ws.hip", "moe_gemm.hip", "moe_mfma.h", "moe_kernels.h", "moe_device.h"):
        with open(os.path.join(ROOT, "sparse_mixture_experts_bias_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"gateup_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(b, workload):
    """The float64 oracle, untuned, on a bounded sample of the same layer."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
    except Exception:
        threads = 1
    ns = min(CPU_SAMPLE_TOKENS[workload], b.T)
    sub = synth.token_subset(b, list(range(ns))).to("cpu")
    ob = O.from_block(sub)
    t0, c0 = time.perf_counter(), time.process_time()
    O.block_forward(ob)
    wall, cpu = time.perf_counter() - t0, time.process_time() - c0
    return {"value": ns / wall, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {ns} of the {b.T} tokens of the same layer, one float64 forward "
                      f"(weights decoded per expert); wall {wall:.2f} s, process CPU {cpu:.2f} s",
            "cpu_seconds": round(cpu, 3), "wall_seconds": round(wall, 3)}


def measured_peak(hbm: bool, dev) -> dict:
    """What a plain library kernel reaches on this machine: a device-to-device copy of 1 GiB
    (bytes read + written per second) or a bf16 8192^3 torch.mm (FLOP/s)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if hbm:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        reps = 10
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        v = 2 * n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
        del src, dst
        return {"value": round(v, 1), "unit": "GB/s", "by": "torch copy_ of 1 GiB device to device (read + write)"}
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    bm = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        c = torch.mm(a, bm)
    reps = 10
    e0.record()
    for _ in range(reps):
        c = torch.mm(a, bm)
    e1.record()
    torch.cuda.synchronize()
    v = 2 * m ** 3 * reps / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, bm, c
    return {"value": round(v, 1), "unit": "TFLOP/s", "by": "torch.mm bf16 8192x8192x8192"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: enough for 1 GiB)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload's layer on this many tokens instead of its own count")
    ap.add_argument("--gu-every", type=int, default=4,
                    help="time the gate/up launch of every N-th timed step with HIP events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this build runs the block on a "
              f"single MI355X; there is no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    import synth
    import sparse_mixture_experts_bias_amd as moe
    from synth.descs import block_desc

    dev = "cuda:0"
    wl = args.workload
    spec = synth.FULL_SPECS[wl]
    if args.tokens > 0:
        from dataclasses import replace
        spec = replace(spec, T=args.tokens)
    log(f"workload {wl}: generating the layer on {dev}")
    b = synth.make_block(spec, dev)
    moe.lib()
    desc0 = block_desc(b)
    y = torch.empty(b.T, b.H, dtype=torch.float32, device=dev)
    idx = torch.empty(b.T, b.K, dtype=torch.int32, device=dev)
    w = torch.empty(b.T, b.K, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.block_ws_bytes(b.x, desc0, with_topk=True) + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:]
    moe.moe_block_forward(b.x, desc0, y, idx, w, ws=ws)
    torch.cuda.synchronize()
    hit = sorted(set(idx.flatten().tolist()))
    wm = work_model(b, hit)
    # weight copies so that the working set rotates through more than 1 GiB
    copies = args.copies
    if copies <= 0:
        touched = wm["step_bytes"]
        copies = max(1, min(16, math.ceil((1 << 30) / max(touched, 1)) + 1))
    blocks = [b] + [synth.clone_weights(b) for _ in range(copies - 1)]
    descs = [desc0] + [block_desc(bb) for bb in blocks[1:]]
    log(f"{copies} weight copies, {wm['experts_hit']} experts hit, {wm['step_bytes'] / 1e6:.1f} MB/step")

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        moe.moe_block_forward(b.x, descs[i % copies], y, idx, w, ws=ws, stream=stream)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    moe.moe_timing_enable(moe.TIMING_GATEUP)  # creates the event pool outside the timed region
    moe.moe_timing_enable(0)
    moe.moe_timing_read()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    every = max(1, args.gu_every)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        timed = i % every == 0
        if timed:
            moe.moe_timing_enable(moe.TIMING_GATEUP)
        moe.moe_block_forward(b.x, descs[i % copies], y, idx, w, ws=ws, stream=stream)
        if timed:
            moe.moe_timing_enable(0)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    n_gu, gu_ms = moe.moe_timing_read()
    moe.moe_timing_enable(0)
    log(f"timed {args.steps} steps: {total_ms:.3f} ms; gate/up launches {n_gu}, {gu_ms:.3f} ms")

    ms_step = total_ms / args.steps
    tokens_s = b.T * args.steps / (total_ms / 1e3)
    gu_avg_s = (gu_ms / max(n_gu, 1)) / 1e3
    hbm_bound = wl in ("c1", "c2", "c5")
    if hbm_bound:
        achieved = wm["gu_bytes"] / gu_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = wm["gu_flops"] / gu_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    # the same roof as a plain library kernel reaches it on this machine (outside the timed region)
    mp = measured_peak(hbm_bound, dev)
    roof["measured_peak"] = mp
    roof["frac_of_measured"] = round(roof["achieved"] / mp["value"], 4)
    roof["traffic"] = measured_traffic(wl)
    roof["kernel"] = "expert_gemm gate/up (grouped, SwiGLU epilogue)"
    roof["kernel_avg_us"] = round(gu_avg_s * 1e6, 2)
    roof["algorithmic_bytes_per_launch"] = wm["gu_bytes"]
    roof["algorithmic_flops_per_launch"] = wm["gu_flops"]

    out = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if b.x.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": f"{wl}: {WORKLOADS[wl]}" + (f" (run on {b.T} tokens)" if args.tokens > 0 else ""),
                   "tokens": b.T, "hidden": b.H, "experts": b.E,
                   "top_k": b.K, "intermediate": b.I, "weight_copies": copies,
                   "inter_dtype": {0: "f32", 1: "bf16", 2: "f16"}[desc0.c.inter_dtype], "output": "f32"},
        "step_hbm_gbs": round(wm["step_bytes"] / (ms_step / 1e3) / 1e9, 1),
        "step_tflops": round(wm["step_flops"] / (ms_step / 1e3) / 1e12, 3),
        "step_algorithmic_bytes": wm["step_bytes"], "step_algorithmic_flops": wm["step_flops"],
        "experts_hit": wm["experts_hit"],
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(b, wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
