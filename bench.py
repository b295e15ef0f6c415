#!/usr/bin/env python3
"""Throughput of the MoE FFN block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c3|c4|c5|c1]

One step = one moe_block_forward call (router, top-k, permutation, grouped
gate/up + SwiGLU, grouped down, combine with the shared expert) over one batch
of synthetic tokens already resident in HBM.  The default workload is the
Klear-shaped decode layer (32 tokens, hidden 2048, 256 experts top-8, 4-bit
affine g64 experts, blended shared expert); the default run also measures the
same layer at prefill (4096 tokens) and reports it under "prefill", the other
half of the metric.  The weights are rotated over several copies so that the
256 MB Infinity Cache cannot serve them.

Prints one JSON line: tokens/s for the whole step (K steps between two events),
the per-step distribution (median, p10, p90 of a second run of K steps with an
event between consecutive steps), the roofline of the dominant kernel (the
grouped gate/up GEMM, timed live with HIP events on the stream it runs on, on
every --gu-every'th step of the timed region: the events cost the step ~2.5 us)
and of the whole step, and the float64 CPU oracle timed on the host cores over
a bounded sample of the same layer (all cores, then one thread).
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
    # the grouped down launch: hit experts' down planes (+ the shared expert's), its input h,
    # its output rows o
    dn_bytes = n * per_dn + (0 if latent_or_f32 else sh_dn)
    dn_bytes += (T * K * I + (0 if latent_or_f32 else T * Is)) * inter
    dn_bytes += (T * K + (0 if latent_or_f32 else T)) * D * inter
    dn_flops = 2 * T * K * I * D + (0 if latent_or_f32 else 2 * T * Is * H)
    return {"step_bytes": step_bytes, "step_flops": step_flops, "gu_bytes": gu_bytes, "gu_flops": gu_flops,
            "dn_bytes": dn_bytes, "dn_flops": dn_flops, "experts_hit": n}


KERNEL_SOURCES = {
    "gateup": ("moe_gemm_ws.hip", "moe_gemm.hip", "moe_mfma.h", "moe_kernels.h", "moe_device.h"),
    "decode_fused": ("moe_decode.hip", "moe_ws.h", "moe_topk.h", "moe_mfma.h", "moe_kernels.h", "moe_device.h"),
    "gateup_tall": ("moe_gemm_tall.hip", "moe_mfma.h", "moe_kernels.h", "moe_device.h"),
}


def kernel_source_sha(kernel="gateup"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_mixture_experts_bias_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel="gateup"):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_sha") != kernel_source_sha(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, workload):
    """The float64 oracle, untuned, on a bounded sample of the same layer: once with
    every BLAS thread the host offers, once with one thread."""
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
    except Exception:
        threadpool_limits, threads = None, 1
    ns = min(CPU_SAMPLE_TOKENS[workload], b.T)
    sub = synth.token_subset(b, list(range(ns))).to("cpu")
    ob = O.from_block(sub)

    def timed():
        t0, c0 = time.perf_counter(), time.process_time()
        O.block_forward(ob)
        return time.perf_counter() - t0, time.process_time() - c0

    wall, cpu = timed()
    out = {"value": ns / wall, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
           "sample": f"first {ns} of the {b.T} tokens of the same layer, one float64 forward "
                     f"(weights decoded per expert); wall {wall:.2f} s, process CPU {cpu:.2f} s",
           "cpu_seconds": round(cpu, 3), "wall_seconds": round(wall, 3)}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            w1, c1 = timed()
        out["one_thread"] = {"value": ns / w1, "unit": "tokens/s", "cores": 1, "wall_seconds": round(w1, 3),
                             "cpu_seconds": round(c1, 3)}
    return out


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


def pct(v, q):
    v = sorted(v)
    if not v:
        return None
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


def measure(wl, steps, warmup, gu_every, copies_arg=0, tokens=0, inter=None, scaled=False):
    """Generate the workload's layer on the GPU and time `steps` block forwards."""
    import torch
    import synth
    import sparse_mixture_experts_bias_amd as moe
    from synth.descs import block_desc

    dev = "cuda:0"
    spec = synth.FULL_SPECS[wl]
    if tokens > 0:
        from dataclasses import replace
        spec = replace(spec, T=tokens)
    log(f"workload {wl}: generating the layer on {dev}")
    b = synth.make_block(spec, dev)
    moe.lib()
    desc0 = block_desc(b, inter, scaled)
    y = torch.empty(b.T, b.H, dtype=torch.float32, device=dev)
    idx = torch.empty(b.T, b.K, dtype=torch.int32, device=dev)
    w = torch.empty(b.T, b.K, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.block_ws_bytes(b.x, desc0, with_topk=True) + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:]
    # which launch carries the experts: the one-launch decode path or the grouped gate/up GEMM
    moe.moe_timing_enable(moe.TIMING_FUSED)
    moe.moe_block_forward(b.x, desc0, y, idx, w, ws=ws)
    moe.moe_timing_enable(0)
    torch.cuda.synchronize()
    fused = moe.moe_timing_read()[0] > 0
    kind = moe.TIMING_FUSED if fused else moe.TIMING_GATEUP
    hit = sorted(set(idx.flatten().tolist()))
    wm = work_model(b, hit)
    # weight copies so that the working set rotates through more than 1 GiB
    copies = copies_arg
    if copies <= 0:
        copies = max(1, min(16, math.ceil((1 << 30) / max(wm["step_bytes"], 1)) + 1))
    blocks = [b] + [synth.clone_weights(b) for _ in range(copies - 1)]
    descs = [desc0] + [block_desc(bb, inter, scaled) for bb in blocks[1:]]
    log(f"{wl}: {copies} weight copies, {wm['experts_hit']} experts hit, {wm['step_bytes'] / 1e6:.1f} MB/step")

    stream = torch.cuda.current_stream()
    step = lambda i: moe.moe_block_forward(b.x, descs[i % copies], y, idx, w, ws=ws, stream=stream)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"{wl}: warmup {warmup} done")

    moe.moe_timing_enable(kind)  # creates the event pool outside the timed region
    moe.moe_timing_enable(0)
    moe.moe_timing_read()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    every = max(1, gu_every)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        timed = i % every == 0
        if timed:
            moe.moe_timing_enable(kind)
        step(i)
        if timed:
            moe.moe_timing_enable(0)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    n_gu, gu_ms = moe.moe_timing_read()
    log(f"{wl}: timed {steps} steps: {total_ms:.3f} ms; {'fused' if fused else 'gate/up'} launches {n_gu}, "
        f"{gu_ms:.3f} ms")

    # per-step distribution: the same steps again, an event between consecutive steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i].record(stream)
        step(i)
    evs[steps].record(stream)
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)]

    # the down launch's average, timed on its own run of steps (outside both timed regions)
    n_dn, dn_ms = 0, 0.0
    if not fused:
        moe.moe_timing_enable(moe.TIMING_DOWN)
        for i in range(min(steps, 20)):
            step(i)
        moe.moe_timing_enable(0)
        n_dn, dn_ms = moe.moe_timing_read()
    return {"b": b, "desc": desc0, "wm": wm, "copies": copies, "total_ms": total_ms, "n_gu": n_gu, "gu_ms": gu_ms,
            "per_step_us": per_step, "n_dn": n_dn, "dn_ms": dn_ms, "fused": fused}


def roofline_of(wl, r, hbm_bound, dev, with_peak=True):
    wm = r["wm"]
    gu_avg_s = (r["gu_ms"] / max(r["n_gu"], 1)) / 1e3
    if r["fused"]:
        # the decode experts launch: gate/up + SwiGLU and down; its algorithmic bytes are both
        # GEMMs' (the h rows it hands from one to the other count once as written and once as read)
        fb = wm["gu_bytes"] + wm["dn_bytes"]
        parts = "gate/up + SwiGLU and down of every slot and of the shared expert"
        achieved = fb / gu_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "scope": f"kernel only: the decode experts launch ({parts})"}
        if with_peak:
            mp = measured_peak(True, dev)
            roof["measured_peak"] = mp
            roof["frac_of_measured"] = round(roof["achieved"] / mp["value"], 4)
        roof["traffic"] = measured_traffic(wl, "decode_fused")
        roof["kernel"] = "decode_fused (" + parts + ")"
        roof["kernel_avg_us"] = round(gu_avg_s * 1e6, 2)
        roof["algorithmic_bytes_per_launch"] = fb
        roof["algorithmic_flops_per_launch"] = wm["gu_flops"] + wm["dn_flops"]
        return roof
    dn_avg_s = (r["dn_ms"] / max(r["n_dn"], 1)) / 1e3
    if hbm_bound:
        achieved = wm["gu_bytes"] / gu_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
        dn = wm["dn_bytes"] / dn_avg_s / 1e9
        roof["down_kernel"] = {"achieved": round(dn, 1), "unit": "GB/s", "frac": round(dn / HBM_PEAK_GBS, 4),
                               "kernel_avg_us": round(dn_avg_s * 1e6, 2),
                               "algorithmic_bytes_per_launch": wm["dn_bytes"]}
    else:
        achieved = wm["gu_flops"] / gu_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
        dn = wm["dn_flops"] / dn_avg_s / 1e12
        roof["down_kernel"] = {"achieved": round(dn, 2), "unit": "TFLOP/s",
                               "frac": round(dn / MFMA_BF16_PEAK_TFLOPS, 4),
                               "kernel_avg_us": round(dn_avg_s * 1e6, 2),
                               "algorithmic_flops_per_launch": wm["dn_flops"]}
    roof["scope"] = "kernel only: the grouped gate/up GEMM (achieved/frac); down_kernel likewise"
    if with_peak:
        mp = measured_peak(hbm_bound, dev)
        roof["measured_peak"] = mp
        roof["frac_of_measured"] = round(roof["achieved"] / mp["value"], 4)
    # (the MFMA-bound workloads run the 128-row prefill kernel, the HBM-bound ones the decode kernels)
    roof["traffic"] = measured_traffic(wl, "gateup" if hbm_bound else "gateup_tall")
    roof["kernel"] = "expert_gemm gate/up (grouped, SwiGLU epilogue)"
    roof["kernel_avg_us"] = round(gu_avg_s * 1e6, 2)
    roof["algorithmic_bytes_per_launch"] = wm["gu_bytes"]
    roof["algorithmic_flops_per_launch"] = wm["gu_flops"]
    return roof


def step_stats(r, steps):
    wm = r["wm"]
    ms = r["total_ms"] / steps
    ps = r["per_step_us"]
    return {
        "ms_per_step": round(ms, 5),
        "step_us_median": round(pct(ps, 0.5), 2), "step_us_p10": round(pct(ps, 0.1), 2),
        "step_us_p90": round(pct(ps, 0.9), 2),
        "step_hbm_gbs": round(wm["step_bytes"] / (ms / 1e3) / 1e9, 1),
        "step_frac_of_hbm_peak": round(wm["step_bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_tflops": round(wm["step_flops"] / (ms / 1e3) / 1e12, 3),
        "step_frac_of_bf16_mfma_peak": round(wm["step_flops"] / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "step_algorithmic_bytes": wm["step_bytes"], "step_algorithmic_flops": wm["step_flops"],
        "experts_hit": wm["experts_hit"],
    }


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
    ap.add_argument("--no-prefill", action="store_true",
                    help="c2 only: skip the 4096-token prefill record of the same layer")
    ap.add_argument("--separate-decode-launches", action="store_true",
                    help="run decode-sized batches with separate router, routing, gate/up, down and combine "
                         "launches")
    ap.add_argument("--single-decode-launch", action="store_true",
                    help="run decode-sized batches of up to 16 tokens in one launch (routing, experts and "
                         "combine) instead of three")
    ap.add_argument("--inter", choices=("auto", "bf16", "f16"), default="auto",
                    help="storage of the intermediates (auto: the layer's default)")
    ap.add_argument("--scaled-mfma", action="store_true",
                    help="MXFP4 experts (c5): run the routed GEMMs on the block-scaled FP4 x FP8 MFMA")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the library runs the block on a "
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

    dev = "cuda:0"
    wl = args.workload
    fusion = 0 if args.separate_decode_launches else (2 if args.single_decode_launch else 1)
    if fusion != 1:
        import sparse_mixture_experts_bias_amd as moe
        moe.moe_set_decode_fusion(fusion)
    import sparse_mixture_experts_bias_amd as moe
    inter = {"auto": None, "bf16": moe.MOE_BF16, "f16": moe.MOE_F16}[args.inter]
    r = measure(wl, args.steps, args.warmup, args.gu_every, args.copies, args.tokens, inter, args.scaled_mfma)
    b = r["b"]
    hbm_bound = wl in ("c1", "c2", "c5")
    roof = roofline_of(wl, r, hbm_bound, dev)
    st = step_stats(r, args.steps)
    tokens_s = b.T * args.steps / (r["total_ms"] / 1e3)
    out = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": st.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if b.x.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": f"{wl}: {WORKLOADS[wl]}" + (f" (run on {b.T} tokens)" if args.tokens > 0 else ""),
                   "tokens": b.T, "hidden": b.H, "experts": b.E,
                   "top_k": b.K, "intermediate": b.I, "weight_copies": r["copies"],
                   "inter_dtype": {0: "f32", 1: "bf16", 2: "f16"}[r["desc"].c.inter_dtype], "output": "f32",
                   "decode_fusion": fusion, "scaled_mfma": bool(args.scaled_mfma)},
        **st,
        "roofline": roof,
    }
    del r
    if wl == "c2" and not args.no_prefill and args.tokens == 0:
        # the metric's other half: the same layer at 4096-token prefill, its own record
        torch.cuda.empty_cache()
        rp = measure("c3", args.steps, args.warmup, args.gu_every, inter=inter)
        pst = step_stats(rp, args.steps)
        pre = {"workload": f"c3: {WORKLOADS['c3']}", "tokens_per_s": round(rp["b"].T * args.steps /
                                                                           (rp["total_ms"] / 1e3), 1),
               "inter_dtype": {0: "f32", 1: "bf16", 2: "f16"}[rp["desc"].c.inter_dtype],
               **pst, "roofline": roofline_of("c3", rp, False, dev, with_peak=False)}
        out["prefill"] = pre
        del rp
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(b, wl)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
