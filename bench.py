#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer (Kimi-K3 shape) on one MI355X.

Default workload: single-token decode, H 3584, I 3072, 896 MXFP4 experts resident in HBM,
top-16.  A step is one pass of the layer's forward hot path for one batch: router logits,
top-k + softmax, grouping, dequant gate/up + SwiGLU, down + weighted combine.  Consecutive
steps take consecutive tokens from a pool of 64 seeded tokens, so they route to different
experts and the 256 MB last-level cache cannot serve the expert bytes of a repeated call.

Prints ONE JSON line on stdout; progress goes to stderr.
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

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), K3 shape"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA (an E4M3 operand against FP4 runs at the fp8 rate)


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# The kernel whose roofline each workload reports, the sources that define it, and what it
# does.
ROOF_KERNEL = {
    "decode1": ("k_dec_fused", ("expert_dec.hip",), "dequant + gate/up + SwiGLU + down + combine"),
    "decode64": ("k_gateup", ("expert_fwd.hip", "expert_frag.h"), "dequant + gate/up + SwiGLU"),
    "rvq16": ("k_gu_lut", ("expert_rvq_lut.hip",), "RVQ3 gate/up as codeword-table lookups"),
    "train4096": ("k_gateup_mm", ("expert_mm.hip",), "dequant + gate/up + SwiGLU"),
}


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for f in ROOF_KERNEL[workload][1] + ("common.h", "moe_internal.h"):
        h.update(open(os.path.join(ROOT, "quantized_moe_route_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_record(workload: str):
    """HBM bytes per gate/up launch from committed rocprofv3 counter runs, if they were taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"gateup_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cpu():
    """The host's CPU model, its logical CPU count and the CPUs this process may run on."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count()
    return {"model": model, "logical_cpus": os.cpu_count(), "cpus_allowed": allowed}


def cpu_baseline(w, x_pool, wr, bias, codes, scales, budget_s: float, dy_pool=None, lora=None, quant=False,
                 shared=None, rvq=None, nthreads=None):
    """The fp64 oracle as it stands, timed on a bounded sample of the same pool: consecutive
    chunks of at most 16 tokens (route + group + forward, and the input gradient when dy_pool
    is given), until budget_s of CPU work; tokens/s over the tokens processed."""
    import oracle
    nthreads = oracle.default_threads() if nthreads is None else nthreads
    if rvq is not None:  # RVQ3 layer: (idx, cb)
        W = oracle.Weights(w.H, w.I, idx=rvq[0], cb=rvq[1], lora=lora)
        Ws = oracle.Weights(w.H, w.I, idx=shared[0], cb=shared[1]) if shared else None
    else:
        W = oracle.Weights(w.H, w.I, codes=codes, scales=scales, lora=lora)
        Ws = oracle.Weights(w.H, w.I, codes=shared[0], scales=shared[1]) if shared else None
    n_sh = shared[0][0].shape[0] if shared else 0
    flat = x_pool.reshape(-1, w.H)
    dflat = None if dy_pool is None else dy_pool.reshape(-1, w.H)
    chunk = min(w.T, 16 if nthreads > 1 else 1)
    n, t0 = 0, time.perf_counter()
    while True:
        xb = oracle.to_f64(flat[n:n + chunk], "bf16")
        if dflat is None and not quant:
            oracle.layer_forward(xb, wr, bias, w.k, W, nthreads=nthreads)
        else:
            ids, p, _ = oracle.route(xb, wr, bias, w.k, nthreads=nthreads)
            oracle.forward(oracle.quantize_mxfp8(xb)[0] if quant else xb, ids, p, W, nthreads=nthreads)
        if Ws is not None:
            oracle.shared_forward(oracle.quantize_mxfp8(xb)[0] if quant else xb, Ws, n_sh, nthreads=nthreads)
        if dflat is not None:
            dyb = oracle.to_f64(dflat[n:n + chunk], "bf16")
            oracle.backward_input(xb, dyb, ids, p, wr, W, nthreads=nthreads)
            if lora is not None:
                oracle.lora_grads(xb, dyb, ids, p, W, nthreads=nthreads)
            if Ws is not None:
                oracle.shared_backward_input(xb, dyb, Ws, n_sh, nthreads=nthreads)
        n += chunk
        el = time.perf_counter() - t0
        if el >= budget_s or n + chunk > flat.shape[0]:
            break
    what = "route + group + forward" + (" of MXFP8-quantized x" if quant else "") \
        + (" + input gradient" if dflat is not None else "")
    if lora is not None:
        what += " with the adapter" + (" and its gradients" if dflat is not None else "")
    if Ws is not None:
        what += f", {n_sh} shared experts"
    return {"value": n / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n} tokens of the timed pool in chunks of {chunk} ({what} with {w.k} experts per "
                      f"token), {el:.1f} s of fp64 CPU work"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode1", choices=["decode1", "decode64", "rvq16", "train4096"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lora", type=int, default=0, metavar="RANK",
                    help="attach a shared low-rank adapter of this rank (LazyLoRA's is 16); the training pass then "
                         "also computes the adapter gradients")
    ap.add_argument("--shared", type=int, default=0, metavar="N",
                    help="add N shared experts (K3 has 2), taken by every token with weight 1")
    ap.add_argument("--mx-gateup", action="store_true",
                    help="block-scaled gate/up (FP4 weights straight into the MFMA; grouped-GEMM workloads)")
    ap.add_argument("--rvq-gather", action="store_true",
                    help="RVQ3 few-token experts on the codeword-gather kernels instead of the table lookups")
    ap.add_argument("--quant-x8", action="store_true",
                    help="activation-quantized prefill: the experts take x quantized to MXFP8")
    ap.add_argument("--no-plain-read", action="store_true",
                    help="skip the reference stream (a plain read of the roofline kernel's byte count)")
    ap.add_argument("--breakdown", action="store_true", help="also time every kernel family (stderr)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the run, copy a buffer of this many MB three times (a kernel of known "
                         "traffic for calibrating hardware byte counters)")
    ap.add_argument("--print-hash", action="store_true", help="print the roofline kernel's source hash and exit")
    ap.add_argument("--spread", type=int, default=3, metavar="N",
                    help="run the timed measurement in N separate processes (this one and N-1 children) and "
                         "report the spread of their ms/step; 1 = this process only")
    ap.add_argument("--scrub-steps", type=int, default=64, metavar="K",
                    help="also time K steps one by one, each after a 1 GiB write that flushes the last-level "
                         "cache (decode workloads; 0 = skip)")
    ap.add_argument("--graph", action="store_true", default=None,
                    help="also time the steps replayed from a captured HIP graph (default on for decode)")
    ap.add_argument("--no-graph", dest="graph", action="store_false")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (every box here has one GPU, "
              "and the layer's multi-GPU sharding is a design, not a build)", file=sys.stderr)
        sys.exit(2)

    if args.print_hash:
        print(kernel_source_hash(args.workload))
        return

    # The other processes of the spread run first, before this one touches the GPU: each is a
    # child that measures the same workload and prints its own JSON line.
    spread = []
    if args.spread > 1 and not args.child:
        import subprocess
        cmd = [sys.executable, os.path.abspath(__file__), "--child", "--spread", "1", "--no-cpu-baseline",
               "--no-plain-read", "--no-graph", "--scrub-steps", "0", "--workload", args.workload,
               "--steps", str(args.steps), "--warmup", str(args.warmup)]
        for flag, on in (("--mx-gateup", args.mx_gateup), ("--quant-x8", args.quant_x8)):
            if on:
                cmd.append(flag)
        if args.lora:
            cmd += ["--lora", str(args.lora)]
        if args.shared:
            cmd += ["--shared", str(args.shared)]
        for i in range(args.spread - 1):
            log(f"spread: process {i + 2} of {args.spread}")
            r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
            if r.returncode != 0:
                sys.exit(f"spread process {i + 2} failed with status {r.returncode}")
            spread.append(json.loads(r.stdout.strip().splitlines()[-1])["ms_per_step"])

    import numpy as np
    import torch

    import moe_synth as syn
    import quantized_moe_route_amd as q
    from quantized_moe_route_amd import _lib as C

    assert torch.cuda.is_available(), "no GPU visible"
    torch.cuda.set_device(0)
    w = syn.WORKLOADS[args.workload]
    POOL = 64 if w.T <= 64 else 2
    train = w.with_dy and w.T > 64
    log(f"workload {w.name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} {w.wfmt}; generating weights")
    wr, bias = syn.router_weight(w), syn.router_bias(w)
    kw = dict(hidden=w.H, inter=w.I, n_experts=w.E, top_k=w.k, max_tokens=w.T, router_w=q.to_device(wr),
              router_b=None if bias is None else q.to_device(bias))
    if w.wfmt == "mxfp4":
        codes, scales = syn.mxfp4_layer(w)
        kw["codes"] = [q.to_device(a) for a in codes]
        kw["scales"] = [q.to_device(a) for a in scales]
        expert_bytes = sum(a[0].nbytes for a in codes) + sum(a[0].nbytes for a in scales)
        gateup_bytes_per_expert = sum(a[0].nbytes for a in codes[:2]) + sum(a[0].nbytes for a in scales[:2])
    else:
        codes = scales = None
        idx, cb = syn.rvq3_layer(w)
        kw["rvq_idx"] = [q.to_device(a) for a in idx]
        kw["rvq_cb"] = [q.to_device(a) for a in cb]
        expert_bytes = sum(a[0].nbytes for a in idx) + sum(a[0].nbytes for a in cb)
        gateup_bytes_per_expert = sum(a[0].nbytes for a in idx[:2]) + sum(a[0].nbytes for a in cb[:2])
    if args.shared:
        sh = syn.shared_experts(w, args.shared)
        kw["shared"] = ([q.to_device(a) for a in sh[0]], [q.to_device(a) for a in sh[1]])
        # every token reads the shared experts' bytes too
        shared_bytes = sum(a.nbytes for a in sh[0]) + sum(a.nbytes for a in sh[1])
        shared_gateup_bytes = sum(a.nbytes for a in sh[0][:2]) + sum(a.nbytes for a in sh[1][:2])
    else:
        shared_bytes = shared_gateup_bytes = 0
    kw["flags"] = ((C.MOE_F_LORA if args.lora else 0) | (C.MOE_F_MX_GATEUP if args.mx_gateup else 0)
                   | (C.MOE_F_QUANT_X8 if args.quant_x8 else 0) | (C.MOE_F_RVQ_GATHER if args.rvq_gather else 0))
    L = q.MoELayer(**kw)
    if args.lora:
        A_h, B_h = syn.lora_adapter(w, args.lora)
        L.set_lora([q.to_device(a) for a in A_h], [q.to_device(b_) for b_ in B_h], 32.0 / args.lora)
    x_host = syn.activations(w, w.T * POOL).reshape(POOL, w.T, w.H)
    x_pool = q.bf16_tensor(x_host.reshape(-1, w.H)).reshape(POOL, w.T, w.H)
    r = L.new_routing(w.T)
    y = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    if train:
        dy_pool = q.bf16_tensor(syn.upstream_grad(w, w.T * POOL)).reshape(POOL, w.T, w.H)
        gu = L.new_saved_gu(w.T)
        dx = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")

    # active experts per pool entry (device routing, read once before any timing)
    U = []
    for i in range(POOL):
        L.route(x_pool[i], r)
        U.append(int(r.n_active.item()))
    log(f"active experts per step: min {min(U)} max {max(U)}")

    def step(i):
        xi = x_pool[i % POOL]
        L.route(xi, r)
        if train:
            L.forward(xi, r, y=y, saved_gu=gu)
            if args.lora:
                L.backward_lora(xi, dy_pool[i % POOL], r, saved_gu=gu, dx=dx)
            else:
                L.backward_input(xi, dy_pool[i % POOL], r, saved_gu=gu, dx=dx)
        else:
            L.forward(xi, r, y=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end)
    if args.child:
        print(json.dumps({"ms_per_step": ms / args.steps}), flush=True)
        L.close()
        return

    def pct(v):
        v = sorted(v)
        at = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]  # noqa: E731
        return {"p10": at(0.10), "p50": at(0.50), "p90": at(0.90), "n": len(v)}

    # Per-step distribution: the same steps again, each between its own pair of events (the
    # event records add a little queue work, so the mean above stays the headline).
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step(args.warmup + i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step_us = pct([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)])
    log(f"per-step us: p10 {per_step_us['p10']:.1f}  median {per_step_us['p50']:.1f}  p90 {per_step_us['p90']:.1f}")
    # The roofline kernel is timed over a second pass of the same steps: per-launch events
    # (hipExtLaunchKernelGGL start/stop stamps) slow the step down, so they stay out of the
    # pass that gives the throughput.
    L.prof_enable([C.PROF_GATEUP], max_launches=args.steps * (2 if args.shared else 1))
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    gu_ms, gu_n = L.prof_read(C.PROF_GATEUP)
    L.prof_enable([])
    # one gate/up launch per step; shared experts: their units join it (few tokens) or take
    # a launch of their own
    assert gu_n == args.steps or (args.shared and gu_n == 2 * args.steps), gu_n
    steps_U = [U[(args.warmup + i) % POOL] for i in range(args.steps)]
    S = w.T * w.k
    x_bytes = w.T * w.H * 2
    S_sh = w.T * args.shared
    roof = ROOF_KERNEL[w.name]
    if args.rvq_gather and w.wfmt == "rvq3":
        roof = ("k_gateup_rvq", ("expert_rvq.hip",), "RVQ3 gate/up as codeword gathers into fp16 MFMAs + SwiGLU")
    fused = roof[0] == "k_dec_fused"
    if fused:
        # the single-token launch runs gate/up, down and the combine: every routed (and
        # shared) expert's bytes, the token row in and y out
        gu_alg = [u * expert_bytes + shared_bytes + x_bytes + w.T * w.H * 4 for u in steps_U]
    else:
        # weights, token rows, the h planes (bf16 hi + lo) and, in the training pass, the saved
        # gate/up pre-activations (fp32 g and u per slot); the RVQ3 table-lookup gate/up writes
        # g and u (fp32) instead of h, and its down pass forms h
        out_b = 8 if roof[0] == "k_gu_lut" else 4
        gu_alg = [u * gateup_bytes_per_expert + x_bytes + S * w.I * out_b + (S * 2 * w.I * 4 if train else 0)
                  + (shared_gateup_bytes + x_bytes + S_sh * w.I * 4 if args.shared else 0) for u in steps_U]
    gu_bytes = sum(gu_alg) / len(gu_alg)
    # gate/up time per step (with shared experts: both launches), from events stamped at the
    # kernels' own start and end
    gu_avg_s = gu_ms / args.steps / 1e3
    achieved = gu_bytes / gu_avg_s / 1e9
    step_bytes = [u * expert_bytes + shared_bytes + wr.nbytes + x_bytes + w.T * w.H * 4 for u in steps_U]
    step_s = ms / 1e3 / args.steps
    tokens_per_s = w.T * args.steps / (ms / 1e3)
    traffic = traffic_record(w.name) if roof is ROOF_KERNEL[w.name] else None
    log(f"{args.steps} steps in {ms:.2f} ms (wall {wall * 1e3:.1f} ms): {step_s * 1e6:.1f} us/step, "
        f"{tokens_per_s:.0f} tokens/s; {roof[0]} {gu_avg_s * 1e6:.1f} us avg, {achieved:.0f} GB/s")

    detail = {"step_hbm_GBps": sum(step_bytes) / len(step_bytes) / step_s / 1e9,
              "step_alg_bytes": sum(step_bytes) / len(step_bytes),
              "active_experts_mean": sum(steps_U) / len(steps_U),
              "roofline_kernel_us": gu_avg_s * 1e6, "roofline_kernel_alg_bytes": gu_bytes,
              "roofline_kernel_GBps": achieved}
    if train:
        # the grouped GEMM is priced against the dense MFMA peak of its operand type: exact
        # bf16 (dequantized FP4 weights, bf16 x; also the two-term block-scaled form, which
        # issues fp8 MFMAs at twice bf16's rate for twice the terms), or E4M3 x against FP4
        # weights when x arrives MXFP8-quantized; 2 S H (2 I) flop per launch
        gu_tflops = 2.0 * (S + S_sh) * w.H * 2 * w.I / gu_avg_s / 1e12
        detail["gateup_flop"] = 2.0 * (S + S_sh) * w.H * 2 * w.I
        single = args.mx_gateup and args.quant_x8
        peak = FP8_PEAK_TFLOPS if single else BF16_PEAK_TFLOPS
        kname = ("k_gateup_mx (block-scaled gate/up + SwiGLU)" if args.mx_gateup
                 else f"{roof[0]} ({roof[2]})")
        roofline = {"bound": "mfma", "kernel": kname, "achieved": gu_tflops, "peak": peak, "unit": "TFLOP/s",
                    "frac": gu_tflops / peak, "traffic": traffic if not args.mx_gateup else None}
    else:
        roofline = {"bound": "hbm", "kernel": f"{roof[0]} ({roof[2]})",
                    "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                    "traffic": traffic}
    if not train and not args.no_plain_read:
        # the practical read rate for the roofline kernel's byte count: a plain coalesced
        # read kernel over the same number of bytes, cold (a different buffer each time)
        import ctypes
        nb = (int(gu_bytes) + 15) // 16 * 16
        bufs = torch.empty((8, nb), dtype=torch.uint8, device="cuda")
        bufs.fill_(1)
        torch.cuda.synchronize()
        t = []
        for i in range(24):
            ms_ = ctypes.c_double()
            C.check(C.lib().moe_prof_hbm_read(bufs[i % 8].data_ptr(), nb, ctypes.c_void_p(
                torch.cuda.current_stream().cuda_stream), ctypes.byref(ms_)), "moe_prof_hbm_read")
            t.append(ms_.value)
        del bufs
        t_plain = sorted(t[8:])[len(t[8:]) // 2] / 1e3
        roofline["plain_read"] = {"bytes": nb, "GBps": nb / t_plain / 1e9, "us": t_plain * 1e6,
                                  "frac": achieved / (nb / t_plain / 1e9)}
        log(f"plain read of {nb} bytes: {t_plain * 1e6:.1f} us = {nb / t_plain / 1e9:.0f} GB/s; the roofline kernel "
            f"reaches {roofline['plain_read']['frac']:.3f} of it")
    if args.breakdown:
        fams = list(range(len(C.PROF_NAMES)))
        L.prof_enable(fams, max_launches=args.steps * (2 if args.shared else 1))
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        for f in fams:
            tot, n = L.prof_read(f)
            if n:
                detail[f"{C.PROF_NAMES[f]}_us"] = tot / n * 1e3
        L.prof_enable([])
        log("breakdown " + json.dumps(detail))

    variants = {}
    if not train and args.scrub_steps > 0:
        # MALL flushed before every step: a 1 GiB write between the steps, outside the timed pairs
        scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        t = []
        for i in range(args.scrub_steps):
            scrub.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(args.warmup + i)
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3)
        del scrub
        variants["mall_scrubbed_step_us"] = pct(t)
        log(f"scrubbed steps us: median {variants['mall_scrubbed_step_us']['p50']:.1f}")
    if args.graph is None:
        args.graph = not train
    if args.graph and not train:
        # The pool's 64 steps captured once into a HIP graph (route + forward of each token),
        # replayed as a whole: no host launch work inside; every replay's outputs are checked
        # against eager calls of the same steps
        ys = torch.empty((POOL, w.T, w.H), dtype=torch.float32, device="cuda")
        rs = [L.new_routing(w.T) for _ in range(POOL)]
        for i in range(POOL):
            L.route(x_pool[i], rs[i])
            L.forward(x_pool[i], rs[i], y=ys[i])
        torch.cuda.synchronize()
        y_eager = ys.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(POOL):
                L.route(x_pool[i], rs[i])
                L.forward(x_pool[i], rs[i], y=ys[i])
        reps = max(1, args.steps // POOL)
        for _ in range(2):
            ys.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(ys, y_eager), "graph replay differs from the eager steps"
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        assert torch.equal(ys, y_eager), "graph replay differs from the eager steps"
        gms = e0.elapsed_time(e1) / (reps * POOL)
        variants["hip_graph"] = {"ms_per_step": gms, "tokens_per_s": w.T / (gms / 1e3), "steps": reps * POOL}
        log(f"graph-replayed steps: {gms * 1e3:.1f} us/step ({reps} replays of {POOL} steps)")
        del g

    base = None
    if not args.no_cpu_baseline:
        log("CPU baseline: fp64 oracle")
        dy_host = syn.upstream_grad(w, w.T * POOL).reshape(POOL, w.T, w.H) if train else None
        kw_cpu = dict(lora=(A_h, B_h, 32.0 / args.lora) if args.lora else None, quant=args.quant_x8,
                      shared=sh if args.shared else None, rvq=None if codes is not None else (idx, cb))
        base = cpu_baseline(w, x_host, wr, bias, codes, scales, args.cpu_seconds, dy_host, **kw_cpu)
        one = cpu_baseline(w, x_host, wr, bias, codes, scales, min(5.0, args.cpu_seconds / 3), dy_host,
                           nthreads=1, **kw_cpu)
        host = host_cpu()
        base["host"] = host
        base["threads_note"] = (f"the oracle uses min(16, logical CPUs) threads: {base['cores']} here; the GPU "
                                f"box grants each GPU a 16-CPU share of its {host['logical_cpus']} logical CPUs")
        base["single_thread"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x mxfp4" if args.mx_gateup and args.quant_x8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: K3-shaped routed-expert layer, {w.T} token(s) per step, H {w.H}, "
                               f"I {w.I}, {w.E} {w.wfmt} experts resident, top-{w.k}, bf16 activations, "
                               + ("forward + input gradient (route + group + experts + combine + dX)" if train
                                  else "forward (route + group + experts + combine)")
                               + (f", shared rank-{args.lora} adapter" + (" with its gradients" if train else "")
                                  if args.lora else "")
                               + (", experts fed MXFP8-quantized x" if args.quant_x8 else "")
                               + (", block-scaled gate/up" if args.mx_gateup else "")
                               + (f", {args.shared} shared experts" if args.shared else ""),
                   "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k, "weights": w.wfmt, "lora_rank": args.lora,
                   "mx_gateup": args.mx_gateup, "quant_x8": args.quant_x8, "n_shared": args.shared},
        "roofline": roofline,
        "cpu_baseline": base,
        "step_us": per_step_us,
        "detail": detail,
    }
    if variants:
        out["variants"] = variants
    if spread:
        allp = [ms / args.steps] + spread
        out["process_spread"] = {"ms_per_step": allp, "min": min(allp), "max": max(allp),
                                 "median": sorted(allp)[len(allp) // 2], "processes": len(allp)}
    print(json.dumps(out), flush=True)
    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copies: 3 x {n * 4} bytes read and written")
    L.close()


if __name__ == "__main__":
    main()
