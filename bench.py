#!/usr/bin/env python3
"""Benchmark of the int4 routed-expert MoE layer on one MI355X.

A step is one decode token through one MoE layer: route (router GEMV, top-k,
batch-union) and forward (fused gate/up dequant-GEMV + SiLU*mul, down
dequant-GEMV, gate-weighted combine into the residual), d=6144, f=2048,
256 experts, top-8, plus one shared expert.  Inputs are seeded synthetic
tensors resident in HBM before timing starts.  Consecutive steps cycle over a
ring of independently generated layer instances (default 8, 41 GB), so the
expert weights come from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line.  `value` is microseconds per token per MoE layer (lower
is better); the line also carries tokens/s, int4 expert-weight GB/s and its
fraction of the 8 TB/s HBM peak, the roofline of the dominant kernel and the
CPU oracle's time on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ring", type=int, default=8, help="independent layer instances cycled over")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("auto", "fp32", "fxp"), default="auto",
                    help="arithmetic path of the headline (auto: fixed-point activations at these shapes)")
    ap.add_argument("--no-compare", action="store_true", help="skip timing the other arithmetic path")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import int4_routed_expert_fp32_amd as cm
    from int4_routed_expert_fp32_amd.runtime import MoeContext

    w = synth.WORKLOADS["decode"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=args.ring, n_shared=w.n_shared, max_tokens=1)
    t0 = time.time()
    for i in range(args.ring):
        R = synth.router(w, i)
        ex = synth.expert_blobs(w, i, 0, w.E)
        sh = synth.shared_blob(w, i)
        ctx.load_layer(i, R, None, ex, sh)
        del ex
        print("loaded layer instance %d/%d (%.1f s)" % (i + 1, args.ring, time.time() - t0), file=sys.stderr,
              flush=True)

    n = args.warmup + args.steps
    X = torch.from_numpy(synth.activations(w.with_(T=n), stream=11)).to(dev)
    res = X.clone()
    idx = torch.empty((n, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((n, w.k), dtype=torch.float32, device=dev)
    unions = [ctx.new_union(1) for _ in range(args.ring)]
    stream = torch.cuda.current_stream(dev)

    flag_of = {"auto": cm.COLIMOE_FWD_AUTO, "fp32": cm.COLIMOE_FWD_FP32, "fxp": cm.COLIMOE_FWD_FXP}

    def step(i, flags):
        layer = i % args.ring
        x = X[i:i + 1]
        U = unions[layer]
        cm.colimoe_route_forward(ctx.ctx, layer, x.data_ptr(), 1, idx[i].data_ptr(), wts[i].data_ptr(), U.abi(),
                                 res[i].data_ptr(), flags)

    def timed(flags):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.warmup, n):
            step(i, flags)
        ev1.record(stream)
        torch.cuda.synchronize()
        ctx.sync()
        return ev0.elapsed_time(ev1) / args.steps

    def per_kernel(flags):
        names = ("route", "topk", "union", "encode", "gateup", "down", "combine")
        cm.colimoe_timing_enable(ctx.ctx, True)
        cm.colimoe_timing_read(ctx.ctx, "route", reset=True)
        for i in range(args.warmup, n):
            step(i, flags)
        kern = {}
        for k in names:
            tot, cnt = cm.colimoe_timing_read(ctx.ctx, k)
            if cnt:
                kern[k] = dict(avg_us=1000.0 * tot / cnt, launches=cnt)
        cm.colimoe_timing_enable(ctx.ctx, False)
        ctx.sync()
        return kern

    head = flag_of[args.path]
    for i in range(args.warmup):
        step(i, head)
    ctx.sync()
    torch.cuda.synchronize()
    ms_step = timed(head)          # headline pass: plain launches
    kern = per_kernel(head)        # the same steps with HIP events around each kernel
    other = None
    if not args.no_compare:
        oflags = cm.COLIMOE_FWD_FP32 if args.path != "fp32" else cm.COLIMOE_FWD_FXP
        for i in range(args.warmup):
            step(i, oflags)
        oms = timed(oflags)
        okern = per_kernel(oflags)
        other = {"path": "fp32" if oflags == cm.COLIMOE_FWD_FP32 else "fxp", "us_per_token": round(1000 * oms, 3),
                 "kernels": {k: round(v["avg_us"], 3) for k, v in okern.items()}}

    be = w.expert_bytes
    gu_bytes = 2 * (w.d * w.f // 2 + 2 * w.d * w.f // 64)     # gate+up int4 + fp16 scales of one expert
    dn_bytes = be - gu_bytes
    experts_touched = w.k + w.n_shared                         # T = 1: k distinct routed + shared
    int4_bytes = experts_touched * be
    us_token = 1000.0 * ms_step
    gbs = int4_bytes / (ms_step * 1e-3) / 1e9
    gu_gbs = experts_touched * gu_bytes / (kern["gateup"]["avg_us"] * 1e-6) / 1e9
    dn_gbs = experts_touched * dn_bytes / (kern["down"]["avg_us"] * 1e-6) / 1e9
    roofline = dict(bound="hbm", kernel="gateup", achieved=round(gu_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gu_gbs / HBM_PEAK_GBS, 4), traffic=None,
                    bytes_per_launch=experts_touched * gu_bytes, avg_launch_us=round(kern["gateup"]["avg_us"], 3))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": "MoE-layer decode us/token + int4 expert-weight GB/s vs HBM peak",
        "value": round(us_token, 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights; fp32 accumulation" + (" (fixed-point activations, exact int4 dot)"
                                                        if args.path != "fp32" else " (fp32 dequant)"),
        "data": "synthetic (seeded int4 gs64 experts, fp16 scales, N(0,1) activations)",
        "config": {"workload": "decode MoE layer d=6144 f=2048 E=256 top-8 + 1 shared, 1 token",
                   "layer_ring": args.ring},
        "tokens_per_s": round(1e6 / us_token, 1),
        "int4_bytes_per_token": int4_bytes,
        "int4_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "kernels": {k: {"avg_us": round(v["avg_us"], 3), "launches": v["launches"]} for k, v in kern.items()},
        "down_gbs": round(dn_gbs, 1),
        "path": args.path,
        "compare": other,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, budget_s):
    """The oracle (route + forward, fp64) on a bounded sample of decode tokens."""
    import numpy as np

    import oracle
    import synth
    oracle.build(force=False)
    L = 0
    R = synth.router(w, L)
    shared = synth.shared_blob(w, L)
    X = synth.activations(w.with_(T=64), stream=11)
    done, t_cpu = 0, 0.0
    blobs = {}
    while done < X.shape[0] and t_cpu < budget_s:
        x = X[done].astype(np.float64)
        t = time.perf_counter()
        l, idx, wt = oracle.route_token(R, None, x, w.k)
        t_cpu += time.perf_counter() - t
        for e in idx:  # input generation is not part of the timed work
            if int(e) not in blobs:
                blobs[int(e)] = synth.expert_blobs(w, L, int(e), int(e) + 1)[0].copy()
        t = time.perf_counter()
        oracle.moe_token(x, w.d, w.f, {int(e): blobs[int(e)] for e in idx}, shared, idx, wt, x, w.E)
        t_cpu += time.perf_counter() - t
        done += 1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(1e6 * t_cpu / done, 1), "unit": "us/token", "cores": threads, "kind": "oracle",
            "sample": "%d decode tokens of the same layer shape (layer instance 0), route + 8 routed + shared "
                      "expert in fp64, %.1f s" % (done, t_cpu)}


if __name__ == "__main__":
    main()
