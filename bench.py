#!/usr/bin/env python3
"""Benchmark of the int4 routed-expert MoE layer on one MI355X.

Headline: one decode token through one MoE layer (d=6144, f=2048, 256 experts,
top-8, plus one shared expert): route (router GEMV, top-k, union lists) and
forward (gate/up dequant-GEMV + SiLU*mul, down dequant-GEMV, gate-weighted
combine into the residual) in one colimoe_route_forward call.  Inputs are
seeded synthetic tensors resident in HBM before timing starts.  Consecutive
steps cycle over a ring of independently generated layer instances (default
8, 41 GB) so the expert weights come from HBM rather than from the 256 MB
Infinity Cache.  `value` is microseconds per token per MoE layer.

The same JSON line also carries the other workloads of the layer, each timed on
its own loaded layers: the 32-layer decode stack (RMSNorm between layers),
the 16-position batch-union call and the 2048-token prefill call (bf16 MFMA
path, with its matrix-core utilisation), plus the roofline of the dominant
decode kernel and the CPU oracle's time on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
TOP_P = 0.7  # the adaptive expert top-p the pages run with
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_gateup_traffic.json")
KERNEL_SOURCES = ("kernels.hip", "device_common.h", "internal.h")


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
    ap.add_argument("--no-top-p", action="store_true", help="skip the adaptive expert top-p line of the decode workload")
    ap.add_argument("--only", choices=("all", "decode", "tiny", "stack32", "union16", "verify", "prefill2048",
                                       "tiered", "int8"),
                    default="all",
                    help="run one workload only (the headline line needs decode)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def hipcc_version():
    import subprocess
    try:
        r = subprocess.run([os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--version"], capture_output=True,
                           text=True, timeout=60)
        return r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return "unknown"


def kernel_source_sha():
    """Hash of what decides the decode kernels' code: their sources, the build
    script (compiler flags) and the compiler's version."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "int4_routed_expert_fp32_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "int4_routed_expert_fp32_amd", "_build.py"), "rb") as f:
        h.update(f.read())
    h.update(hipcc_version().encode())
    return h.hexdigest()


# the gate/up kernel of a one-token call (d = 6144: three 64-chunk steps per row)
DECODE_GATEUP_KERNEL = "k_gateup_one<3>"


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or rec.get("source_sha256") != kernel_source_sha():
        return None
    return int(k["fetch_bytes"] + k["write_bytes"])


def host_protocol():
    """Facts of the measurement protocol that need no GPU: host CPU, ROCm,
    source identity, command.  Gathered before the GPU is initialised (the
    tools run as child processes)."""
    import platform
    import subprocess
    info = {"command": " ".join([os.path.basename(sys.executable)] + sys.argv), "host": platform.node()}
    try:
        with open("/proc/cpuinfo") as f:
            models = [l.split(":", 1)[1].strip() for l in f if l.startswith("model name")]
        info["cpu_model"] = models[0] if models else "unknown"
        info["cpu_threads_online"] = len(models)
    except OSError:
        info["cpu_model"] = "unknown"
    info["cpu_affinity"] = len(os.sched_getaffinity(0))
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = "unknown"
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=30)
        info["git_commit"] = r.stdout.strip() if r.returncode == 0 else "unavailable (tree without .git)"
    except (OSError, subprocess.SubprocessError):
        info["git_commit"] = "unavailable"
    h = hashlib.sha256()
    for sub in ("include", os.path.join("int4_routed_expert_fp32_amd", "csrc")):
        d = os.path.join(ROOT, sub)
        for name in sorted(os.listdir(d)):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + f.read())
    with open(os.path.abspath(__file__), "rb") as f:
        h.update(f.read())
    info["source_sha256"] = h.hexdigest()
    try:
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60)
        for line in r.stdout.splitlines():
            if "Max Clock Freq" in line and "gfx" in info.get("_last_agent", ""):
                info["gpu_max_clock_mhz"] = int(line.split(":")[1].split("(")[0].strip())
                break
            if line.strip().startswith("Name:") and "gfx" in line:
                info["_last_agent"] = line
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    info.pop("_last_agent", None)
    return info


def gpu_protocol(torch, dev):
    p = torch.cuda.get_device_properties(dev)
    return {"gpu": p.name, "arch": getattr(p, "gcnArchName", "unknown"), "compute_units": p.multi_processor_count,
            "hbm_bytes": p.total_memory, "torch": torch.__version__, "hip_runtime": torch.version.hip}


def calibration_copy(torch, dev):
    """A plain device copy of known size (256 MiB read + 256 MiB written): the
    reference point that scales FETCH_SIZE / WRITE_SIZE counters to bytes."""
    a = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def stream_ceiling(torch, dev, stream):
    """Read-only HBM bandwidth on this machine: column sums of a 4096-row, 4 GiB
    fp32 matrix (every byte read once, 1 MiB written, far beyond the Infinity
    Cache; the fastest read-only form among the reductions tried), timed with
    events; the reference the decode fractions are also quoted against."""
    a = torch.ones((4096, 1 << 18), dtype=torch.float32, device=dev)
    for _ in range(3):
        a.sum(0)
    torch.cuda.synchronize()
    reps = 10
    ms = event_time(torch, stream, lambda: [a.sum(0) for _ in range(reps)]) / reps
    del a
    torch.cuda.empty_cache()
    return {"gbs": round((1 << 32) / (ms * 1e-3) / 1e9, 1),
            "how": "column sums of a 4096 x 262144 fp32 matrix (4 GiB read once), 10 reps"}


def per_kernel(cm, ctx, run, names=("route", "topk", "union", "encode", "gateup", "down", "combine", "rmsnorm")):
    cm.colimoe_timing_enable(ctx.ctx, True)
    for k in names:
        cm.colimoe_timing_read(ctx.ctx, k, reset=True)
    run()
    kern = {}
    for k in names:
        tot, cnt = cm.colimoe_timing_read(ctx.ctx, k)
        if cnt:
            kern[k] = dict(avg_us=1000.0 * tot / cnt, launches=cnt)
    cm.colimoe_timing_enable(ctx.ctx, False)
    ctx.sync()
    return kern


def event_time(torch, stream, run):
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    run()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1)  # ms


def windowed_time(torch, stream, run, lo, hi, n_win=5):
    """Times steps lo..hi-1 (run(a, b) enqueues steps a..b-1) in n_win equal
    consecutive sub-windows, events between them and no host synchronisation
    inside: (ms per step over all of them, [ms per step of each window])."""
    bounds = [lo + (hi - lo) * i // n_win for i in range(n_win + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n_win):
        run(bounds[i], bounds[i + 1])
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) / max(bounds[i + 1] - bounds[i], 1) for i in range(n_win)]
    return evs[0].elapsed_time(evs[-1]) / (hi - lo), per


def graph_time(torch, ctx, run, reps=3):
    """ms per replay of `run` captured into one HIP graph (the context's calls
    are enqueued on the capture stream while capturing, then the stream is
    put back)."""
    cap = torch.cuda.Stream()
    old = ctx.stream
    torch.cuda.synchronize()
    ctx.set_stream(cap)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run()
    torch.cuda.synchronize()
    with torch.cuda.stream(cap):
        g.replay()
        torch.cuda.synchronize()
        ms = event_time(torch, cap, lambda: [g.replay() for _ in range(reps)]) / reps
    ctx.set_stream(old)
    del g
    torch.cuda.synchronize()
    return ms


def load_ring(ctx, synth, w, n, tag):
    t0 = time.time()
    for i in range(n):
        ex = synth.expert_blobs(w, i, 0, w.E)
        ctx.load_layer(i, synth.router(w, i), synth.bias(w, i), ex, synth.shared_blob(w, i))
        del ex
        if i % 8 == 7 or i == n - 1:
            log("%s: loaded layer %d/%d (%.1f s)" % (tag, i + 1, n, time.time() - t0))


def bench_decode(args, torch, np, synth, cm, MoeContext, dev, stream):
    w = synth.WORKLOADS["decode"]
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=args.ring, n_shared=w.n_shared, max_tokens=1)
    load_ring(ctx, synth, w, args.ring, "decode")
    n = args.warmup + args.steps
    X = torch.from_numpy(synth.activations(w.with_(T=n), stream=11)).to(dev)
    res = X.clone()
    idx = torch.empty((n, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((n, w.k), dtype=torch.float32, device=dev)
    unions = [ctx.new_union(1) for _ in range(args.ring)]
    flag_of = {"auto": cm.COLIMOE_FWD_AUTO, "fp32": cm.COLIMOE_FWD_FP32, "fxp": cm.COLIMOE_FWD_FXP}

    def step(i, flags):
        layer = i % args.ring
        cm.colimoe_route_forward(ctx.ctx, layer, X[i].data_ptr(), 1, idx[i].data_ptr(), wts[i].data_ptr(),
                                 unions[layer].abi(), res[i].data_ptr(), flags)

    def steps(flags, lo, hi):
        return lambda: [step(i, flags) for i in range(lo, hi)]

    head = flag_of[args.path]
    steps(head, 0, args.warmup)()
    ctx.sync()
    # exactly `steps` timed steps, in five consecutive sub-windows
    ms, win = windowed_time(torch, stream, lambda a, b: steps(head, a, b)(), args.warmup, n)
    ctx.sync()
    kern = per_kernel(cm, ctx, steps(head, args.warmup, n))
    # the same steps captured into one HIP graph and replayed
    gms = graph_time(torch, ctx, steps(head, args.warmup, n)) / args.steps
    timing = {"median_window_us": round(1000 * sorted(win)[len(win) // 2], 3),
              "window_us": [round(1000 * v, 3) for v in win],
              "graph_replay_us_per_token": round(1000 * gms, 3)}
    topp = None
    if not args.no_top_p:
        # adaptive expert top-p at the pages' value (p = 0.7): time per token and
        # routed experts read (sampled outside the timed region)
        cm.colimoe_set_expert_top_p(ctx.ctx, TOP_P)
        steps(head, 0, args.warmup)()
        tms = event_time(torch, stream, steps(head, args.warmup, n)) / args.steps
        kept = []
        for i in range(args.warmup, min(n, args.warmup + 64)):
            step(i, head)
            kept.append(int(unions[i % args.ring].n_unique.item()))
        cm.colimoe_set_expert_top_p(ctx.ctx, 1.0)
        ctx.sync()
        km = float(np.mean(kept))
        tb = (km + w.n_shared) * w.expert_bytes
        topp = {"p": TOP_P, "us_per_token": round(1000 * tms, 3), "routed_experts_mean": round(km, 3),
                "int4_bytes_per_token_mean": int(tb), "int4_gbs": round(tb / (tms * 1e-3) / 1e9, 1),
                "sampled_tokens": len(kept)}
    other = None
    if not args.no_compare:
        oflags = cm.COLIMOE_FWD_FP32 if args.path != "fp32" else cm.COLIMOE_FWD_FXP
        steps(oflags, 0, args.warmup)()
        oms = event_time(torch, stream, steps(oflags, args.warmup, n)) / args.steps
        okern = per_kernel(cm, ctx, steps(oflags, args.warmup, n))
        other = {"path": "fp32" if oflags == cm.COLIMOE_FWD_FP32 else "fxp", "us_per_token": round(1000 * oms, 3),
                 "kernels": {k: round(v["avg_us"], 3) for k, v in okern.items()}}
    ctx.close()
    del ctx, X, res
    torch.cuda.empty_cache()
    return w, ms, kern, other, topp, timing


def bench_stack32(args, torch, np, synth, cm, MoeContext, dev, stream):
    w = synth.WORKLOADS["stack32"]
    need = w.n_layers * (w.E + w.n_shared) * w.expert_bytes
    free, _ = torch.cuda.mem_get_info()
    if free < need * 1.05:
        return {"skipped": "needs %.1f GB of device memory, %.1f GB free" % (need / 1e9, free / 1e9)}
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=w.n_layers, n_shared=w.n_shared, max_tokens=1)
    load_ring(ctx, synth, w, w.n_layers, "stack32")
    ntok, warm = 24, 4
    X0 = torch.from_numpy(synth.activations(w.with_(T=ntok + warm), stream=5)).to(dev)
    r = X0.clone()
    x = torch.empty_like(X0)
    idx = torch.empty((w.n_layers, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.n_layers, w.k), dtype=torch.float32, device=dev)
    U = ctx.new_union(1)
    nu_total = []

    def token(i):
        # layer 0 takes x_0 itself; every later layer is one call: RMSNorm of
        # the residual, route, experts, combine
        cm.colimoe_route_forward(ctx.ctx, 0, X0[i].data_ptr(), 1, idx[0].data_ptr(), wts[0].data_ptr(), U.abi(),
                                 r[i].data_ptr(), cm.COLIMOE_FWD_AUTO)
        for l in range(1, w.n_layers):
            cm.colimoe_rmsnorm_route_forward(ctx.ctx, l, r[i].data_ptr(), 1, 1e-6, x[i].data_ptr(), idx[l].data_ptr(),
                                             wts[l].data_ptr(), U.abi(), cm.COLIMOE_FWD_AUTO)

    for i in range(warm):
        token(i)
    ctx.sync()
    ms = event_time(torch, stream, lambda: [token(i) for i in range(warm, warm + ntok)]) / ntok
    ctx.sync()
    kern = per_kernel(cm, ctx, lambda: [token(i) for i in range(warm, warm + 4)])
    gms = graph_time(torch, ctx, lambda: [token(i) for i in range(warm, warm + ntok)]) / ntok
    ctx.close()
    del ctx, X0, r, x
    torch.cuda.empty_cache()
    bytes_tok = w.n_layers * (w.k + w.n_shared) * w.expert_bytes
    gbs = bytes_tok / (ms * 1e-3) / 1e9
    return {"workload": "32-layer decode stack, d=6144 f=2048 E=256 top-8 + shared, Zipf(1.1) bias, RMSNorm "
                        "eps 1e-6 between layers, 1 token; all 32 layers resident (%.1f GB)" % (need / 1e9),
            "us_per_token": round(1000 * ms, 2), "tokens_per_s": round(1000.0 / ms, 1),
            "us_per_layer": round(1000 * ms / w.n_layers, 3), "int4_bytes_per_token": bytes_tok,
            "int4_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "tokens_timed": ntok,
            "graph_replay_us_per_token": round(1000 * gms, 2),
            "graph_replay_hbm_frac": round(bytes_tok / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernels": {k: round(v["avg_us"], 3) for k, v in kern.items()}}


def bench_tiny(args, torch, np, synth, cm, MoeContext, dev, stream):
    """The tiny layer (d=256 f=128 E=16 top-2, no shared expert), one token per
    call: latency-bound, its weights stay in the caches."""
    w = synth.WORKLOADS["tiny"]
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=1)
    load_ring(ctx, synth, w, 1, "tiny")
    n, warm = 400, 40
    X = torch.from_numpy(synth.activations(w.with_(T=n), stream=13)).to(dev)
    res = X.clone()
    idx = torch.empty((n, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((n, w.k), dtype=torch.float32, device=dev)
    U = ctx.new_union(1)

    def run(a, b):
        for i in range(a, b):
            cm.colimoe_route_forward(ctx.ctx, 0, X[i].data_ptr(), 1, idx[i].data_ptr(), wts[i].data_ptr(), U.abi(),
                                     res[i].data_ptr(), cm.COLIMOE_FWD_AUTO)

    run(0, warm)
    ctx.sync()
    ms, win = windowed_time(torch, stream, run, warm, n)
    gms = graph_time(torch, ctx, lambda: run(warm, n)) / (n - warm)
    ctx.close()
    del ctx, X, res
    return {"workload": "tiny MoE layer d=256 f=128 E=16 top-2, no shared expert, 1 token (fp32 path)",
            "us_per_call": round(1000 * ms, 3), "median_window_us": round(1000 * sorted(win)[2], 3),
            "graph_replay_us_per_call": round(1000 * gms, 3), "calls_timed": n - warm}


def bench_union16(args, torch, np, synth, cm, MoeContext, dev, stream):
    w = synth.WORKLOADS["union16"]
    ring = 4
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=ring, n_shared=w.n_shared, max_tokens=w.T)
    load_ring(ctx, synth, w, ring, "union16")
    nb, warm = 32, 4
    Xs = [torch.from_numpy(synth.activations(w, stream=100 + b)).to(dev) for b in range(nb + warm)]
    res = [x.clone() for x in Xs]
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    unions = [ctx.new_union(w.T) for _ in range(nb + warm)]

    def call(b):
        cm.colimoe_route_forward(ctx.ctx, b % ring, Xs[b].data_ptr(), w.T, idx.data_ptr(), wts.data_ptr(),
                                 unions[b].abi(), res[b].data_ptr(), cm.COLIMOE_FWD_AUTO)

    for b in range(warm):
        call(b)
    ctx.sync()
    ms = event_time(torch, stream, lambda: [call(b) for b in range(warm, warm + nb)]) / nb
    ctx.sync()
    kern = per_kernel(cm, ctx, lambda: [call(b) for b in range(warm, warm + nb)])
    nus = [int(unions[b].n_unique.item()) for b in range(warm, warm + nb)]
    ctx.close()
    del ctx
    torch.cuda.empty_cache()
    bytes_call = (float(np.mean(nus)) + w.n_shared) * w.expert_bytes
    gbs = bytes_call / (ms * 1e-3) / 1e9
    return {"workload": "batch-union call, 16 positions (pairwise correlation 0.6, Zipf(1.1) bias), d=6144 f=2048 "
                        "E=256 top-8 + shared", "us_per_call": round(1000 * ms, 2),
            "tokens_per_s": round(w.T * 1000.0 / ms, 1), "unique_experts_mean": round(float(np.mean(nus)), 2),
            "int4_bytes_per_call": int(bytes_call), "int4_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "calls_timed": nb,
            "kernels": {k: round(v["avg_us"], 3) for k, v in kern.items()}}


def bench_verify(args, torch, np, synth, cm, MoeContext, dev, stream):
    """T = 1..4 draft positions per call (batch-union recipe): the cost of each
    extra position in time and in expert bytes, with plain top-k and with the
    pages' expert top-p 0.7 (fewer experts read per position)."""
    w4 = synth.WORKLOADS["verify4"]
    ring = 4
    ctx = MoeContext(w4.d, w4.f, w4.E, w4.k, n_layers=ring, n_shared=w4.n_shared, max_tokens=w4.T)
    load_ring(ctx, synth, w4, ring, "verify")
    nb, warm = 48, 4
    out = {"workload": "multi-position verify: T = 1..4 positions per call (pairwise correlation 0.6, Zipf(1.1) "
                       "bias), d=6144 f=2048 E=256 top-8 + shared", "per_T": {}}
    # plain top-k, then the pages' expert top-p 0.7 on the same calls
    for p, key in ((1.0, "per_T"), (0.7, "per_T_top_p_0.7")):
        out.setdefault(key, {})
        ctx.set_expert_top_p(p)
        for T in (1, 2, 3, 4):
            w = w4.with_(T=T)
            Xs = [torch.from_numpy(synth.activations(w, stream=300 + b)).to(dev) for b in range(nb + warm)]
            res = [x.clone() for x in Xs]
            idx = torch.empty((T, w.k), dtype=torch.int32, device=dev)
            wts = torch.empty((T, w.k), dtype=torch.float32, device=dev)
            unions = [ctx.new_union(T) for _ in range(nb + warm)]

            def call(b):
                cm.colimoe_route_forward(ctx.ctx, b % ring, Xs[b].data_ptr(), T, idx.data_ptr(), wts.data_ptr(),
                                         unions[b].abi(), res[b].data_ptr(), cm.COLIMOE_FWD_AUTO)

            for b in range(warm):
                call(b)
            ctx.sync()
            ms = event_time(torch, stream, lambda: [call(b) for b in range(warm, warm + nb)]) / nb
            ctx.sync()
            kern = per_kernel(cm, ctx, lambda: [call(b) for b in range(warm, warm + nb)])
            nus = [int(unions[b].n_unique.item()) for b in range(warm, warm + nb)]
            bytes_call = (float(np.mean(nus)) + w.n_shared) * w.expert_bytes
            out[key][T] = {"us_per_call": round(1000 * ms, 2), "us_per_position": round(1000 * ms / T, 2),
                           "unique_experts_mean": round(float(np.mean(nus)), 2), "int4_bytes_per_call": int(bytes_call),
                           "int4_gbs": round(bytes_call / (ms * 1e-3) / 1e9, 1),
                           "kernels": {k: round(v["avg_us"], 3) for k, v in kern.items()}}
            del Xs, res, unions
    ctx.set_expert_top_p(1.0)
    ctx.close()
    del ctx
    torch.cuda.empty_cache()
    return out


def bench_tiered(args, torch, np, synth, cm, MoeContext, dev, stream):
    """Tiered placement: the first 4 layers of the stacked-decode recipe kept in
    pinned host memory, served through an HBM cache of 256 expert slots (64
    per layer: a quarter of each layer's 256 routed experts); one token at a
    time through the 4 layers.  Each layer call copies its routing to the host
    and streams the missing experts over PCIe, so the time is wall-clock time.
    Every configuration starts from a fresh cache, is warmed with the same 32
    tokens and timed on the same 32 other tokens: per-layer LRU alone; with the
    next layer's router run one layer ahead, prefetching the first `depth`
    experts of its prediction; and with the learned pin (each layer's most
    used experts pinned after the warm-up) or automatic repinning on top."""
    w = synth.WORKLOADS["stack32"].with_(n_layers=4)
    slots = 256
    per_layer = slots // w.n_layers
    n_pin = per_layer - w.n_shared - w.k
    ntok, warm = 32, 32
    X_warm = torch.from_numpy(synth.activations(w.with_(T=warm), stream=5)).to(dev)
    X_time = torch.from_numpy(synth.activations(w.with_(T=ntok), stream=6)).to(dev)
    blobs = [(synth.router(w, l), synth.bias(w, l), synth.expert_blobs(w, l, 0, w.E), synth.shared_blob(w, l))
             for l in range(w.n_layers)]

    def config(depth, pin=False, autorepin=0):
        ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=w.n_layers, n_shared=w.n_shared, max_tokens=1)
        ctx.set_expert_cache(slots)
        for l in range(w.n_layers):
            ctx.load_layer_host(l, *blobs[l])
        ctx.cache_set_prefetch(depth)
        if autorepin:
            ctx.cache_set_autorepin(autorepin, n_pin)
        idx = torch.empty((w.n_layers, w.k), dtype=torch.int32, device=dev)
        wts = torch.empty((w.n_layers, w.k), dtype=torch.float32, device=dev)
        U = ctx.new_union(1)

        def run(X0):
            r = X0.clone()
            x = torch.empty_like(X0)
            a = ctx.cache_info()
            t = time.perf_counter()
            for i in range(X0.shape[0]):
                cm.colimoe_route_forward(ctx.ctx, 0, X0[i].data_ptr(), 1, idx[0].data_ptr(), wts[0].data_ptr(),
                                         U.abi(), r[i].data_ptr(), cm.COLIMOE_FWD_AUTO)
                for l in range(1, w.n_layers):
                    cm.colimoe_rmsnorm_route_forward(ctx.ctx, l, r[i].data_ptr(), 1, 1e-6, x[i].data_ptr(),
                                                     idx[l].data_ptr(), wts[l].data_ptr(), U.abi(),
                                                     cm.COLIMOE_FWD_AUTO)
            ctx.sync()
            return time.perf_counter() - t, a, ctx.cache_info()

        run(X_warm)
        if pin:
            ctx.cache_repin(n_pin)
        dt, a, b = run(X_time)
        ctx.close()
        n = X_time.shape[0]
        hits, misses = b.hits - a.hits, b.misses - a.misses
        out = {"us_per_token": round(1e6 * dt / n, 1), "us_per_layer": round(1e6 * dt / n / w.n_layers, 1),
               "tokens_per_s": round(n / dt, 2), "hit_rate": round(hits / max(hits + misses, 1), 4),
               "misses_per_token": round(misses / n, 2), "pcie_gbs": round(misses * w.expert_bytes / dt / 1e9, 1)}
        pr = b.predicted - a.predicted
        if pr:
            pf = b.prefetched - a.prefetched
            out.update({"prediction_hit_rate": round((b.predicted_hits - a.predicted_hits) / pr, 4),
                        "prefetched_per_token": round(pf / n, 2),
                        "prefetched_used_per_token": round((b.prefetched_used - a.prefetched_used) / n, 2)})
        return out

    t0 = time.time()
    res = {"lru": config(0)}
    for depth in (1, 2, 4, w.k):
        res["prefetch%d" % depth] = config(depth)
    best = min((1, 2, 4, w.k), key=lambda d: res["prefetch%d" % d]["us_per_token"])
    res["learned_pin"] = config(0, pin=True)
    res["learned_pin_prefetch%d" % best] = config(best, pin=True)
    res["autorepin8_prefetch%d" % best] = config(best, autorepin=8)
    log("tiered: %d configurations in %.1f s" % (len(res), time.time() - t0))
    top = res["learned_pin_prefetch%d" % best]
    del X_warm, X_time, blobs
    torch.cuda.empty_cache()
    return {"workload": "tiered placement: 4 layers of the stacked-decode recipe (d=6144 f=2048 E=256 top-8 + shared, "
                        "Zipf(1.1) bias, RMSNorm between) with routed experts in pinned host memory (%.1f GB), an HBM "
                        "cache of %d expert slots (%.1f GB, %d per layer), 1 token; each configuration from a fresh "
                        "cache, warmed on the same %d tokens, timed on the same %d others" % (
                            w.n_layers * w.E * w.expert_bytes / 1e9, slots, slots * w.expert_bytes / 1e9,
                            per_layer, warm, ntok),
            "configs": res, "pinned_per_layer": n_pin, "best_prefetch_depth": best,
            "us_per_token": top["us_per_token"], "hit_rate": top["hit_rate"]}


def bench_int8(args, torch, np, synth, cm, MoeContext, dev, stream):
    """The decode layer with int8 gs64 experts (twice the int4 bytes), 1 token,
    on a ring of 4 independently generated layers (each token reads 356 MB,
    beyond the Infinity Cache)."""
    w = synth.WORKLOADS["decode"].with_(bits=8)
    ring = 4
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=ring, n_shared=w.n_shared, max_tokens=1,
                     cfg_flags=cm.COLIMOE_CFG_INT8)
    load_ring(ctx, synth, w, ring, "int8")
    nt, warm = 100, 10
    X = torch.from_numpy(synth.activations(w.with_(T=nt + warm), stream=12)).to(dev)
    res = X.clone()
    idx = torch.empty((nt + warm, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((nt + warm, w.k), dtype=torch.float32, device=dev)
    U = ctx.new_union(1)

    def step(i):
        cm.colimoe_route_forward(ctx.ctx, i % ring, X[i].data_ptr(), 1, idx[i].data_ptr(), wts[i].data_ptr(), U.abi(),
                                 res[i].data_ptr(), cm.COLIMOE_FWD_AUTO)

    for i in range(warm):
        step(i)
    ctx.sync()
    ms = event_time(torch, stream, lambda: [step(i) for i in range(warm, warm + nt)]) / nt
    ctx.sync()
    kern = per_kernel(cm, ctx, lambda: [step(i) for i in range(warm, warm + nt)])
    ctx.close()
    del ctx, X, res
    torch.cuda.empty_cache()
    bytes_tok = (w.k + w.n_shared) * w.expert_bytes
    gbs = bytes_tok / (ms * 1e-3) / 1e9
    return {"workload": "decode MoE layer with int8 gs64 experts, d=6144 f=2048 E=256 top-8 + shared, 1 token, ring "
                        "of %d layers" % ring, "us_per_token": round(1000 * ms, 2),
            "int8_bytes_per_token": bytes_tok, "int8_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "tokens_timed": nt, "kernels": {k: round(v["avg_us"], 3) for k, v in kern.items()}}


def bench_prefill(args, torch, np, synth, cm, MoeContext, dev, stream):
    w = synth.WORKLOADS["prefill2048"]
    ring = 2
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=ring, n_shared=w.n_shared, max_tokens=w.T)
    load_ring(ctx, synth, w, ring, "prefill2048")
    nb, warm = 8, 2
    X = torch.from_numpy(synth.activations(w, stream=0)).to(dev)
    res = X.clone()
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    U = ctx.new_union(w.T)

    def call(b):
        cm.colimoe_route_forward(ctx.ctx, b % ring, X.data_ptr(), w.T, idx.data_ptr(), wts.data_ptr(), U.abi(),
                                 res.data_ptr(), cm.COLIMOE_FWD_AUTO)

    for b in range(warm):
        call(b)
    ctx.sync()
    ms = event_time(torch, stream, lambda: [call(b) for b in range(warm, warm + nb)]) / nb
    ctx.sync()
    kern = per_kernel(cm, ctx, lambda: [call(b) for b in range(warm, warm + nb)])
    nu = int(U.n_unique.item())
    ctx.close()
    del ctx, X, res
    torch.cuda.empty_cache()
    pairs = w.T * w.k
    flops = 2.0 * 3 * w.d * w.f * (pairs + w.T * w.n_shared)
    gemm_us = kern.get("gateup", {}).get("avg_us", 0.0) + kern.get("down", {}).get("avg_us", 0.0)
    bytes_call = (nu + w.n_shared) * w.expert_bytes
    gbs = bytes_call / (ms * 1e-3) / 1e9
    return {"workload": "prefill call, 2048 tokens, Zipf(1.1) bias, d=6144 f=2048 E=256 top-8 + shared, bf16 MFMA "
                        "grouped GEMM", "ms_per_call": round(ms, 4), "tokens_per_s": round(w.T * 1000.0 / ms, 1),
            "unique_experts": nu, "expert_flops": flops,
            "mfma_util": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "mfma_util_gemm_kernels": round(flops / (gemm_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4) if gemm_us else None,
            "int4_bytes_per_call": bytes_call, "int4_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "calls_timed": nb, "kernels": {k: round(v["avg_us"], 3) for k, v in kern.items()}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import int4_routed_expert_fp32_amd as cm
    from int4_routed_expert_fp32_amd.runtime import MoeContext

    proto = host_protocol()  # before the GPU is initialised
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    proto.update(gpu_protocol(torch, dev))
    stream = torch.cuda.current_stream(dev)
    calibration_copy(torch, dev)
    ceiling = stream_ceiling(torch, dev, stream)
    log("read-only stream ceiling: %.1f GB/s" % ceiling["gbs"])
    common = (args, torch, np, synth, cm, MoeContext, dev, stream)

    extra = {}
    for name, fn in (("tiny", bench_tiny), ("stack32", bench_stack32), ("union16", bench_union16), ("verify", bench_verify),
                     ("prefill2048", bench_prefill), ("tiered", bench_tiered), ("int8", bench_int8)):
        if args.only in ("all", name):
            extra[name] = fn(*common)
            log("%s: %s" % (name, json.dumps({k: v for k, v in extra[name].items() if k != "kernels"})))
    if args.only not in ("all", "decode"):
        print(json.dumps(extra), flush=True)
        return

    w, ms_step, kern, other, topp, timing = bench_decode(*common)
    be = w.expert_bytes
    gu_bytes = 2 * (w.d * w.f // 2 + 2 * w.d * w.f // 64)     # gate+up int4 + fp16 scales of one expert
    dn_bytes = be - gu_bytes
    experts_touched = w.k + w.n_shared                         # T = 1: k distinct routed + shared
    # the fixed-point one-token path runs the shared expert's gate/up in the
    # top-k launch: the gate/up launch reads the k routed experts only
    gu_experts = w.k if args.path != "fp32" else experts_touched
    int4_bytes = experts_touched * be
    us_token = 1000.0 * ms_step
    gbs = int4_bytes / (ms_step * 1e-3) / 1e9
    gu_gbs = gu_experts * gu_bytes / (kern["gateup"]["avg_us"] * 1e-6) / 1e9
    dn_gbs = experts_touched * dn_bytes / (kern["down"]["avg_us"] * 1e-6) / 1e9
    roofline = dict(bound="hbm", kernel=DECODE_GATEUP_KERNEL, achieved=round(gu_gbs, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(gu_gbs / HBM_PEAK_GBS, 4), traffic=measured_traffic(DECODE_GATEUP_KERNEL),
                    bytes_per_launch=gu_experts * gu_bytes, avg_launch_us=round(kern["gateup"]["avg_us"], 3))

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        samples = []
        cpu = cpu_baseline(w, args.cpu_seconds, keep=samples)
        parity = parity_check(torch, np, synth, cm, MoeContext, dev, w, samples)

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
        "dtype": "int4 weights, fp32 accumulation" + (" (fixed-point activations, exact int4 dot)"
                                                        if args.path != "fp32" else " (fp32 dequant)"),
        "data": "synthetic (seeded int4 gs64 experts, fp16 scales, N(0,1) activations)",
        "config": {"workload": "decode MoE layer d=6144 f=2048 E=256 top-8 + 1 shared, 1 token",
                   "layer_ring": args.ring},
        "protocol": dict(proto, seed=w.seed, cache_state="experts resident in HBM; %d independently generated "
                         "layer instances cycled (%.1f GB between reuses of one layer's weights)" % (
                             args.ring, (args.ring - 1) * (w.E + w.n_shared) * w.expert_bytes / 1e9),
                         timed="%d steps after %d warmup steps, HIP events on the stream, in 5 consecutive "
                               "sub-windows" % (args.steps, args.warmup)),
        "timing": timing,
        "tokens_per_s": round(1e6 / us_token, 1),
        "int4_bytes_per_token": int4_bytes,
        "int4_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "stream_ceiling": ceiling,
        "frac_of_stream_ceiling": round(gbs / ceiling["gbs"], 4),
        "kernels": {k: {"avg_us": round(v["avg_us"], 3), "launches": v["launches"]} for k, v in kern.items()},
        "down_gbs": round(dn_gbs, 1),
        "path": args.path,
        "compare": other,
        "expert_top_p": topp,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "workloads": extra,
    }
    print(json.dumps(out), flush=True)


def _omp_threads(n=None):
    """OpenMP threads the oracle's parallel regions use: sets them when n is
    given (on this thread), returns the current setting."""
    import ctypes
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    if n is not None:
        gomp.omp_set_num_threads(int(n))
    return int(gomp.omp_get_max_threads())


ORACLE_STREAM = 11  # activation stream of the oracle's sample tokens


def _oracle_tokens(w, budget_s, max_tokens=64, keep=None):
    """us per token of the oracle (route + forward, fp64) on decode-shaped
    tokens of layer instance 0, within about budget_s seconds of oracle time;
    `keep` (a list) receives (token, logits, idx, out) of every token done."""
    import numpy as np

    import oracle
    import synth
    R = synth.router(w, 0)
    b = synth.bias(w, 0)
    shared = synth.shared_blob(w, 0) if w.n_shared else None
    X = synth.activations(w.with_(T=max_tokens), stream=ORACLE_STREAM)
    done, t_cpu = 0, 0.0
    blobs = {}
    while done < X.shape[0] and t_cpu < budget_s:
        x = X[done].astype(np.float64)
        t = time.perf_counter()
        l, idx, wt = oracle.route_token(R, b, x, w.k)
        t_cpu += time.perf_counter() - t
        for e in idx:  # input generation is not part of the timed work
            if int(e) not in blobs:
                blobs[int(e)] = synth.expert_blobs(w, 0, int(e), int(e) + 1)[0].copy()
        t = time.perf_counter()
        out, _ = oracle.moe_token(x, w.d, w.f, {int(e): blobs[int(e)] for e in idx}, shared, idx, wt, x, w.E)
        t_cpu += time.perf_counter() - t
        if keep is not None:
            keep.append((done, l, idx.copy(), out))
        done += 1
    return 1e6 * t_cpu / done, done, t_cpu


def cpu_baseline(w, budget_s, keep=None):
    """The oracle (route + forward, fp64) on a bounded sample of decode tokens,
    on the process's cores; then on one core, for the decode and the tiny
    layer.  `keep` receives the sample's oracle results (for the parity
    check)."""
    import oracle
    import synth
    oracle.build(force=False)
    cores = len(os.sched_getaffinity(0))
    threads = _omp_threads()
    us, done, t_cpu = _oracle_tokens(w, budget_s, keep=keep)
    prev = _omp_threads(1)
    one = {}
    for name, ww, budget in (("decode", w, max(4.0, budget_s / 3)), ("tiny", synth.WORKLOADS["tiny"], 1.0)):
        u1, d1, t1 = _oracle_tokens(ww, budget)
        one[name] = {"us_per_token": round(u1, 1), "tokens": d1, "seconds": round(t1, 2)}
    _omp_threads(threads if threads else prev)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "unknown")
    except OSError:
        pass
    return {"value": round(us, 1), "unit": "us/token", "cores": threads or cores, "kind": "oracle",
            "sample": "%d decode tokens of the same layer shape (layer instance 0), route + 8 routed + shared "
                      "expert in fp64, %.1f s" % (done, t_cpu),
            "cpu_model": model, "affinity_cores": cores, "omp_threads": threads, "one_core": one}


def parity_check(torch, np, synth, cm, MoeContext, dev, w, samples):
    """The library on the oracle sample's tokens (layer instance 0, residual =
    x, one call each, both fp32-class paths) against the oracle's outputs:
    worst |gpu - oracle| / (1e-3 (1 + |oracle|)) per path, tokens whose k-th
    and (k+1)-th oracle logits lie within 1e-5 (near-ties, where another
    routing is also correct), and routings that differ elsewhere."""
    ctx = MoeContext(w.d, w.f, w.E, w.k, n_layers=1, n_shared=w.n_shared, max_tokens=1)
    ctx.load_layer(0, synth.router(w, 0), synth.bias(w, 0), synth.expert_blobs(w, 0, 0, w.E),
                   synth.shared_blob(w, 0) if w.n_shared else None)
    X = synth.activations(w.with_(T=max(t for t, _, _, _ in samples) + 1), stream=ORACLE_STREAM)
    idx = torch.empty((1, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((1, w.k), dtype=torch.float32, device=dev)
    out = {"tokens": len(samples), "bound": "|gpu - oracle| <= 1e-3 (1 + |oracle|) per output",
           "oracle": "fp64, the cpu_baseline sample's tokens on layer instance 0, residual = x"}
    near = 0
    for t, l, _, _ in samples:
        ls = np.sort(l)[::-1]
        near += int(ls[w.k - 1] - ls[w.k] < 1e-5)
    out["near_ties"] = near
    for name, flag in (("fxp", cm.COLIMOE_FWD_FXP), ("fp32", cm.COLIMOE_FWD_FP32)):
        worst, differ, compared = 0.0, 0, 0
        for t, l, oidx, oout in samples:
            x = torch.from_numpy(X[t:t + 1]).to(dev)
            res = x.clone()
            cm.colimoe_route_forward(ctx.ctx, 0, x.data_ptr(), 1, idx.data_ptr(), wt.data_ptr(), None, res.data_ptr(),
                                     flag)
            ctx.sync()
            if set(idx.cpu().numpy()[0].tolist()) != set(oidx.tolist()):
                ls = np.sort(l)[::-1]
                differ += int(not ls[w.k - 1] - ls[w.k] < 1e-5)
                continue
            g = res.cpu().numpy()[0].astype(np.float64)
            worst = max(worst, float(np.max(np.abs(g - oout) / (1e-3 * (1.0 + np.abs(oout))))))
            compared += 1
        out[name] = {"worst_ratio_to_bound": round(worst, 4), "tokens_compared": compared,
                     "routing_mismatches": differ}
    ctx.close()
    del ctx
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
