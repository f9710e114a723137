"""Benchmark of the Muon optimizer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one full Muon step (momentum, Newton-Schulz with five iterations,
weight update) over every matrix of the workload, inputs resident in HBM.
Defaults: 3 untimed warm-up steps, 10 timed steps; `step_ms` gives the
median, p90, min and max of the per-step times from HIP events.
Default workload: the Kimi-K2-MoE-layer-shaped batch, 384 experts x
(2048x7168 gate, 2048x7168 up, 7168x2048 down) = 1152 bf16 matrices.

Prints one JSON line. `value` is Newton-Schulz TFLOP/s counted with the SYRK
saving (algorithmic FLOPs: upper triangles of the two symmetric products plus
the full B X) divided by the whole step time. `roofline` describes the
dominant kernel (largest share of step time): algorithmic FLOPs per launch
over its average launch duration, both taken live from HIP events that the
library records around each of its launches on the launch stream.
`cpu_baseline` times the CPU oracle (float32, numpy/BLAS on the host cores)
on a bounded sample of the same matrices.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12   # dense bf16 MFMA, 2516.6 TFLOP/s
# workspace of the timed run: three groups of 384 views for the MoE-layer
# batch (a 2048 x 7168 view takes 142.6 MB: X and X^T twice, A hi/lo, B)
WS_GB_DEFAULT = 56.0
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="kimi_moe_layer")
    p.add_argument("--workspace-gb", type=float, default=WS_GB_DEFAULT)
    p.add_argument("--pack", choices=["cost", "rr"], default="cost")
    p.add_argument("--aa", choices=["plain", "split"], default="plain",
                   help="A*A from bf16(A) (default) or from A as bf16 hi + lo")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="budget of the CPU-oracle sample (0 disables it)")
    p.add_argument("--no-phase-timing", action="store_true")
    p.add_argument("--matrices", type=int, default=0,
                   help="use only the first N matrices of the workload (diagnostics; 0 = all)")
    p.add_argument("--tp", type=int, default=0,
                   help="simulate the tensor-parallel (distributed) mode with this many column "
                        "shards per matrix on this one GPU; tall matrices enter transposed")
    p.add_argument("--adamw", action="store_true",
                   help="also time one AdamW step (float32 moments) over the same parameters, "
                        "for the Muon/AdamW optimizer-step ratio")
    p.add_argument("--place-ranks", type=int, default=0,
                   help="also place the matrices on R simulated data-parallel ranks, round robin "
                        "vs LPT, with costs measured per matrix shape (0 = off)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (3 times) and exit: the reference "
                        "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return p.parse_args()


class Sampler:
    """Socket power and shader clock sampled from sysfs (hwmon power1_input,
    pp_dpm_sclk) every few milliseconds in a background thread while the
    timed steps run. Reads files only; makes no GPU call."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        dev = "/sys/class/drm/card0/device"
        pw = glob.glob(dev + "/hwmon/hwmon*/power1_input")
        self.pw = pw[0] if pw else None
        self.sclk = dev + "/pp_dpm_sclk" if os.path.exists(dev + "/pp_dpm_sclk") else None
        self.period = period_s
        self.w, self.mhz = [], []
        self.stop = False
        self.th = threading.Thread(target=self.run, daemon=True)

    def read_sclk(self):
        with open(self.sclk) as f:
            for line in f:
                if "*" in line:
                    return float(line.split(":")[1].strip().lower().split("mhz")[0])
        return None

    def run(self):
        while not self.stop:
            try:
                if self.pw:
                    with open(self.pw) as f:
                        self.w.append(int(f.read()) / 1e6)
                if self.sclk:
                    v = self.read_sclk()
                    if v:
                        self.mhz.append(v)
            except (OSError, ValueError):
                pass
            time.sleep(self.period)

    def __enter__(self):
        self.th.start()
        return self

    def __exit__(self, *exc):
        self.stop = True
        self.th.join()

    def summary(self):
        out = {"source": "sysfs hwmon power1_input and pp_dpm_sclk, sampled every 5 ms over the timed steps",
               "samples": len(self.w)}
        if self.w:
            out["avg_w"] = round(sum(self.w) / len(self.w), 1)
            out["max_w"] = round(max(self.w), 1)
        if self.mhz:
            out["sclk_mhz_avg"] = round(sum(self.mhz) / len(self.mhz), 1)
        cap = None
        if self.pw:
            try:
                with open(self.pw.replace("power1_input", "power1_cap")) as f:
                    cap = int(f.read()) / 1e6
            except (OSError, ValueError):
                cap = None
        out["cap_w"] = cap
        return out


def environment():
    """Host, runtime and device facts recorded beside the numbers."""
    import platform
    import torch
    env = {"host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
           "python": platform.python_version(), "torch": torch.__version__, "hip": torch.version.hip}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    if torch.cuda.is_available():
        pr = torch.cuda.get_device_properties(0)
        env["device"] = pr.name
        env["gcn_arch"] = getattr(pr, "gcnArchName", None)
        env["compute_units"] = pr.multi_processor_count
    try:
        from threadpoolctl import threadpool_info
        env["blas"] = [{"api": i.get("internal_api"), "threads": i.get("num_threads"), "version": i.get("version")}
                       for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        env["blas"] = None
    return env


def cpu_baseline(wl, budget_s, col_blocks=None):
    """Time the CPU oracle (float32) on matrices of the workload until the
    budget is spent; report algorithmic TFLOP/s."""
    import numpy as np
    from muon_newton_schulz_03_amd import accounting as acc
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()
                       if i.get("internal_api") in ("openblas", "mkl", "blis")), default=0)
    except Exception:
        threads = 0
    if not threads:
        threads = len(os.sched_getaffinity(0))
    cb = wl.col_blocks if col_blocks is None else col_blocks
    rng = np.random.default_rng(wl.seed)
    shapes = list(dict.fromkeys(wl.shapes))  # distinct shapes, in order
    flops = 0.0
    done = []
    t0 = time.perf_counter()
    i = 0
    while True:
        r, c = shapes[i % len(shapes)]
        G = (rng.standard_normal((r, c)) * wl.std_g).astype(np.float32)
        M = (rng.standard_normal((r, c)) * wl.std_m).astype(np.float32)
        W = (rng.standard_normal((r, c)) * wl.std_w).astype(np.float32)
        t = time.perf_counter()
        oracle.muon_step(W, G, M, lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov, iters=wl.iters,
                         col_blocks=cb, dtype=np.float32)
        el = time.perf_counter() - t
        f = sum(acc.flops_algorithmic(*acc.wide(*v), wl.iters) for v in acc.views([(r, c)], cb))
        flops += f
        done.append((f"{r}x{c}", el))
        i += 1
        if time.perf_counter() - t0 > budget_s:
            break
    busy = sum(e for _, e in done)
    return {
        "value": round(flops / busy / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"float32 oracle muon_step on {len(done)} matrices "
                  f"({', '.join(sorted(set(s for s, _ in done)))}) of the same workload, "
                  f"{busy:.1f} s of CPU time",
    }


def measure_placement(mu, M, wl, ranks, mode):
    """Per-matrix Newton-Schulz cost measured on the GPU for every distinct
    shape (muon_ns_batched over up to 64 matrices of that shape, median of 3
    runs), then the placement of all matrices on `ranks` ranks, round robin
    against LPT (muon_place)."""
    import statistics
    import torch
    by_shape = {}
    for i, t in enumerate(M):
        by_shape.setdefault(tuple(t.shape), []).append(i)
    per_ms = {}
    for shape, idx in by_shape.items():
        sub = [M[i].clone() for i in idx[:64]]
        cb = [wl.col_blocks] * len(sub)
        mu.muon_ns_batched(sub, iters=wl.iters, mode=mode, col_blocks=cb)  # warm-up
        runs = []
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            mu.muon_ns_batched(sub, iters=wl.iters, mode=mode, col_blocks=cb)
            torch.cuda.synchronize()
            runs.append((time.perf_counter() - t0) * 1e3 / len(sub))
        per_ms[shape] = statistics.median(runs)
        del sub
    costs = [per_ms[tuple(t.shape)] for t in M]
    out = {"ranks": ranks,
           "cost": "measured muon_ns_batched ms per matrix, by shape (up to 64 matrices, median of 3)",
           "ms_per_matrix": {f"{r}x{c}": round(v, 4) for (r, c), v in per_ms.items()}}
    for pol in ("rr", "lpt"):
        _, load, imb = mu.muon_place(costs, ranks, pol)
        out[pol] = {"max_rank_ms": round(max(load), 3), "imbalance": round(imb, 4)}
    return out


def measure_adamw(mu, W, G, steps, warmup):
    """Time muon_adamw_step over the workload's parameters with float32
    moments; HBM bytes per element: read W, g, m, v and write W, m, v."""
    import torch
    Mo = [torch.zeros(t.shape, dtype=torch.float32, device=t.device) for t in W]
    V = [torch.zeros(t.shape, dtype=torch.float32, device=t.device) for t in W]
    kw = dict(lr=1e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    for k in range(warmup):
        mu.muon_adamw_step(W, G, Mo, V, step=k + 1, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        mu.muon_adamw_step(W, G, Mo, V, step=warmup + k + 1, **kw)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    es = W[0].element_size()
    nbytes = sum(t.numel() for t in W) * (3 * es + 16)
    return {"ms_per_step": round(ms, 3), "moments": "float32",
            "bytes_per_step": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def kernel_code_hash():
    """sha256 of the GEMM kernels' source (kernels.hip and layout.h) with the
    comments and blank space taken out, so that a comment edit does not void
    counters taken on the same code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in ("kernels.hip", "layout.h"):
        src = open(os.path.join(ROOT, "muon_newton_schulz_03_amd", "csrc", name)).read()
        src = re.sub(r"//[^\n]*", "", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` recorded in the profile summary for this
    workload, or None when there is none or the kernel code changed since."""
    import re
    path = os.path.join(ROOT, "profiles", f"muon_step_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^kernel_code_sha256: ([0-9a-f]{64})$", text, re.M)
    if not m or m.group(1) != kernel_code_hash():
        return None
    m = re.search(r"^traffic_bytes_per_launch " + re.escape(kernel) + r": (\d+)$", text, re.M)
    return int(m.group(1)) if m else None


def main():
    args = parse()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {args.calibrate_copy} MiB x 3", flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(no multi-GPU path is implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    import muon_newton_schulz_03_amd as mu
    from muon_newton_schulz_03_amd import accounting as acc
    from muon_newton_schulz_03_amd.workloads import WORKLOADS, make_inputs

    mu.load_library()
    wl = WORKLOADS[args.workload]
    if args.matrices:
        import dataclasses
        wl = dataclasses.replace(wl, name=f"{wl.name}[:{args.matrices}]", shapes=wl.shapes[:args.matrices])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mode = (mu.MUON_PACK_COST if args.pack == "cost" else mu.MUON_PACK_RR)
    mode |= mu.MUON_AA_SPLIT if args.aa == "split" else mu.MUON_AA_PLAIN
    if args.tp > 0:
        import dataclasses
        # distributed mode shards the long side of wide matrices: a tall
        # matrix enters transposed (same Newton-Schulz work)
        wl = dataclasses.replace(wl, name=f"{wl.name}_tp{args.tp}", col_blocks=args.tp,
                                 shapes=[(min(r, c), max(r, c)) for r, c in wl.shapes])
        mode |= mu.MUON_NS_DISTRIBUTED
    elif wl.col_blocks > 1:
        mode |= mu.MUON_NS_BLOCKWISE
    print(f"[bench] workload {wl.name}: {len(wl.shapes)} matrices; generating inputs", file=sys.stderr,
          flush=True)
    W, G, M = make_inputs(wl, device=dev)
    torch.cuda.synchronize()
    cb = [wl.col_blocks] * len(W)
    descs = [mu.mat_of(t, c) for t, c in zip(W, cb)]
    full = mu.muon_workspace_size(descs, mode)
    ws_bytes = min(full, int(args.workspace_gb * (1 << 30)))
    ws_bytes = max(ws_bytes, mu.muon_workspace_min_size(descs, mode))
    ws = mu.Workspace(ws_bytes, device=dev)
    plan = mu.muon_plan_info(descs, iters=wl.iters, mode=mode, workspace_bytes=ws_bytes)
    stream = torch.cuda.current_stream()

    def step():
        mu.muon_step(W, G, M, lr=wl.lr, beta=wl.beta, nesterov=wl.nesterov, iters=wl.iters,
                     mode=mode, col_blocks=cb, workspace=ws.buf[:ws_bytes])

    print(f"[bench] workspace {ws_bytes / 2**30:.1f} GiB, {len(plan['chunks'])} groups; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timing = not args.no_phase_timing
    if timing:
        mu.muon_set_phase_timing(True)
        mu.muon_phase_times()  # clear
    # per-step HIP events on the launch stream (the library launches on the
    # current stream), besides the wall clock around the whole timed region
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with Sampler() as sampler:
        t0 = time.perf_counter()
        ev[0].record(stream)
        for k in range(args.steps):
            step()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    per_step = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps))
    phases = mu.muon_phase_times() if timing else None
    mu.muon_set_phase_timing(False)
    ms_step = elapsed * 1e3 / args.steps
    print(f"[bench] {args.steps} steps, {ms_step:.2f} ms/step", file=sys.stderr, flush=True)

    blocks = 1 if args.tp > 0 else wl.col_blocks  # distributed mode computes the whole matrix
    f_nom, f_alg = acc.workload_flops(wl.shapes, wl.iters, blocks)
    g_f, a_f, b_f = acc.workload_phase_flops(wl.shapes, blocks)
    tflops_alg = f_alg / (ms_step * 1e-3) / 1e12
    tflops_nom = f_nom / (ms_step * 1e-3) / 1e12

    out = {
        "metric": "Newton-Schulz TFLOP/s (SYRK-counted) and % bf16 MFMA peak; Muon step ms/layer-set",
        "value": round(tflops_alg, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "matrices": len(wl.shapes),
            "col_blocks": wl.col_blocks,
            "iters": wl.iters,
            "pack": args.pack,
            "tp": args.tp,
            "aa": args.aa,
            "workspace_gib": round(ws_bytes / 2**30, 2),
            "groups": len(plan["chunks"]),
        },
        "step_ms": {"median": round(statistics.median(per_step), 3),
                    "p90": round(per_step[math.ceil(0.9 * len(per_step)) - 1], 3),
                    "min": round(per_step[0], 3), "max": round(per_step[-1], 3)},
        "power": sampler.summary(),
        "env": environment(),
        "tflops_nominal": round(tflops_nom, 2),
        "pct_peak_alg": round(100 * tflops_alg / PEAK_BF16_TFLOPS, 2),
        "pct_peak_nominal": round(100 * tflops_nom / PEAK_BF16_TFLOPS, 2),
    }
    if phases:
        per_step = {k: (v[0] / args.steps, v[1] // max(args.steps, 1)) for k, v in phases.items()
                    if k not in ("adamw", "reduce") or v[1] > 0}
        out["phase_ms_per_step"] = {k: round(v[0], 3) for k, v in per_step.items()}
        out["launches_per_step"] = {k: int(v[1]) for k, v in per_step.items()}
        ns_ms = sum(per_step[k][0] for k in ("norm", "gram", "aa", "bx"))
        out["ns_ms_per_step"] = round(ns_ms, 3)
        out["ns_tflops_alg"] = round(f_alg / (ns_ms * 1e-3) / 1e12, 2)
        out["ns_pct_peak_alg"] = round(100 * out["ns_tflops_alg"] / PEAK_BF16_TFLOPS, 2)
        flops_of = {"gram": g_f * wl.iters, "aa": a_f * wl.iters, "bx": b_f * wl.iters}
        dom = max(("gram", "aa", "bx"), key=lambda k: per_step[k][0])
        launches = max(per_step[dom][1], 1)
        avg_ms = per_step[dom][0] / launches
        fl_launch = flops_of[dom] / launches
        ach = fl_launch / (avg_ms * 1e-3) / 1e12
        out["roofline"] = {
            "bound": "mfma",
            "kernel": {"gram": "gemm_bf16_kernel<0> (SYRK Gram)", "aa": "gemm_bf16_kernel<1> (SYRK A*A + poly)",
                       "bx": "gemm_bf16_kernel<2> (GEMM B*X + (a + diag B) X)"}[dom],
            "achieved": round(ach, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": (recorded_traffic(wl.name, {"gram": "gemm_bf16_kernel<0>", "aa": "gemm_bf16_kernel<1>",
                                                   "bx": "gemm_bf16_kernel<2>"}[dom])
                        if args.pack == "cost" and args.aa == "plain" and args.workspace_gb == WS_GB_DEFAULT
                        else None),
            "flops_per_launch": fl_launch,
            "avg_launch_ms": round(avg_ms, 4),
        }
        mhz = out["power"].get("sclk_mhz_avg")
        if mhz:
            # the same work against the peak at the shader clock measured during the run
            out["roofline"]["frac_at_measured_clock"] = round(ach / (256 * 4096 * mhz * 1e6 / 1e12), 4)
        pb = acc.prep_bytes(wl.shapes, 2 if wl.dtype == "bf16" else 4,
                            transposed=wl.dtype == "bf16" and wl.iters > 0)
        out["prep_gbs"] = round(pb / (per_step["prep"][0] * 1e-3) / 1e9, 1) if per_step["prep"][0] > 0 else None
        out["prep_frac_hbm"] = round(out["prep_gbs"] / PEAK_HBM_GBS, 4) if out["prep_gbs"] else None
    if args.tp > 0 and phases:
        P = args.tp
        red = per_step.get("reduce", (0.0, 0))[0]
        out["distributed"] = {
            "shards": P,
            "note": "all P shards run on this GPU; A*A runs once per shard (redundantly, as on every rank); "
                    "the packed-triangle sum stands in for the all-reduce",
            "reduce_ms_per_step": round(red, 3),
            "per_rank_ms_estimate": round((per_step["gram"][0] + per_step["aa"][0] + per_step["bx"][0]
                                           + per_step["prep"][0] + per_step["finish"][0]) / P
                                          + per_step["norm"][0] + red / P, 3),
        }
    if args.place_ranks > 0:
        print(f"[bench] placement over {args.place_ranks} simulated ranks", file=sys.stderr, flush=True)
        out["placement"] = measure_placement(mu, M, wl, args.place_ranks, mode)
    if args.adamw:
        print("[bench] timing AdamW over the same parameters", file=sys.stderr, flush=True)
        del ws
        M.clear()
        torch.cuda.empty_cache()
        out["adamw"] = measure_adamw(mu, W, G, args.steps, args.warmup)
        out["adamw"]["muon_over_adamw"] = round(ms_step / out["adamw"]["ms_per_step"], 2)
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, col_blocks=blocks)
        # the sample's rate stands for the whole workload: the CPU time one
        # full step would take at that rate
        out["cpu_baseline"]["extrapolated_step_s"] = round(f_alg / (out["cpu_baseline"]["value"] * 1e12), 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
