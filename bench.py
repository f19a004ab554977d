"""Benchmark of the LatentMoE layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config readme_acc] [--no-cpu-baseline]

One step = one forward of the whole layer (router + top-K', dispatch order,
down-projection and shared experts, both grouped expert GEMMs, combine,
up-projection) over one batch of seeded synthetic tokens already resident in
HBM.  Prints one JSON line: whole-job tokens/s, the roofline position of the
dominant kernel (timed with HIP events on the forward's stream during the
timed steps), and the fp64 CPU oracle timed on a bounded token sample.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LatentMoE layer fwd tokens/s at 1 GPU; % bf16 MFMA peak / % HBM BW"
PEAK = {"bf16": 2500.0, "f32": 157.3}      # dense MFMA TFLOP/s (MI355X published)
HBM_PEAK_GBS = 8000.0


def stage_work(sh, T):
    """Algorithmic work per launch of each stage: (kind, amount)."""
    P = T * sh.top_k
    es = 2 if sh.dtype == "bf16" else 4
    ldzh = sh.l + sh.n_shared * sh.m_shared
    return {
        # one pass over x: router scores, z and the shared-expert hidden layer
        "gemm_x_router_down_shared1": ("flop", 2.0 * T * sh.d * (sh.n_experts + ldzh)),
        "grouped_gemm1_relu2": ("flop", 2.0 * P * sh.l * sh.m),
        "grouped_gemm2": ("flop", 2.0 * P * sh.m * sh.l),
        "gemm_up_shared2": ("flop", 2.0 * T * ldzh * sh.d),
        # gather P rows of l, write T rows of l, read pos and gate
        "combine": ("byte", float(P * sh.l * es + T * sh.l * es + P * 8)),
        # read the T x N' fp32 scores, write idx/gate/rank (12 bytes per slot)
        "router_select": ("byte", float(T * sh.n_experts * 4 + P * 12)),
        "dispatch_scan": ("byte", None),
        "dispatch_finalize": ("byte", None),
    }


def kernel_source_sha() -> str:
    import glob
    import hashlib
    src = sorted(glob.glob(os.path.join(ROOT, "mixture_experts_layer_latentmoe_amd", "csrc", "*")))
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in src)).hexdigest()[:16]


def profiled_traffic(cfg: str, stage: str):
    """HBM bytes per launch of `stage` from the committed rocprofv3 counter
    summary (FETCH_SIZE / WRITE_SIZE scaled by a copy kernel of known size),
    or None when there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{cfg}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    sha, val = None, None
    for line in open(path):
        if line.startswith("# kernel sources sha256[:16] of csrc/*:"):
            sha = line.split(":")[-1].strip()
        if line.startswith(f"traffic_bytes[{stage}]:"):
            val = float(line.split(":")[-1])
    return val if (sha == kernel_source_sha() and val is not None) else None


def cpu_baseline(wl, target_s=12.0):
    """The oracle as it stands, on all host threads, on a bounded sample."""
    from oracle import oracle
    T = wl.shape.T
    rng = np.random.default_rng(123)
    n = min(T, 8)
    toks = np.sort(rng.choice(T, size=n, replace=False))
    t0 = time.perf_counter()
    oracle.forward(wl, tokens=toks, want=("y",))
    dt = time.perf_counter() - t0
    per_tok = dt / n
    n2 = int(min(T, max(n, target_s / max(per_tok, 1e-9))))
    toks = np.sort(rng.choice(T, size=n2, replace=False))
    t0 = time.perf_counter()
    oracle.forward(wl, tokens=toks, want=("y",))
    dt = time.perf_counter() - t0
    return {"value": n2 / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{n2} of {T} tokens (seeded), full layer per token in fp64, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="readme_acc")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stage-timing", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain elementwise copy of 256 MiB (3 launches) so that profiler "
                         "byte counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); this layer is measured on one "
              "GPU's share and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_latentmoe_amd import _abi
    from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
    from synth import get_config, make_workload

    sh = get_config(args.config)
    print(f"[bench] generating {sh.name} (seeded)", file=sys.stderr, flush=True)
    wl = make_workload(sh)
    dev = "cuda:0"
    layer = LatentMoE.from_workload(wl, device=dev)
    x = to_device(wl.tensors["x"], sh.dtype, dev)
    y = torch.empty_like(x)
    T = sh.T
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer.forward(x, y)
    torch.cuda.synchronize()

    timing = not args.no_stage_timing
    if timing:
        _abi.latentmoe_profile_begin(layer.handle, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.forward(x, y)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    stages = _abi.latentmoe_profile_end(layer.handle) if timing else {}
    print(f"[bench] timed {args.steps} steps in {dt:.3f} s", file=sys.stderr, flush=True)

    ms_per_step = dt / args.steps * 1e3
    value = T * args.steps / dt
    work = stage_work(sh, T)
    stage_out = {}
    roof = None
    if stages:
        for name, (ms, n) in stages.items():
            if n:
                avg_us = ms / n * 1e3
                kind, amt = work.get(name, ("byte", None))
                e = {"avg_us": round(avg_us, 2), "launches": n}
                if amt is not None:
                    if kind == "flop":
                        e["tflops"] = round(amt / (avg_us * 1e-6) / 1e12, 1)
                    else:
                        e["gbs"] = round(amt / (avg_us * 1e-6) / 1e9, 1)
                stage_out[name] = e
        dom = max((k for k in stage_out if work.get(k, ("", None))[1] is not None),
                  key=lambda k: stage_out[k]["avg_us"])
        kind, amt = work[dom]
        avg_s = stage_out[dom]["avg_us"] * 1e-6
        if kind == "flop":
            ach = amt / avg_s / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK[sh.dtype],
                    "unit": "TFLOP/s", "frac": round(ach / PEAK[sh.dtype], 4),
                    "traffic": profiled_traffic(sh.name, dom)}
        else:
            ach = amt / avg_s / 1e9
            roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": profiled_traffic(sh.name, dom)}
    total_flop = sum(a for k, (kd, a) in work.items() if kd == "flop")
    layer.close()
    if args.copy_calibration:
        # reads 256 MiB and writes 256 MiB per launch
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.add(a, 0.0, out=b)
        torch.cuda.synchronize()

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": f"{sh.name}: LatentMoE layer forward, T={T} d={sh.d} l={sh.l} m={sh.m} "
                               f"N'={sh.n_experts} K'={sh.top_k} S={sh.n_shared}x{sh.m_shared} "
                               f"{sh.variant} {sh.dtype}", "tokens": T},
        "layer_tflops": round(total_flop / (ms_per_step * 1e-3) / 1e12, 1),
        "roofline": roof, "cpu_baseline": cpu, "stages": stage_out,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
