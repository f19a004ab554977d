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


def stage_work(sh, T, n_active):
    """Algorithmic work per launch of each stage: (flop, bytes).

    bytes counts every operand once: weights, activations read, outputs
    written.  n_active = experts that receive at least one token (the grouped
    GEMMs stream only those experts' weights).  None = not counted."""
    P = T * sh.top_k
    es = 2 if sh.dtype == "bf16" else 4
    fp8 = sh.expert_dtype == "fp8"
    ew = 1 if fp8 else es            # bytes per routed-expert weight
    ms = sh.n_shared * sh.m_shared
    ldzh = sh.l + ms
    N, d, l, m = sh.n_experts, sh.d, sh.l, sh.m
    g = 2 if sh.expert_act == "swiglu" else 1  # gated: a gate matrix beside each W1
    nx = N + l + g * ms                         # B columns of the pass over x
    return {
        # one pass over x: router scores (fp32 out), z and the shared-expert hidden layer
        "gemm_x_router_down_shared1": (2.0 * T * d * nx,
                                       es * (T * d + d * nx + T * ldzh) + 4.0 * T * N),
        # expert weights (+ their fp32 column scales for E4M3 banks), rows in and out
        "grouped_gemm1_relu2": (2.0 * P * l * m * g, g * (ew * n_active * l * m + (4.0 * n_active * m if fp8 else 0.0))
                                + es * (P * l + P * m) + 4.0 * P),
        "grouped_gemm2": (2.0 * P * m * l, ew * n_active * m * l + (4.0 * n_active * l if fp8 else 0.0)
                          + es * (P * m + P * l)),
        "gemm_up_shared2": (2.0 * T * ldzh * d, es * (ldzh * d + T * ldzh + T * d)),
        # gather P rows of l, write T rows of l, read pos and gate
        "combine": (None, float(P * l * es + T * l * es + P * 8)),
        # read the T x N' fp32 scores, write idx/gate/rank (12 bytes per slot)
        "router_select": (None, float(T * N * 4 + P * 12)),
        "dispatch_scan": (None, None),
        "dispatch_finalize": (None, None),
    }


def roofline_of(flop, nbytes, avg_s, dtype):
    """Position of one kernel against the roof that bounds it: MFMA when its
    flops take longer at peak than its bytes at HBM peak, else HBM."""
    t_mfma = flop / (PEAK[dtype] * 1e12) if flop else 0.0
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) if nbytes else 0.0
    if flop and t_mfma >= t_hbm:
        ach = flop / avg_s / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK[dtype], "unit": "TFLOP/s",
                "frac": round(ach / PEAK[dtype], 4)}
    ach = nbytes / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4)}


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


def weight_bytes(sh) -> int:
    """Bytes of one repacked copy of the layer's weights."""
    es = 4 if sh.dtype == "f32" else 2
    eb = 1 if sh.expert_dtype == "fp8" else es
    mats = 3 if sh.expert_act == "swiglu" else 2
    dense = sh.d * (sh.n_experts + sh.l) + sh.l * sh.d + mats * sh.n_shared * sh.d * sh.m_shared
    return 2 * dense * es + mats * sh.n_experts * sh.l * sh.m * eb  # the dense part twice: tiled + fragment-major


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="readme_acc")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stage-timing", action="store_true")
    ap.add_argument("--weight-copies", type=int, default=0,
                    help="independently repacked weight copies that consecutive steps rotate through "
                         "(0: enough for 2 GB of weights, at least 2, at most 8), so that no step finds "
                         "its weights in the 256 MB last-level cache from the step before")
    ap.add_argument("--backward", action="store_true",
                    help="also time the layer's backward pass (its forward recompute included) over the same "
                         "steps and report it under \"backward\"")
    ap.add_argument("--graph", action="store_true",
                    help="also replay the forward from captured HIP graphs (one per weight copy) over the same "
                         "steps and report it under \"graph\"; the headline value stays the eager forward")
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
    R = args.weight_copies or min(8, max(2, -(-2_000_000_000 // weight_bytes(sh))))
    layers = [LatentMoE.from_workload(wl, device=dev) for _ in range(R)]
    layer = layers[0]
    x = to_device(wl.tensors["x"], sh.dtype, dev)
    y = torch.empty_like(x)
    T = sh.T
    print(f"[bench] {R} weight copies; warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(max(args.warmup, R)):
        layers[i % R].forward(x, y)
    torch.cuda.synchronize()

    def profile_begin(n, mask=_abi.ALL_STAGES):
        for L in layers:
            _abi.latentmoe_profile_begin(L.handle, n, mask)

    def profile_end():
        tot = {}
        for L in layers:
            for k, (ms, n) in _abi.latentmoe_profile_end(L.handle).items():
                a, b = tot.get(k, (0.0, 0))
                tot[k] = (a + ms, b + n)
        return tot

    timing = not args.no_stage_timing
    counts = layer.forward_debug(x, want=("counts",))["counts"].cpu().numpy()
    n_active = int((counts > 0).sum())
    work = stage_work(sh, T, n_active)
    names = {_abi.latentmoe_stage_name(i): i for i in range(_abi.LATENTMOE_MAX_STAGES)
             if _abi.latentmoe_stage_name(i)}

    def stage_table(stages):
        out = {}
        for name, (ms, n) in stages.items():
            if n:
                avg_us = ms / n * 1e3
                flop, nbytes = work.get(name, (None, None))
                e = {"avg_us": round(avg_us, 2), "launches": n}
                if flop:
                    e["tflops"] = round(flop / (avg_us * 1e-6) / 1e12, 1)
                if nbytes:
                    e["gbs"] = round(nbytes / (avg_us * 1e-6) / 1e9, 1)
                if flop or nbytes:
                    r = roofline_of(flop, nbytes, avg_us * 1e-6, sh.dtype)
                    e["bound"], e["frac"] = r["bound"], r["frac"]
                out[name] = e
        return out

    # Untimed pass with every stage timed: the per-stage breakdown, and which
    # stage dominates.  (Two event records per stage and forward cost a few
    # microseconds each, too much to leave in the timed region.)
    stage_out, dom = {}, None
    if timing:
        nb = min(args.steps, 10)
        profile_begin(nb)
        for i in range(nb):
            layers[i % R].forward(x, y)
        stage_out = stage_table(profile_end())
        dom = max((k for k in stage_out if "frac" in stage_out[k]), key=lambda k: stage_out[k]["avg_us"])
        # the timed region records events around the dominant stage only
        profile_begin(args.steps, 1 << names[dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        layers[i % R].forward(x, y)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {dt:.3f} s", file=sys.stderr, flush=True)
    ms_per_step = dt / args.steps * 1e3
    value = T * args.steps / dt
    roof = None
    if timing:
        timed = stage_table(profile_end())[dom]
        flop, nbytes = work[dom]
        roof = {"kernel": dom, **roofline_of(flop, nbytes, timed["avg_us"] * 1e-6, sh.dtype),
                "avg_us": timed["avg_us"], "launches": timed["launches"],
                "traffic": profiled_traffic(sh.name, dom)}
    total_flop = sum(f for f, _ in work.values() if f)
    graph_out = None
    if args.graph:
        # one graph per weight copy, captured on a side stream after a warm-up
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for L in layers:
                L.forward(x, y)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for L in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                L.forward(x, y)
            graphs.append(g)
        for i in range(max(args.warmup, R)):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        tg = (time.perf_counter() - tg0) / args.steps
        graph_out = {"ms_per_step": round(tg * 1e3, 4), "tokens_per_s": round(T / tg, 1),
                     "note": "forward replayed from HIP graphs, same weight-copy rotation"}
        del graphs
    bwd = None
    if args.backward and sh.expert_dtype != "fp8":
        # algorithmic work: the recomputed forward (no up-projection), the
        # data gradients and the weight gradients of every GEMM: 3F - F_up
        gemm_flop = total_flop - work["gemm_up_shared2"][0] + 2.0 * total_flop
        dy = torch.randn_like(x)
        for i in range(max(2, R)):
            layers[i % R].backward(x, dy)
        torch.cuda.synchronize()
        tb0 = time.perf_counter()
        for i in range(args.steps):
            layers[i % R].backward(x, dy)
        torch.cuda.synchronize()
        tb = (time.perf_counter() - tb0) / args.steps
        bwd = {"ms_per_step": round(tb * 1e3, 4), "tokens_per_s": round(T / tb, 1),
               "algorithmic_tflops": round(gemm_flop / tb / 1e12, 1),
               "note": "forward recompute + data and weight gradients (fp32), weight copies rotated as above"}
        print(f"[bench] backward {args.steps} steps in {tb * args.steps:.3f} s", file=sys.stderr, flush=True)
    for L in layers:
        L.close()
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
                               f"{sh.variant} {sh.dtype}"
                               + (" (routed experts E4M3 + per-column scales)" if sh.expert_dtype == "fp8" else "")
                               + (" SwiGLU experts" if sh.expert_act == "swiglu" else ""),
                   "tokens": T, "experts_with_tokens": n_active, "weight_copies": R},
        "layer_tflops": round(total_flop / (ms_per_step * 1e-3) / 1e12, 1),
        "roofline": roof, "cpu_baseline": cpu, "stages": stage_out,
        **({"backward": bwd} if bwd else {}),
        **({"graph": graph_out} if graph_out else {}),
        "stages_note": "per-stage HIP-event times from an untimed pass of min(steps, 10) forwards; "
                       "roofline.avg_us is the dominant kernel timed over the timed region",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
