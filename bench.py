"""Benchmark of the LatentMoE layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config wide_prefill] [--also readme_acc,...]
                    [--no-cpu-baseline]

One step = one forward of the whole layer (router + top-K', dispatch order,
down-projection and shared experts, both grouped expert GEMMs, combine,
up-projection) over one batch of seeded synthetic tokens already resident in
HBM.  Prints one JSON line: whole-job tokens/s of the headline workload
(wide_prefill, the largest of the named single-GPU workloads), the roofline
position of its dominant kernel (timed with HIP events on the forward's
stream over a second run of the K timed steps: the throughput steps record no
events, which cost the stream about 3 us each), the fp64 CPU oracle timed on a
bounded token
sample, and the same measurements for the other named workloads under
"workloads".

Algorithmic work of a kernel: its flops, and the bytes of the weights it
touches plus its own inputs and outputs as the layer defines them (x, z and
the gathered z rows, Y, u, y).  Intermediates that exist only because the
layer runs as separate kernels -- the hidden activations H between the two
expert GEMMs where they run unfused, and the fp32 router scores between the
pass over x and the selection -- are reported as staged bytes beside it, not
counted.  A kernel's roof is MFMA when its flops at peak take longer than its
algorithmic bytes at HBM peak, else HBM.
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
HEADLINE = "wide_prefill"
ALSO = "readme_acc,zipf_skew,decode_eff,decode_eff_fp8"


def stage_work(sh, T, n_active):
    """Algorithmic work per launch of each stage: (flop, algorithmic bytes,
    staged bytes).  n_active = experts that receive at least one token (the
    grouped GEMMs stream only those experts' weights).  None = not counted."""
    P = T * sh.top_k
    es = 2 if sh.dtype == "bf16" else 4
    fp8 = sh.expert_dtype == "fp8"
    ew = 1 if fp8 else es            # bytes per routed-expert weight
    ms = sh.n_shared * sh.m_shared
    ldzh = sh.l + ms
    N, d, l, m = sh.n_experts, sh.d, sh.l, sh.m
    g = 2 if sh.expert_act == "swiglu" else 1  # gated: a gate matrix beside each W1
    nx = N + l + g * ms                         # B columns of the pass over x
    w1 = g * (ew * n_active * l * m + (4.0 * n_active * m if fp8 else 0.0))
    w2 = ew * n_active * m * l + (4.0 * n_active * l if fp8 else 0.0)
    return {
        # one pass over x: z and the shared-expert hidden layer out; the fp32
        # router scores are staged for the selection
        "gemm_x_router_down_shared1": (2.0 * T * d * nx, es * (T * d + d * nx + T * ldzh), 4.0 * T * N),
        # scores in, experts and gates out
        "router_select": (None, float(T * N * 4 + P * 8), float(P * 4)),
        "dispatch_scan": (None, None, None),
        "dispatch_finalize": (None, None, None),
        # W1 of the active experts, the gathered z rows (and their indices) in;
        # H out is staged
        "grouped_gemm1_relu2": (2.0 * P * l * m * g, w1 + es * P * l + 4.0 * P, float(es * P * m)),
        # W2 of the active experts, Y out; H in is staged
        "grouped_gemm2": (2.0 * P * m * l, w2 + es * P * l, float(es * P * m)),
        # both expert GEMMs in one kernel, H on chip: W1 and W2 of the active
        # experts, the gathered z rows (and their indices) in, Y out
        "expert_mlp": (2.0 * P * l * m * (g + 1), w1 + w2 + es * P * l + 4.0 * P + es * P * l, 0.0),
        # Y rows gathered, u written, positions and gates read
        "combine": (None, float(P * l * es + T * l * es + P * 8), 0.0),
        "gemm_up_shared2": (2.0 * T * ldzh * d, es * (ldzh * d + T * ldzh + T * d), 0.0),
    }


def layer_work(sh, T, n_active):
    """The whole layer: flops of every GEMM, and the bytes of the weights it
    touches plus x in and y out."""
    es = 2 if sh.dtype == "bf16" else 4
    ew = 1 if sh.expert_dtype == "fp8" else es
    g = 2 if sh.expert_act == "swiglu" else 1
    ms = sh.n_shared * sh.m_shared
    N, d, l, m = sh.n_experts, sh.d, sh.l, sh.m
    w = (es * d * (N + l + g * ms) + es * (l + ms) * d + ew * n_active * (g + 1) * l * m
         + (4.0 * n_active * (g * m + l) if sh.expert_dtype == "fp8" else 0.0))
    # every GEMM once: the fused expert MLP's flops are those of the two grouped GEMMs
    flop = sum(f for k, (f, _, _) in stage_work(sh, T, n_active).items() if f and k != "expert_mlp")
    return flop, w + 2.0 * es * T * d


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


# ---- rocprofv3 summaries (profiles/*.txt) -----------------------------------

STAGE_OF_TAG = {0: "gemm_x_router_down_shared1", 1: "grouped_gemm1_relu2", 2: "grouped_gemm2", 3: "gemm_up_shared2",
                4: "backward_dgrad", 5: "backward_wgrad", 6: "backward_wgrad_experts", 7: "backward_x_recompute",
                8: "backward_gemm1_recompute"}
# kernel template -> position of the stage tag among its integer arguments
# (-1: the last one)
TAG_POS = {"gemm_kernel": 7, "skinny_gemm_kernel": -1, "fewrow_split_kernel": -1, "gemm_tn_kernel": 0}
FIXED_STAGE = {"expert_mlp_kernel": "expert_mlp", "router_select_kernel": "router_select",
               "route_tiny_kernel": "router_select", "dispatch_small_kernel": "dispatch_finalize",
               "finalize_kernel": "dispatch_finalize", "chunk_scan_kernel": "dispatch_scan",
               "combine_kernel": "combine", "splitk_reduce_kernel": "splitk_reduce",
               "transpose_kernel": "repack_transpose (create only)",
               "fragmajor_kernel": "repack_fragmajor (create only)",
               # the backward's element-wise and re-layout kernels
               "xpass_act_kernel": "backward_x_recompute_act", "gather_sum8_kernel": "backward_gather_sum",
               "shared_act_grad_kernel": "backward_shared_act_grad",
               "gate_combine_grad_kernel": "backward_gate_combine_grad", "retile_kernel": "backward_retile",
               "split_cols_kernel": "backward_split_cols", "gather_rows_kernel": "backward_gather_rows"}


def stage_of_kernel(name: str) -> str:
    """Layer stage of a kernel symbol as rocprofv3 prints it (mangled or not)."""
    import re
    for k, st in FIXED_STAGE.items():
        if k in name:
            return st
    for k, pos in TAG_POS.items():
        if re.search(r"(^|[^a-z_])" + k, name):
            if "<" in name:  # demangled: the integer (and bool) arguments in order
                vals = [a.strip() for a in name[name.index("<") + 1:name.rindex(">")].split(",")]
                ints = [int(v == "true") if v in ("true", "false") else int(v) for v in vals
                        if v in ("true", "false") or v.lstrip("-").isdigit()]
            else:            # mangled: Li<n>E / Lb<n>E in order
                ints = [int(v) for v in re.findall(r"L[ib](\d+)E", name)]
            if not ints or len(ints) <= pos:
                return k
            return STAGE_OF_TAG.get(ints[pos], f"{k}[{ints[pos]}]")
    if "elementwise" in name or "vectorized" in name:
        return "torch elementwise (the copy calibration in traffic runs)"
    return name.split("(")[0][:60]


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def summarize_trace(d):
    """Per stage: launches, average / min / max kernel duration (us)."""
    import csv
    dur = {}
    for f in _csvs(d, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            st = stage_of_kernel(r["Kernel_Name"])
            dur.setdefault(st, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"{'stage / kernel':44s} {'calls':>6s} {'avg_us':>12s} {'min_us':>12s} {'max_us':>12s}"]
    for st, v in sorted(dur.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
        lines.append(f"{st:44s} {len(v):6d} {sum(v) / len(v):12.2f} {min(v):12.2f} {max(v):12.2f}")
    return "\n".join(lines)


def _counters(d):
    import csv
    per = {}  # stage -> counter -> [per-dispatch value]
    dur = {}
    for f in _csvs(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            st = stage_of_kernel(r["Kernel_Name"])
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per.setdefault(st, {}).setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            per[st][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
            if "End_Timestamp" in r and r.get("End_Timestamp"):
                dur.setdefault(st, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return per, dur


def summarize_pmc(d):
    """Per stage: the average per dispatch of every counter collected, and
    derived figures where their inputs are there: MFMA busy share of the
    shader cycles (SQ_VALU_MFMA_BUSY_CYCLES over 4 SIMDs x 256 CUs of
    GRBM_GUI_ACTIVE / 8 XCDs), the share of cycles the vector L1s wait on
    pending misses (TCP_PENDING_STALL_CYCLES summed over the 256 L1s, over 256
    x GRBM_GUI_ACTIVE / 8), the L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))
    and the effective shader clock (GRBM_GUI_ACTIVE / 8 per kernel time)."""
    per, dur = _counters(d)
    lines = []
    for st in sorted(per):
        c = {k: sum(v.values()) / len(v) for k, v in per[st].items()}
        n = max(len(v) for v in per[st].values())
        us = dur.get(st, {})
        avg_us = sum(us.values()) / len(us) if us else None
        parts = [f"{k}={v:.6g}" for k, v in sorted(c.items())]
        der = []
        if "GRBM_GUI_ACTIVE" in c and avg_us:
            der.append(f"shader_clock_GHz={c['GRBM_GUI_ACTIVE'] / 8 / (avg_us * 1e3):.3f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
            der.append(f"mfma_busy={c['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * 256 * c['GRBM_GUI_ACTIVE'] / 8):.3f}")
        if "TCP_PENDING_STALL_CYCLES_sum" in c and "GRBM_GUI_ACTIVE" in c:
            der.append(f"l1_pending_stall={c['TCP_PENDING_STALL_CYCLES_sum'] / (256 * c['GRBM_GUI_ACTIVE'] / 8):.3f}")
        hit, miss = c.get("TCC_HIT_sum", c.get("TCC_HIT")), c.get("TCC_MISS_sum", c.get("TCC_MISS"))
        if hit is not None and miss is not None and hit + miss > 0:
            der.append(f"l2_hit_rate={hit / (hit + miss):.3f}")
        lines.append(f"{st} (dispatches {n}" + (f", avg {avg_us:.1f} us" if avg_us else "") + "): "
                     + " ".join(parts + der))
    return "\n".join(lines)


def summarize_traffic(d_fetch, d_write):
    """HBM bytes per launch and stage from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), scaled by what the counters read for the copy calibration
    (a torch add of 64 Mi fp32: 256 MiB read and 256 MiB written)."""
    f, _ = _counters(d_fetch)
    w, _ = _counters(d_write)
    cal = "torch elementwise (the copy calibration in traffic runs)"
    fk = f[cal]["FETCH_SIZE"]
    wk = w[cal]["WRITE_SIZE"]
    f_cal, w_cal = sum(fk.values()) / len(fk), sum(wk.values()) / len(wk)
    ff, wf = (256 << 20) / (f_cal * 1024), (256 << 20) / (w_cal * 1024)
    lines = [f"# calibration: a torch elementwise add of 64Mi fp32 reads 256 MiB and writes 256 MiB per launch;",
             f"#   it reads FETCH_SIZE {f_cal:.1f} KiB and WRITE_SIZE {w_cal:.1f} KiB,",
             f"#   so bytes = FETCH_SIZE_KiB * 1024 * {ff:.4f} and WRITE_SIZE_KiB * 1024 * {wf:.4f}",
             f"fetch_factor: {ff:.4f}", f"write_factor: {wf:.4f}",
             f"{'stage / kernel':44s} {'launches':>8s} {'FETCH_KiB':>10s} {'WRITE_KiB':>12s} {'read_MB':>12s} "
             f"{'written_MB':>12s}"]
    for st in sorted(set(f) & set(w)):
        if st == cal:
            continue
        fv = sum(f[st]["FETCH_SIZE"].values()) / len(f[st]["FETCH_SIZE"])
        wv = sum(w[st]["WRITE_SIZE"].values()) / len(w[st]["WRITE_SIZE"])
        rb, wb = fv * 1024 * ff, wv * 1024 * wf
        lines.append(f"{st:44s} {len(f[st]['FETCH_SIZE']):8d} {fv:10.1f} {wv:12.1f} {rb / 1e6:12.1f} {wb / 1e6:12.1f}")
        lines.append(f"traffic_bytes[{st}]: {rb + wb:.0f}")
    return "\n".join(lines)


def cpu_baseline(wl, target_s=12.0):
    """The oracle as it stands, on all host threads, on a bounded sample."""
    from oracle import oracle
    T = wl.shape.T
    rng = np.random.default_rng(123)
    # two pilots that keep every thread busy (a few tokens per thread): a call
    # costs a fixed part (the weights' conversion) plus a part per token
    n = min(T, max(8, 4 * oracle.max_threads()))
    times = []
    for k in (n, 2 * n):
        toks = np.sort(rng.choice(T, size=min(T, k), replace=False))
        t0 = time.perf_counter()
        oracle.forward(wl, tokens=toks, want=("y",))
        times.append(time.perf_counter() - t0)
    per_tok = max((times[1] - times[0]) / n, times[1] / (2 * n) / 4, 1e-9)
    fixed = max(times[0] - per_tok * n, 0.0)
    n2 = int(min(T, max(n, (target_s - fixed) / per_tok)))
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


def describe(sh):
    return (f"{sh.name}: LatentMoE layer forward, T={sh.T} d={sh.d} l={sh.l} m={sh.m} "
            f"N'={sh.n_experts} K'={sh.top_k} S={sh.n_shared}x{sh.m_shared} {sh.variant} {sh.dtype}"
            + (" (routed experts E4M3 + per-column scales)" if sh.expert_dtype == "fp8" else "")
            + (" SwiGLU experts" if sh.expert_act == "swiglu" else ""))


def measure(name, args, log):
    """Time `args.steps` forwards of workload `name` (weights rotated over R
    independent copies); returns the measurement dict and the workload."""
    import torch
    from mixture_experts_layer_latentmoe_amd import _abi
    from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
    from synth import get_config, make_workload

    sh = get_config(name)
    log(f"generating {sh.name} (seeded)")
    wl = make_workload(sh)
    dev = "cuda:0"
    R = args.weight_copies or min(8, max(2, -(-2_000_000_000 // weight_bytes(sh))))
    layers = [LatentMoE.from_workload(wl, device=dev) for _ in range(R)]
    layer = layers[0]
    x = to_device(wl.tensors["x"], sh.dtype, dev)
    y = torch.empty_like(x)
    T = sh.T
    log(f"{sh.name}: {R} weight copies; warmup {args.warmup}")
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

    def stage_entry(name, avg_us, n):
        flop, nbytes, staged = work.get(name, (None, None, None))
        e = {"avg_us": round(avg_us, 2), "launches": n}
        if flop:
            e["tflops"] = round(flop / (avg_us * 1e-6) / 1e12, 1)
        if nbytes:
            e["gbs"] = round(nbytes / (avg_us * 1e-6) / 1e9, 1)
            e["algorithmic_bytes"] = nbytes
        if staged:
            e["staged_bytes"] = staged
        if flop or nbytes:
            r = roofline_of(flop, nbytes, avg_us * 1e-6, sh.dtype)
            e["bound"], e["frac"] = r["bound"], r["frac"]
        tr = profiled_traffic(sh.name, name)
        if tr is not None and nbytes:
            e["traffic"] = tr
            e["traffic_over_algorithmic"] = round(tr / nbytes, 3)
        return e

    # Untimed pass with every stage timed: the per-stage breakdown, and which
    # stage dominates.  (Two event records per stage and forward cost a few
    # microseconds each, too much to leave in the timed region.)
    stage_out, dom = {}, None
    if timing:
        nb = min(args.steps, 10)
        profile_begin(nb)
        for i in range(nb):
            layers[i % R].forward(x, y)
        stage_out = {k: stage_entry(k, ms / n * 1e3, n) for k, (ms, n) in profile_end().items() if n}
        dom = max((k for k in stage_out if "frac" in stage_out[k]), key=lambda k: stage_out[k]["avg_us"])
    # the throughput: K forwards with no events in between (an event record
    # costs the stream about 3 us, 5 % of a decode step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        layers[i % R].forward(x, y)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"{sh.name}: timed {args.steps} steps in {dt:.3f} s")
    ms_per_step = dt / args.steps * 1e3
    roof = None
    if timing:
        # the dominant kernel: the same K forwards again, with HIP events on
        # the forward's stream around that stage only
        profile_begin(args.steps, 1 << names[dom])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            layers[i % R].forward(x, y)
        torch.cuda.synchronize()
        log(f"{sh.name}: timed {args.steps} steps with events around {dom} in {time.perf_counter() - t1:.3f} s")
        tot = profile_end()[dom]
        e = stage_entry(dom, tot[0] / tot[1] * 1e3, tot[1])
        flop, nbytes, staged = work[dom]
        roof = {"kernel": dom, **roofline_of(flop, nbytes, e["avg_us"] * 1e-6, sh.dtype),
                "traffic": e.get("traffic"), "algorithmic_bytes": nbytes, "staged_bytes": staged,
                "traffic_over_algorithmic": e.get("traffic_over_algorithmic"), "flop": flop,
                "avg_us": e["avg_us"], "launches": e["launches"]}
    lflop, lbytes = layer_work(sh, T, n_active)
    t_roof = max(lflop / (PEAK[sh.dtype] * 1e12), lbytes / (HBM_PEAK_GBS * 1e9))
    out = {
        "tokens_per_s": round(T * args.steps / dt, 1), "ms_per_step": round(ms_per_step, 4),
        "workload": describe(sh), "tokens": T, "experts_with_tokens": n_active, "weight_copies": R,
        "layer_tflops": round(lflop / (ms_per_step * 1e-3) / 1e12, 1),
        "layer_roofline": {"bound": "mfma" if lflop / (PEAK[sh.dtype] * 1e12) >= lbytes / (HBM_PEAK_GBS * 1e9)
                           else "hbm", "flop": lflop, "algorithmic_bytes": lbytes,
                           "roofline_tokens_per_s": round(T / t_roof, 1),
                           "frac": round(t_roof / (ms_per_step * 1e-3), 4)},
        "roofline": roof, "stages": stage_out,
    }
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
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                L.forward(x, y)
            graphs.append(gr)
        for i in range(max(args.warmup, R)):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        tg = (time.perf_counter() - tg0) / args.steps
        # the R forwards of one rotation in a single graph (one graph launch per R steps)
        grall = torch.cuda.CUDAGraph()
        with torch.cuda.graph(grall):
            for L in layers:
                L.forward(x, y)
        n_rot = max(1, args.steps // R)
        for _ in range(max(1, args.warmup // R)):
            grall.replay()
        torch.cuda.synchronize()
        ta0 = time.perf_counter()
        for _ in range(n_rot):
            grall.replay()
        torch.cuda.synchronize()
        ta = (time.perf_counter() - ta0) / (n_rot * R)
        out["graph"] = {"ms_per_step": round(tg * 1e3, 4), "tokens_per_s": round(T / tg, 1),
                        "note": "forward replayed from HIP graphs, one graph per step, same weight-copy rotation",
                        "rotation_graph": {"ms_per_step": round(ta * 1e3, 4), "tokens_per_s": round(T / ta, 1),
                                           "steps": n_rot * R,
                                           "note": "the R forwards of one weight-copy rotation captured as one "
                                                   "graph, replayed steps / R times"}}
        del graphs, grall
    if args.backward and sh.expert_dtype != "fp8":
        # algorithmic work: the recomputed forward (no up-projection), the
        # data gradients and the weight gradients of every GEMM: 3F - F_up
        gemm_flop = 3.0 * lflop - work["gemm_up_shared2"][0]
        dy = torch.randn_like(x)
        for i in range(max(2, R)):
            layers[i % R].backward(x, dy)
        torch.cuda.synchronize()
        tb0 = time.perf_counter()
        for i in range(args.steps):
            layers[i % R].backward(x, dy)
        torch.cuda.synchronize()
        tb = (time.perf_counter() - tb0) / args.steps
        out["backward"] = {"ms_per_step": round(tb * 1e3, 4), "tokens_per_s": round(T / tb, 1),
                           "algorithmic_tflops": round(gemm_flop / tb / 1e12, 1),
                           "note": "forward recompute + data and weight gradients (fp32), weight copies "
                                   "rotated as above"}
        log(f"{sh.name}: backward {args.steps} steps in {tb * args.steps:.3f} s")
    for L in layers:
        L.close()
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out, wl


def main():
    if len(sys.argv) >= 3 and sys.argv[1] == "--summarize":
        # python bench.py --summarize trace|pmc DIR | traffic FETCH_DIR WRITE_DIR [--title TEXT] [--cmd TEXT]...
        kind, rest = sys.argv[2], sys.argv[3:]
        head = []
        while len(rest) >= 2 and rest[-2] in ("--title", "--cmd"):
            head.insert(0, ("# " if rest[-2] == "--title" else "# command: ") + rest[-1])
            rest = rest[:-2]
        head.append(f"# kernel sources sha256[:16] of csrc/*: {kernel_source_sha()}")
        body = {"trace": lambda: summarize_trace(rest[0]), "pmc": lambda: summarize_pmc(rest[0]),
                "traffic": lambda: summarize_traffic(rest[0], rest[1])}[kind]()
        print("\n".join(head + [body]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=HEADLINE, help="the headline workload")
    ap.add_argument("--also", default=ALSO,
                    help="comma-separated further workloads measured in the same run and reported under "
                         "\"workloads\" (empty: none)")
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
                    help="also replay the forward from captured HIP graphs (one per weight copy, and one "
                         "holding the forwards of a whole weight-copy rotation) over the same steps and report "
                         "them under \"graph\"; the headline value stays the eager forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain elementwise copy of 256 MiB (3 launches) so that profiler "
                         "byte counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); this layer is measured on one "
              "GPU's share and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    head, wl = measure(args.config, args, log)
    others = {}
    for name in [n for n in args.also.split(",") if n and n != args.config]:
        others[name], _ = measure(name, args, log)
    if args.copy_calibration:
        # reads 256 MiB and writes 256 MiB per launch
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.add(a, 0.0, out=b)
        torch.cuda.synchronize()

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)
    sh = wl.shape
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": sh.dtype,
        "data": "synthetic",
        "config": {"workload": head["workload"], "tokens": head["tokens"],
                   "experts_with_tokens": head["experts_with_tokens"], "weight_copies": head["weight_copies"]},
        "layer_tflops": head["layer_tflops"], "layer_roofline": head["layer_roofline"],
        "roofline": head["roofline"], "cpu_baseline": cpu, "stages": head["stages"],
        **({"backward": head["backward"]} if "backward" in head else {}),
        **({"graph": head["graph"]} if "graph" in head else {}),
        "workloads": others,
        "stages_note": "per-stage HIP-event times from an untimed pass of min(steps, 10) forwards; "
                       "value and ms_per_step from the K timed forwards, which record no events; "
                       "roofline.avg_us is the dominant kernel timed with HIP events on the forward's "
                       "stream over a second timed region of the same K forwards; algorithmic "
                       "bytes = weights touched + the kernel's own inputs and outputs, staged_bytes = H "
                       "between the expert GEMMs and the fp32 router scores",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
