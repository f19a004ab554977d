"""Helpers for the GPU parity tests: run the HIP layer through the C ABI and
compare it with the fp64 oracle run on the same seeded inputs.

Routing is checked three ways on every token:
  * the selection rule as a function: the oracle's own top-K' (score
    descending, lower index first on ties) and renormalised gates, applied
    to the GPU's fp32 scores, must give the GPU's experts in the GPU's slot
    order bit for bit, and its gates to a bound derived from fp32 rounding;
  * the scores themselves: the GPU's fp32 scores must be within DELTA/2 of
    the oracle's own fp64 scores;
  * decided tokens (every gap among the oracle's top K'+1 scores at least
    DELTA, so no rounding below DELTA/2 can reorder them): the GPU's experts,
    slot order and gates equal the oracle's fp64 routing.
The dispatch permutation is the oracle's counting sort of the GPU's own
expert choices, bit for bit, and satisfies its defining properties.  Stages
and the layer output are compared with the oracle's fp64 values (the oracle
never sees anything the GPU computed except in the two selection and
dispatch checks above, where it is the checker of a function of the GPU's
scores and choices).
"""

import sys

import numpy as np
import torch

from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
from oracle import oracle
from tests import tolerances as TOL
from tests.helpers import DELTA, decided_mask, elem_err, near_tie_mask, rel_max_err  # noqa: F401

GATE_ULPS = 2.0 ** -24  # unit roundoff of fp32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def run_gpu(wl, layer=None, debug=True, device="cuda:0"):
    say(f"[gpu] {wl.shape.name}: T={wl.shape.T} d={wl.shape.d} N'={wl.shape.n_experts} K'={wl.shape.top_k} "
        f"dtype={wl.shape.dtype}")
    own = layer is None
    if own:
        layer = LatentMoE.from_workload(wl, device=device)
    x = to_device(wl.tensors["x"], wl.shape.dtype, device)
    out = layer.forward_debug(x) if debug else {"y": layer.forward(x)}
    torch.cuda.synchronize()
    res = {k: to_np(v) for k, v in out.items()}
    if own:
        layer.close()
    return res


def oracle_routing(wl):
    """The oracle's routing for every token (scores, experts, gates only)."""
    return oracle.forward(wl, want=("logits", "idx", "gate"))


def check_dispatch_properties(out, K, N):
    """counts/offsets/pos/perm_token are the stable counting sort of the
    GPU's own idx: these properties admit exactly one answer."""
    idx = out["idx"]
    T = idx.shape[0]
    P = T * K
    counts = np.bincount(idx.reshape(-1), minlength=N)
    assert np.array_equal(out["counts"], counts)
    assert np.array_equal(out["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    pos, perm, off = out["pos"], out["perm_token"], out["offsets"]
    assert np.array_equal(np.sort(pos.reshape(-1)), np.arange(P))           # bijection
    assert np.all(perm[pos] == np.arange(T)[:, None])                       # inverse
    assert np.all((pos >= off[idx]) & (pos < off[idx + 1]))                 # in its expert's range
    seg = np.repeat(np.arange(N), counts)                                   # expert of each row
    same = seg[1:] == seg[:-1]
    assert np.all(np.diff(perm)[same] > 0)                                  # tokens ascending


def check_dispatch_exact(out, N):
    """The oracle's counting sort of the GPU's expert choices, bit for bit."""
    dp = oracle.dispatch(out["idx"], N)
    assert np.array_equal(out["counts"], dp.counts)
    assert np.array_equal(out["offsets"], dp.offsets)
    assert np.array_equal(out["pos"], dp.pos)
    assert np.array_equal(out["perm_token"], dp.perm)


def gate_bound(lg, idx):
    """Relative error bound of the GPU's fp32 gates against the exact
    renormalised softmax of the same fp32 scores: the difference d = s_k -
    s_max is rounded once (u |d|), exp adds its argument's error and at most
    2 u of its own, the sum of up to 64 positive terms in a 6-level tree 6 u,
    the division u: per gate (|d_k| + max_j |d_j| + 11) u."""
    s = np.take_along_axis(lg, idx.astype(np.int64), axis=1)
    d = np.abs(s - s.max(axis=1, keepdims=True))
    return (d + d.max(axis=1, keepdims=True) + 11.0) * GATE_ULPS


def check_routing(out, wl, route_ref):
    """Every token: the GPU's selection and gates against the oracle's rule
    on the GPU's own scores, the scores against the oracle's fp64 scores, and
    (decided tokens) the routing against the oracle's fp64 routing.  Returns
    the decided-token mask."""
    sh = wl.shape
    K, N = sh.top_k, sh.n_experts
    lg_gpu = out["logits"].astype(np.float64)  # exact widening
    idx = out["idx"]
    # 1. the selection rule and the gates as functions of the GPU's scores
    sel = oracle.select(lg_gpu, K)
    bad = np.nonzero(np.any(idx != sel, axis=1))[0]
    assert bad.size == 0, f"selection differs from the rule on the GPU's scores at tokens {bad[:10]}"
    g_rule = oracle.gates(lg_gpu, idx)
    rel = np.abs(out["gate"].astype(np.float64) - g_rule) / g_rule
    bound = gate_bound(lg_gpu, idx)
    say(f"[gpu]   selection = oracle rule on the GPU's scores for all {len(idx)} tokens; gates: max rel err "
        f"{rel.max():.2e} (max bound {bound.max():.2e})")
    assert np.all(rel <= bound), float(np.max(rel / bound))
    # 2. the scores
    lg_ref = route_ref.logits
    err = float(np.max(np.abs(lg_gpu - lg_ref)))
    dec = decided_mask(lg_ref, K)
    say(f"[gpu]   scores: max |fp32 - fp64| = {err:.2e} (must be < {DELTA / 2:.0e}); "
        f"decided tokens {dec.sum()} of {len(dec)}")
    assert err < DELTA / 2, err
    assert dec.mean() >= 0.5
    # 3. decided tokens: the oracle's own fp64 routing
    bad = np.nonzero(np.any(idx[dec] != route_ref.idx[dec], axis=1))[0]
    assert bad.size == 0, f"routing differs on decided tokens {np.nonzero(dec)[0][bad[:10]]}"
    np.testing.assert_allclose(out["gate"][dec], route_ref.gate[dec], rtol=1e-5, atol=1e-7)
    # 4. dispatch: the oracle's counting sort of the GPU's choices
    check_dispatch_properties(out, K, N)
    check_dispatch_exact(out, N)
    same = np.array_equal(idx, route_ref.idx)
    say(f"[gpu]   dispatch bit-exact; routing equals the oracle's fp64 routing on "
        f"{'every token' if same else f'{np.sum(np.all(idx == route_ref.idx, axis=1))} of {len(idx)} tokens'}")
    return dec


def check_output(out, wl, ref, tokens):
    """The contract on tokens whose K'-th and (K'+1)-th oracle scores differ
    by at least 1e-3: max (|y - y_oracle| - half an output ulp) <= bar RMS."""
    sh = wl.shape
    keep = ~near_tie_mask(ref.logits, sh.top_k, 1e-3)
    assert keep.sum() >= max(1, int(0.5 * len(tokens)))
    err = TOL.y_err(out["y"][tokens][keep], ref.y[keep], sh.dtype)
    bar = TOL.y_bar(sh)
    say(f"[gpu]   y: max (err - half ulp) / RMS = {err:.3e} over {keep.sum()} of {len(tokens)} tokens (bar {bar})")
    assert err <= bar, err
    return err


STAGES = ("z", "h", "y_perm", "u", "y", "h_shared")


def gpu_stages(out, sh, tk):
    """The GPU's stage arrays for tokens tk (routed stages in slot order)."""
    pos = out["pos"][tk].reshape(-1)
    st = {"z": out["z"][tk], "h": out["h"][pos], "y_perm": out["y_perm"][pos], "u": out["u"][tk], "y": out["y"][tk]}
    if sh.n_shared > 0:
        st["h_shared"] = out["h_shared"][tk]
    return st


def oracle_stages(ref, sh, sel):
    """The oracle's stage arrays for its rows sel, laid out as gpu_stages."""
    st = {"z": ref.z[sel], "h": ref.h[sel].reshape(-1, sh.m), "y_perm": ref.o[sel].reshape(-1, sh.l),
          "u": ref.u[sel], "y": ref.y[sel]}
    if sh.n_shared > 0:
        st["h_shared"] = ref.hs[sel]
    return st


def check_stages(out, wl, ref, tokens, decided):
    """Each intermediate, on decided tokens (same routing on both sides)."""
    sh = wl.shape
    sel = np.nonzero(decided)[0]
    g, r = gpu_stages(out, sh, tokens[sel]), oracle_stages(ref, sh, sel)
    errs = {k: elem_err(g[k], r[k]) for k in g}
    _assert_stage_errs(sh, errs)
    return errs


def _assert_stage_errs(sh, errs):
    say("[gpu]   stage errors, max |d| / (|ref| + RMS): " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        bar = TOL.stage_bar(sh, k)
        assert v <= bar, (k, v, bar)


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


class _Contract:
    """The oracle's scores and output for the contract check."""

    def __init__(self, logits, y):
        self.logits, self.y = logits, y


def check_tokens_chunked(out, wl, tokens, decided, chunk=512):
    """The contract and every stage over many tokens, with the oracle run
    in chunks (its stage outputs for thousands of tokens do not fit in memory
    at once).  Each stage's error is formed against its RMS over all the
    compared entries, exactly as one comparison would."""
    sh = wl.shape
    want = ("logits", "idx", "gate", "z", "h", "o", "u", "hs", "y")
    # the oracle's stages kept in float32 (its rounding, 6e-8 relative, is far
    # below every bar)
    refs = {}
    y_all, lg_all = [], []
    for c0 in range(0, len(tokens), chunk):
        tk = tokens[c0:c0 + chunk]
        ref = oracle.forward(wl, tokens=tk, want=want)
        for k, b in oracle_stages(ref, sh, np.nonzero(decided[tk])[0]).items():
            refs.setdefault(k, []).append(b.astype(np.float32))
        y_all.append(ref.y)
        lg_all.append(ref.logits)
    check_output(out, wl, _Contract(np.concatenate(lg_all), np.concatenate(y_all)), tokens)
    g = gpu_stages(out, sh, tokens[decided[tokens]])
    errs = {k: elem_err(g[k], np.concatenate(refs[k]).astype(np.float64)) for k in g}
    _assert_stage_errs(sh, errs)
    return errs


def full_check(wl, n_sample=None):
    out = run_gpu(wl)
    route = oracle_routing(wl)
    dec = check_routing(out, wl, route)
    toks = sample_tokens(wl.shape.T, n_sample or wl.shape.T)
    if len(toks) > 512:
        check_tokens_chunked(out, wl, toks, dec)
        return out
    ref = oracle.forward(wl, tokens=toks, want=("logits", "idx", "gate", "z", "h", "o", "u", "hs", "y"))
    check_output(out, wl, ref, toks)
    check_stages(out, wl, ref, toks, dec[toks])
    return out
