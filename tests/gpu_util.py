"""Helpers for the GPU parity tests: run the HIP layer through the C ABI and
compare it with the fp64 oracle run on the same seeded inputs.

Nothing the GPU returns is ever fed to the oracle.  The oracle computes its
own routing from its own fp64 scores; the comparison then splits tokens:

  * decided tokens -- every gap between consecutive scores among the oracle's
    top K'+1 is at least DELTA.  The test first checks that the GPU's fp32
    scores are within DELTA/2 of the oracle's, so no rounding can reorder a
    decided token: there the GPU's experts, slot order and gates must equal
    the oracle's exactly (gates to fp32 rounding).
  * the rest -- the GPU's selection must still be a valid top-K' of the
    oracle's scores (within DELTA), in non-increasing score order.

The dispatch permutation is checked against its defining properties (which
determine it uniquely from idx), and bit for bit against the oracle's
counting sort whenever the GPU's routing equals the oracle's on every token.
"""

import sys

import numpy as np
import torch

from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
from oracle import oracle
from tests.helpers import near_tie_mask

TOL = {"bf16": 2e-2, "f32": 1e-4}   # y: max |err| <= TOL * RMS(reference)
# Synthetic shapes narrower than the named workloads (d <= 256, few terms per
# sum) carry more relative error from the bf16 intermediates (z, H, Y, u,
# h_s each rounded once to bf16, unit roundoff 2^-9): an exact emulation of
# those rounding points, without any kernel, already reaches 1.6-2.5e-2 at
# d 128 / l 64 with no shared expert.  Twice the spec bar covers it.
TOL_NARROW_BF16 = 4e-2


# Gated experts, stage H only: h = silu(g) v multiplies two sums that both
# carry the bf16 rounding of z, so H has heavier relative error than relu^2's
# h on the |d| / (|ref| + RMS) scale.  The exact emulation of the bf16
# rounding points (z, H rounded once; sums exact), with no kernel, reaches
# 2.53e-2 at the shaping-paper widths (l 640, m 512; 300 tokens), where
# relu^2 experts reach 0.78e-2; the HIP path matches that emulation.  Twice
# the layer's bar covers it.  y keeps the layer's bar.
GATED_H_FACTOR = 2.0


def tol_for(sh):
    if sh.dtype == "bf16" and sh.name == "custom" and sh.d <= 256:
        return TOL_NARROW_BF16
    return TOL[sh.dtype]


DELTA = 2e-5                        # decided-token margin on the scores


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


def rel_max_err(got, ref):
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def elem_err(got, ref):
    """max |got - ref| / (|ref| + RMS(ref)): relative for large entries,
    RMS-relative for small ones (suits heavy-tailed squared-ReLU outputs)."""
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + max(rms, 1e-30))))


def decided_mask(logits, K, delta=DELTA):
    N = logits.shape[1]
    srt = -np.sort(-logits, axis=1)[:, :min(K + 1, N)]
    if srt.shape[1] < 2:
        return np.ones(logits.shape[0], dtype=bool)
    return np.all(srt[:, :-1] - srt[:, 1:] >= delta, axis=1)


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


def check_routing(out, wl, route_ref):
    """Returns the decided-token mask."""
    sh = wl.shape
    K, N = sh.top_k, sh.n_experts
    lg_gpu = out["logits"].astype(np.float64)
    lg_ref = route_ref.logits
    err = float(np.max(np.abs(lg_gpu - lg_ref)))
    dec = decided_mask(lg_ref, K)
    say(f"[gpu]   scores: max |fp32 - fp64| = {err:.2e} (must be < {DELTA / 2:.0e}); "
        f"decided tokens {dec.sum()} of {len(dec)}")
    assert err < DELTA / 2, err
    assert dec.mean() >= 0.5
    idx = out["idx"]
    bad = np.nonzero(np.any(idx[dec] != route_ref.idx[dec], axis=1))[0]
    assert bad.size == 0, f"routing differs on decided tokens {np.nonzero(dec)[0][bad[:10]]}"
    np.testing.assert_allclose(out["gate"][dec], route_ref.gate[dec], rtol=1e-5, atol=1e-7)
    for t in np.nonzero(~dec)[0]:
        s, sel = lg_ref[t], idx[t]
        assert len(set(sel.tolist())) == K and sel.min() >= 0 and sel.max() < N
        assert np.all(np.diff(s[sel]) <= DELTA)
        rest = np.delete(s, sel)
        assert rest.size == 0 or s[sel].min() >= rest.max() - DELTA
        assert abs(out["gate"][t].sum() - 1.0) < 1e-5
    check_dispatch_properties(out, K, N)
    if np.array_equal(idx, route_ref.idx):
        dp = oracle.dispatch(route_ref.idx, N)
        assert np.array_equal(out["counts"], dp.counts)
        assert np.array_equal(out["offsets"], dp.offsets)
        assert np.array_equal(out["pos"], dp.pos)
        assert np.array_equal(out["perm_token"], dp.perm)
        say("[gpu]   routing equals the oracle's on every token; dispatch bit-exact")
    return dec


def check_output(out, wl, ref, tokens):
    """The contract: max |y - y_oracle| <= tol * RMS(y_oracle) over tokens
    whose K'-th and (K'+1)-th oracle scores differ by at least 1e-3."""
    sh = wl.shape
    keep = ~near_tie_mask(ref.logits, sh.top_k, 1e-3)
    assert keep.sum() >= max(1, int(0.5 * len(tokens)))
    err = rel_max_err(out["y"][tokens][keep], ref.y[keep])
    tol = tol_for(sh)
    say(f"[gpu]   y: max err / RMS = {err:.3e} over {keep.sum()} of {len(tokens)} tokens (tol {tol})")
    assert err <= tol, err
    return err


def check_stages(out, wl, ref, tokens, decided):
    """Each intermediate, on decided tokens (same routing on both sides)."""
    sh = wl.shape
    tol = tol_for(sh)
    sel = np.nonzero(decided)[0]
    tk = tokens[sel]
    pos = out["pos"][tk].reshape(-1)
    pairs = {"z": (out["z"][tk], ref.z[sel]),
             "h": (out["h"][pos], ref.h[sel].reshape(-1, sh.m)),
             "y_perm": (out["y_perm"][pos], ref.o[sel].reshape(-1, sh.l)),
             "u": (out["u"][tk], ref.u[sel]),
             "y": (out["y"][tk], ref.y[sel])}
    if sh.n_shared > 0:
        pairs["h_shared"] = (out["h_shared"][tk], ref.hs[sel])
    errs = {k: elem_err(a, b) for k, (a, b) in pairs.items()}
    say("[gpu]   stage errors, max |d| / (|ref| + RMS): " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        t = tol * GATED_H_FACTOR if (k == "h" and sh.expert_act == "swiglu" and sh.dtype == "bf16") else tol
        assert v <= t, (k, v, t)
    return errs


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


def full_check(wl, n_sample=None):
    out = run_gpu(wl)
    route = oracle_routing(wl)
    dec = check_routing(out, wl, route)
    toks = sample_tokens(wl.shape.T, n_sample or wl.shape.T)
    ref = oracle.forward(wl, tokens=toks, want=("logits", "idx", "gate", "z", "h", "o", "u", "hs", "y"))
    check_output(out, wl, ref, toks)
    check_stages(out, wl, ref, toks, dec[toks])
    return out
