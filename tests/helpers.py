"""Small helpers shared by the tests (no layer arithmetic here)."""

import numpy as np

from synth import LayerShape, Workload
from synth.generate import f32_to_bf16_bits


def shape(name="custom", T=8, d=8, l=4, m=6, n_experts=4, top_k=2, n_shared=1,
          m_shared=5, alpha=2, variant="acc", dtype="f32", seed=0, zipf_s=None, expert_dtype=None,
          expert_act="relu2"):
    return LayerShape(name, T=T, d=d, l=l, m=m, n_experts=n_experts, top_k=top_k,
                      n_shared=n_shared, m_shared=m_shared, alpha=alpha,
                      variant=variant, dtype=dtype, seed=seed, zipf_s=zipf_s,
                      expert_dtype=expert_dtype, expert_act=expert_act)


def workload_from_arrays(sh: LayerShape, arrays: dict) -> Workload:
    """Build a workload from float arrays (exactly representable in the
    shape's dtype).  Missing shared banks become empty."""
    t = {}
    names = ["x", "w_router", "w_down", "w1", "w2", "w_up", "w1_s", "w2_s"]
    if sh.expert_act == "swiglu":
        names += ["w1g", "w1g_s"]
    for k in names:
        a = np.asarray(arrays[k], dtype=np.float32)
        if sh.dtype == "bf16":
            bits = f32_to_bf16_bits(a)
            assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), a), k
            t[k] = bits
        else:
            t[k] = np.ascontiguousarray(a)
    b = arrays.get("b_router")
    t["b_router"] = None if b is None else np.asarray(b, dtype=np.float32)
    return Workload(sh, t)


def random_arrays(sh: LayerShape, rng, scale=1.0):
    """Random float32 inputs of the right shapes, N(0, scale^2/fan_in)."""
    def nrm(shape, fan):
        return (rng.standard_normal(shape) * scale / np.sqrt(fan)).astype(np.float32)
    S = sh.n_shared
    a = {
        "x": rng.standard_normal((sh.T, sh.d)).astype(np.float32),
        "w_router": nrm((sh.d, sh.n_experts), sh.d),
        "w_down": nrm((sh.d, sh.l), sh.d),
        "w1": nrm((sh.n_experts, sh.l, sh.m), sh.l),
        "w2": nrm((sh.n_experts, sh.m, sh.l), sh.m),
        "w_up": nrm((sh.l, sh.d), sh.l),
        "w1_s": nrm((S, sh.d, sh.m_shared), sh.d),
        "w2_s": nrm((S, sh.m_shared, sh.d), sh.m_shared),
    }
    if sh.has_bias:
        a["b_router"] = rng.standard_normal(sh.n_experts).astype(np.float32)
    if sh.expert_act == "swiglu":  # drawn last: the other arrays do not depend on it
        a["w1g"] = nrm((sh.n_experts, sh.l, sh.m), sh.l)
        a["w1g_s"] = nrm((S, sh.d, sh.m_shared), sh.d)
    if sh.dtype == "bf16":
        from synth import round_to_bf16
        a = {k: (round_to_bf16(v) if k != "b_router" else v) for k, v in a.items()}
    return a


def random_workload(sh: LayerShape, seed=0, scale=1.0) -> Workload:
    return workload_from_arrays(sh, random_arrays(sh, np.random.default_rng(seed), scale))


def near_tie_mask(logits: np.ndarray, K: int, gap: float = 1e-3) -> np.ndarray:
    """True for tokens whose K-th and (K+1)-th largest scores differ by < gap."""
    if K >= logits.shape[1]:
        return np.zeros(logits.shape[0], dtype=bool)
    srt = -np.sort(-logits, axis=1)
    return (srt[:, K - 1] - srt[:, K]) < gap


def random_fp8_workload(sh: LayerShape, seed=0, pow2_scales=False) -> Workload:
    """A random workload whose W1/W2 are FP8 (E4M3) banks with per-column
    scales (the input recipe's quantizer), the rest as for random_workload.
    pow2_scales: replace every scale by a power of two (varying per expert and
    column), so that decode(q) * scale is exact in bf16."""
    from synth.generate import quantize_e4m3_columns
    assert sh.expert_dtype == "fp8"
    rng = np.random.default_rng(seed)
    arrays = random_arrays(sh, rng)
    t = dict(workload_from_arrays(sh, arrays).tensors)
    for k in (("w1", "w2", "w1g") if sh.expert_act == "swiglu" else ("w1", "w2")):
        w = arrays[k]
        q = np.empty(w.shape, dtype=np.uint8)
        sc = np.empty((w.shape[0], w.shape[2]), dtype=np.float32)
        for e in range(w.shape[0]):
            q[e], sc[e] = quantize_e4m3_columns(w[e])
        if pow2_scales:
            sc = np.ldexp(np.float32(1.0), rng.integers(-9, -3, size=sc.shape)).astype(np.float32)
        t[k], t[k + "_scale"] = q, sc
    return Workload(sh, t)


# ---- comparison metrics (used by the GPU parity tests and by the CPU test
# that derives their tolerances from the emulated bf16 rounding points) ----

DELTA = 2e-5  # decided-token margin on the scores


def rel_max_err(got, ref):
    """max |got - ref| / RMS(ref): the layer output's contract metric."""
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def elem_err(got, ref):
    """max |got - ref| / (|ref| + RMS(ref)): relative for large entries,
    RMS-relative for small ones (suits heavy-tailed squared-ReLU outputs)."""
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + max(rms, 1e-30))))


def decided_mask(logits, K, delta=DELTA):
    """True for tokens whose top-(K'+1) scores are pairwise at least delta
    apart: no rounding smaller than delta / 2 can change their routing."""
    N = logits.shape[1]
    srt = -np.sort(-logits, axis=1)[:, :min(K + 1, N)]
    if srt.shape[1] < 2:
        return np.ones(logits.shape[0], dtype=bool)
    return np.all(srt[:, :-1] - srt[:, 1:] >= delta, axis=1)
