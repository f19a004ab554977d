"""Emulation of the bf16 rounding points of the HIP layer, in numpy fp64.

TEST CODE.  It models where the HIP path of a bf16 layer rounds: every
intermediate it stores in bf16 is rounded once to the nearest bf16 (ties to
even); every sum is taken in fp64 (the kernels sum in fp32, whose rounding is
2^16 times finer than bf16's and is ignored here).  Compared against the fp64
oracle with the parity tests' own metrics, the emulated error is the part of
the GPU's error that storing intermediates in bf16 causes by itself, with no
kernel involved; the tolerances of the parity tests are derived from it
(tests/test_tolerance_derivation.py).

Rounding points modelled (forward, the layer of the explainer page "LatentMoE:
NVIDIA's Latent Mixture of Experts Explained Through Equations, Architecture,
Code and ..."; its Figures 3, 6, 8, 9 and LatentMoE code block):
  z = R(x W_down);  h_s = R(act(x W1_s));  H = R(act(z W1_e));
  Y = R(H W2_e);    u = R(sum_k g_k Y_k);  y = R([u | h_s] [W_up ; W2_s])
Backward (the gradient of that forward; the backward pass of the layer):
  the recompute rounds the raw x-pass output (z and the shared
  pre-activations a_s) and forms h_s = R(act(a_s)) from the rounded a_s;
  the routed pre-activations A stay fp32 (unrounded here); then
  [du | dh_s] = R(dy [W_up ; W2_s]^T),  d a_s = R(act'(a_s) dh_s),
  dY_k = R(g_k du),  ds_k = R(g_k (dg_k - sum_j g_j dg_j)) with
  dg_k = <du, Y_k>,  dA = R((dY W2_e^T) act'(A)),  dz_k = R(dA W1_e^T),
  dz = R(sum_k dz_k),  dx = R([ds | dz | d a_s] Wx^T); weight gradients are
  fp32 sums of products of those rounded operands.
Routing (the set, slot order and gates) is the oracle's fp64 routing.
"""

import numpy as np
from scipy.special import expit

from oracle import oracle
from synth.generate import bf16_bits_to_f32, f32_to_bf16_bits


def R(a):
    """Round to the nearest bf16 (ties to even), returned as float64."""
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


def _bank(wl, name):
    """An expert bank in float64; E4M3 banks decoded by the oracle's decoder
    and scaled per expert and output column."""
    if wl.shape.expert_dtype != "fp8":
        return wl.f64(name)
    dec = oracle.fp8_decode(wl.tensors[name])
    return dec * np.asarray(wl.tensors[name + "_scale"], dtype=np.float64)[:, None, :]


def _silu(v):
    return v * expit(v)


def _dsilu(v):
    s = expit(v)
    return s * (1.0 + v * (1.0 - s))


class _Weights:
    def __init__(self, wl):
        sh = wl.shape
        self.gated = sh.expert_act == "swiglu"
        self.S = sh.n_shared
        self.w_down = wl.f64("w_down")
        self.w_up = wl.f64("w_up")
        self.w_router = wl.f64("w_router")
        self.w1 = _bank(wl, "w1")
        self.w2 = _bank(wl, "w2")
        self.w1g = _bank(wl, "w1g") if self.gated else None
        self.w1_s = wl.f64("w1_s") if self.S else None
        self.w2_s = wl.f64("w2_s") if self.S else None
        self.w1g_s = wl.f64("w1g_s") if (self.S and self.gated) else None


def _shared_pre(x, W):
    """Per shared expert: (value pre-activation, gate pre-activation or None)."""
    out = []
    for j in range(W.S):
        a = x @ W.w1_s[j]
        g = x @ W.w1g_s[j] if W.gated else None
        out.append((a, g))
    return out


def _act(a, g):
    return _silu(g) * a if g is not None else np.square(np.maximum(a, 0.0))


def forward(wl, route):
    """Emulated bf16 forward of a bf16 workload; ``route`` is the oracle's
    routing (idx [T, K'], gate [T, K']).  Returns z, hs, h [T, K', m],
    o [T, K', l], u, y (float64 holding bf16 values)."""
    sh = wl.shape
    assert sh.dtype == "bf16"
    W = _Weights(wl)
    x = wl.f64("x")
    T, K = route.idx.shape
    z = R(x @ W.w_down)
    hs = np.concatenate([R(_act(a, g)) for a, g in _shared_pre(x, W)], axis=1) if W.S else np.zeros((T, 0))
    h = np.zeros((T, K, sh.m))
    o = np.zeros((T, K, sh.l))
    for e in np.unique(route.idx):
        t, k = np.nonzero(route.idx == e)
        a = z[t] @ W.w1[e]
        he = R(_act(a, z[t] @ W.w1g[e] if W.gated else None))
        h[t, k] = he
        o[t, k] = R(he @ W.w2[e])
    u = R(np.einsum("tk,tkl->tl", route.gate, o))
    y_acc = u @ W.w_up
    for j in range(W.S):
        y_acc = y_acc + hs[:, j * sh.m_shared:(j + 1) * sh.m_shared] @ W.w2_s[j]
    return {"z": z, "hs": hs, "h": h, "o": o, "u": u, "y": R(y_acc)}


def backward(wl, route, dy):
    """Emulated bf16 backward of a bf16 workload for dy [T, d] (float64 of
    bf16 values).  Returns dx and the weight gradients, named as by
    oracle.backward (expert banks for every expert)."""
    sh = wl.shape
    assert sh.dtype == "bf16" and sh.expert_dtype != "fp8"
    W = _Weights(wl)
    x = wl.f64("x")
    T, K = route.idx.shape
    N, l, m, ms, S = sh.n_experts, sh.l, sh.m, sh.m_shared, sh.n_shared
    g = route.gate
    # recompute: the raw x-pass output in bf16
    z = R(x @ W.w_down)
    pre = [(R(a), (R(gp) if gp is not None else None)) for a, gp in _shared_pre(x, W)]
    hs = np.concatenate([R(_act(a, gp)) for a, gp in pre], axis=1) if S else np.zeros((T, 0))
    A, Ag, H, Y = {}, {}, {}, {}
    rows = {}
    for e in np.unique(route.idx):
        t, k = np.nonzero(route.idx == e)
        rows[e] = (t, k)
        A[e] = z[t] @ W.w1[e]
        Ag[e] = z[t] @ W.w1g[e] if W.gated else None
        H[e] = R(_act(A[e], Ag[e]))
        Y[e] = R(H[e] @ W.w2[e])
    Yp = np.zeros((T, K, l))
    for e, (t, k) in rows.items():
        Yp[t, k] = Y[e]
    u = R(np.einsum("tk,tkl->tl", g, Yp))
    # [du | dh_s]
    du = R(dy @ W.w_up.T)
    dhs = [R(dy @ W.w2_s[j].T) for j in range(S)]
    # shared pre-activations
    da_s, dag_s = [], []
    for (a, gp), dh in zip(pre, dhs):
        if gp is None:
            da_s.append(R(2.0 * np.maximum(a, 0.0) * dh))
            dag_s.append(None)
        else:
            da_s.append(R(dh * _silu(gp)))
            dag_s.append(R(dh * a * _dsilu(gp)))
    # gates and combine
    dg = np.einsum("tl,tkl->tk", du, Yp)
    gdg = np.sum(g * dg, axis=1, keepdims=True)
    dsk = R(g * (dg - gdg))
    ds = np.zeros((T, N))
    np.put_along_axis(ds, route.idx.astype(np.int64), dsk, axis=1)
    dYp = R(g[:, :, None] * du[:, None, :])
    # expert data gradients
    dzp = np.zeros((T, K, l))
    dA, dAg = {}, {}
    for e, (t, k) in rows.items():
        dH = dYp[t, k] @ W.w2[e].T
        if W.gated:
            dA[e] = R(dH * _silu(Ag[e]))
            dAg[e] = R(dH * A[e] * _dsilu(Ag[e]))
            dzp[t, k] = R(dA[e] @ W.w1[e].T + dAg[e] @ W.w1g[e].T)
        else:
            dA[e] = R(dH * 2.0 * np.maximum(A[e], 0.0))
            dzp[t, k] = R(dA[e] @ W.w1[e].T)
    dz = R(dzp.sum(axis=1))
    dx_acc = ds @ W.w_router.T + dz @ W.w_down.T
    for j in range(S):
        dx_acc = dx_acc + da_s[j] @ W.w1_s[j].T
        if W.gated:
            dx_acc = dx_acc + dag_s[j] @ W.w1g_s[j].T
    out = {"dx": R(dx_acc), "dw_router": x.T @ ds, "dw_down": x.T @ dz, "dw_up": u.T @ dy}
    if wl.shape.has_bias:
        out["db_router"] = ds.sum(axis=0)
    dw1 = np.zeros((N, l, m))
    dw2 = np.zeros((N, m, l))
    dw1g = np.zeros((N, l, m)) if W.gated else None
    for e, (t, k) in rows.items():
        dw2[e] = H[e].T @ dYp[t, k]
        dw1[e] = z[t].T @ dA[e]
        if W.gated:
            dw1g[e] = z[t].T @ dAg[e]
    out["dw1"], out["dw2"] = dw1, dw2
    if W.gated:
        out["dw1g"] = dw1g
    if S:
        out["dw1_s"] = np.stack([x.T @ da for da in da_s])
        out["dw2_s"] = np.stack([hs[:, j * ms:(j + 1) * ms].T @ dy for j in range(S)])
        if W.gated:
            out["dw1g_s"] = np.stack([x.T @ da for da in dag_s])
    return out
