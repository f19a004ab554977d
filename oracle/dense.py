"""Brute-force dense evaluation of the LatentMoE layer in numpy fp64.

TEST INFRASTRUCTURE ONLY.  A second, independently written formulation used
to pin the C oracle: instead of running only the selected experts, it runs
EVERY routed expert on every token and multiplies its output by a dense gate
matrix that is zero outside each token's selection.  The sparse loop of the
explainer page's LatentMoE code block and this dense masked sum are equal by
definition; agreeing to ~1e-12 shows neither implementation dropped, swapped
or mis-indexed a term.

Page: "LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through
Equations, Architecture, Code and ..." -- Figure 3 (router, softmax, top-K),
Figure 6 (down/up projections), Figure 8 (the three paths of the layer),
Figure 9 (latent expert = two matrices around a squared ReLU), and the MoE
code block (renormalisation of the K selected weights).  Gated experts (the
explainer's feed-forward section: a gate matrix next to W1) use torch's
``silu`` as the activation of the gate branch, so this file and the C
oracle do not share the activation either.
"""

import numpy as np


def select_lexsort(s: np.ndarray, K: int) -> np.ndarray:
    """Row-wise top-K: sort keys (-score, index); numpy's lexsort sorts by the
    last key first, so the expert index breaks ties in ascending order."""
    T, N = s.shape
    out = np.empty((T, K), dtype=np.int32)
    ar = np.arange(N)
    for t in range(T):
        order = np.lexsort((ar, -s[t]))
        out[t] = order[:K]
    return out


def softmax_rows(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def dense_gate_matrix(s: np.ndarray, K: int) -> np.ndarray:
    """G[t, e] = renormalised softmax weight if e is selected for t, else 0."""
    sel = select_lexsort(s, K)
    p = softmax_rows(s)
    mask = np.zeros_like(p)
    np.put_along_axis(mask, sel.astype(np.int64), 1.0, axis=1)
    pm = p * mask
    return pm / pm.sum(axis=1, keepdims=True)


def sq_relu(a: np.ndarray) -> np.ndarray:
    return np.square(np.maximum(a, 0.0))


def silu_torch(a: np.ndarray) -> np.ndarray:
    import torch
    return torch.nn.functional.silu(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))).numpy()


def layer_dense(x, w_router, b_router, w_down, w1, w2, w_up, w1_s, w2_s, K, w1g=None, w1g_s=None):
    """All arguments float64 numpy arrays in the [in, out] layout.  With gate
    banks w1g [N', l, m] and w1g_s [S, d, m_s] the experts are gated:
    silu(a W_g) * (a W1) in place of relu(a W1)^2.

    Returns dict with logits s, dense gates G, z, u, y.
    """
    def act(a_in, w_val, w_gate):
        if w_gate is None:
            return sq_relu(a_in @ w_val)
        return silu_torch(a_in @ w_gate) * (a_in @ w_val)

    s = x @ w_router
    if b_router is not None:
        s = s + b_router[None, :]
    G = dense_gate_matrix(s, K)
    z = x @ w_down
    u = np.zeros((x.shape[0], w_down.shape[1]))
    for e in range(w1.shape[0]):
        u += G[:, e:e + 1] * (act(z, w1[e], None if w1g is None else w1g[e]) @ w2[e])
    y = u @ w_up
    for j in range(w1_s.shape[0]):
        y = y + act(x, w1_s[j], None if w1g_s is None else w1g_s[j]) @ w2_s[j]
    return {"logits": s, "G": G, "z": z, "u": u, "y": y}


def expert_bank_f64(wl, name):
    """W1, W2 or W_g of a workload in float64.  FP8 (E4M3) banks are decoded with
    torch's float8_e4m3fn type -- a decoder independent of the C oracle's --
    and scaled per expert and output column: W[e, i, j] = decode(q) * s[e, j]
    (exact in float64)."""
    if wl.shape.expert_dtype != "fp8":
        return wl.f64(name)
    import torch
    q = np.ascontiguousarray(wl.tensors[name], dtype=np.uint8)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = np.asarray(wl.tensors[name + "_scale"], dtype=np.float64)
    return dec * sc[:, None, :]


def layer_dense_from_workload(wl, tokens=None):
    f = wl.f64
    x = f("x") if tokens is None else f("x")[np.asarray(tokens)]
    b = wl.tensors.get("b_router")
    b = None if (b is None or not wl.shape.has_bias) else np.asarray(b, dtype=np.float64)
    S = wl.shape.n_shared
    w1s = f("w1_s") if S > 0 else np.zeros((0, wl.shape.d, 1))
    w2s = f("w2_s") if S > 0 else np.zeros((0, 1, wl.shape.d))
    gated = wl.shape.expert_act == "swiglu"
    w1g = expert_bank_f64(wl, "w1g") if gated else None
    w1gs = (f("w1g_s") if S > 0 else np.zeros((0, wl.shape.d, 1))) if gated else None
    return layer_dense(x, f("w_router"), b, f("w_down"), expert_bank_f64(wl, "w1"),
                       expert_bank_f64(wl, "w2"), f("w_up"), w1s, w2s, wl.shape.top_k, w1g, w1gs)


def dispatch_argsort(idx: np.ndarray, N: int):
    """Dispatch order via a stable argsort of the flattened expert ids:
    returns counts, offsets, pos, perm (same meaning as the C oracle)."""
    T, K = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")     # (t, k) pairs sorted by expert, then t
    counts = np.bincount(flat, minlength=N).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pos = np.empty(T * K, dtype=np.int32)
    pos[order] = np.arange(T * K, dtype=np.int32)
    perm = (order // K).astype(np.int32)
    return counts, offsets, pos.reshape(T, K), perm
