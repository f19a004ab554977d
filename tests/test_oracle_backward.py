"""Pins of the oracle's backward pass (SURVEY-listed next step: the layer's
gradient, through the renormalised softmax gates; the top-K' choice is
piecewise constant and passes no gradient).

  * torch autograd on a dense float64 formulation written here with torch
    ops (every expert on every token, masked by a dense gate matrix whose
    selection is fixed and whose values are the differentiable renormalised
    softmax): an independent route to every gradient;
  * central finite differences of <dy, y> through the oracle's own forward,
    on coordinates whose perturbation leaves the routing unchanged;
  * the gates' Jacobian: a uniform shift of all scores changes nothing, so
    the score gradient of every token sums to zero.
"""

import numpy as np
import pytest
import torch

from oracle import oracle
from synth.generate import Workload
from tests.helpers import random_workload, shape

torch.set_default_dtype(torch.float64)


def _shape(**kw):
    base = dict(T=7, d=16, l=8, m=12, n_experts=6, top_k=3, n_shared=1, m_shared=8, dtype="f32")
    base.update(kw)
    return shape(**base)


def _torch_dense_grads(wl, dy, idx):
    """Gradients by torch autograd on a dense formulation with the routing
    fixed to ``idx`` (each token's selected experts)."""
    sh = wl.shape
    f = lambda k: torch.tensor(wl.f64(k), requires_grad=True)
    P = {k: f(k) for k in ("w_router", "w_down", "w1", "w2", "w_up")}
    S = sh.n_shared
    if S > 0:
        P["w1_s"], P["w2_s"] = f("w1_s"), f("w2_s")
    gated = sh.expert_act == "swiglu"
    if gated:
        P["w1g"] = f("w1g")
        if S > 0:
            P["w1g_s"] = f("w1g_s")
    b = wl.tensors.get("b_router")
    if b is not None and sh.has_bias:
        P["b_router"] = torch.tensor(np.asarray(b, np.float64), requires_grad=True)
    x = torch.tensor(wl.f64("x"), requires_grad=True)
    s = x @ P["w_router"] + (P["b_router"] if "b_router" in P else 0.0)
    mask = torch.zeros(s.shape)
    mask[torch.arange(sh.T)[:, None], torch.tensor(idx, dtype=torch.long)] = 1.0
    e = torch.exp(s - s.max(dim=1, keepdim=True).values) * mask
    G = e / e.sum(dim=1, keepdim=True)
    z = x @ P["w_down"]
    act = (lambda a, ag: torch.nn.functional.silu(ag) * a) if gated else (lambda a, ag: torch.relu(a) ** 2)
    u = torch.zeros(sh.T, sh.l)
    for ex in range(sh.n_experts):
        ag = z @ P["w1g"][ex] if gated else None
        u = u + G[:, ex:ex + 1] * (act(z @ P["w1"][ex], ag) @ P["w2"][ex])
    y = u @ P["w_up"]
    for j in range(S):
        ag = x @ P["w1g_s"][j] if gated else None
        y = y + act(x @ P["w1_s"][j], ag) @ P["w2_s"][j]
    (y * torch.tensor(dy)).sum().backward()
    out = {"dx": x.grad.numpy(), "dw_router": P["w_router"].grad.numpy(), "dw_down": P["w_down"].grad.numpy(),
           "dw1": P["w1"].grad.numpy(), "dw2": P["w2"].grad.numpy(), "dw_up": P["w_up"].grad.numpy()}
    if S > 0:
        out["dw1_s"], out["dw2_s"] = P["w1_s"].grad.numpy(), P["w2_s"].grad.numpy()
    if gated:
        out["dw1g"] = P["w1g"].grad.numpy()
        if S > 0:
            out["dw1g_s"] = P["w1g_s"].grad.numpy()
    if "b_router" in P:
        out["db_router"] = P["b_router"].grad.numpy()
    return out


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("kw", [dict(), dict(dtype="bf16"), dict(n_shared=0), dict(top_k=1), dict(top_k=6),
                                dict(expert_act="swiglu"), dict(expert_act="swiglu", n_shared=2, dtype="bf16"),
                                dict(zipf_s=1.1)])
def test_backward_matches_torch_autograd(kw):
    wl = random_workload(_shape(**kw), seed=21)
    dy = np.random.default_rng(5).standard_normal((wl.shape.T, wl.shape.d))
    r = oracle.forward(wl, want=("idx",))
    got = oracle.backward(wl, dy)
    ref = _torch_dense_grads(wl, dy, r.idx)
    for k, v in ref.items():
        assert _rel(got[k], v) < 1e-11, k
    if wl.shape.has_bias:
        assert "db_router" in ref
    # the score gradient is a renormalised-softmax gradient: it sums to zero
    # over each token's experts, so the bias gradient sums to zero too
    assert abs(got["db_router"].sum()) < 1e-12 * max(1.0, np.abs(got["db_router"]).max())


def _loss(wl, dy):
    return float(np.sum(oracle.forward(wl, want=("y",)).y * dy))


def _perturbed(wl, name, index, delta):
    t = dict(wl.tensors)
    a = np.array(t[name], dtype=np.float32)
    a[index] += np.float32(delta)
    t[name] = a
    return Workload(wl.shape, t)


@pytest.mark.parametrize("act", ["relu2", "swiglu"])
def test_backward_matches_finite_differences(act):
    # float32 storage: the perturbed values are stored exactly
    wl = random_workload(_shape(expert_act=act), seed=23)
    rng = np.random.default_rng(7)
    dy = rng.standard_normal((wl.shape.T, wl.shape.d))
    g = oracle.backward(wl, dy)
    idx0 = oracle.forward(wl, want=("idx",)).idx
    names = [("x", "dx"), ("w_router", "dw_router"), ("w_down", "dw_down"), ("w1", "dw1"), ("w2", "dw2"),
             ("w_up", "dw_up"), ("w1_s", "dw1_s"), ("w2_s", "dw2_s")] + \
            ([("w1g", "dw1g"), ("w1g_s", "dw1g_s")] if act == "swiglu" else [])
    h = 2.0 ** -12
    checked = 0
    for name, gname in names:
        arr = wl.tensors[name]
        for _ in range(6):
            index = tuple(int(rng.integers(0, n)) for n in arr.shape)
            plus, minus = _perturbed(wl, name, index, h), _perturbed(wl, name, index, -h)
            if not (np.array_equal(oracle.forward(plus, want=("idx",)).idx, idx0) and
                    np.array_equal(oracle.forward(minus, want=("idx",)).idx, idx0)):
                continue  # the perturbation moved a routing decision
            fd = (_loss(plus, dy) - _loss(minus, dy)) / (2 * h)
            an = g[gname][index]
            # central difference: error O(h^2) times third derivatives (the
            # perturbed values are float32 stores of x +- h, exact here)
            assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (name, index, fd, an)
            checked += 1
    assert checked >= 3 * len(names)


def test_backward_listed_experts_equal_full():
    wl = random_workload(_shape(), seed=29)
    dy = np.random.default_rng(3).standard_normal((wl.shape.T, wl.shape.d))
    full = oracle.backward(wl, dy)
    part = oracle.backward(wl, dy, experts=[4, 1])
    for k in ("dw1", "dw2"):
        assert np.array_equal(part[k][0], full[k][4]) and np.array_equal(part[k][1], full[k][1])
    for k in ("dx", "dw_router", "dw_up", "dw1_s"):
        assert np.array_equal(part[k], full[k])
