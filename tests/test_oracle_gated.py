"""Pins of the oracle's gated (SwiGLU) experts.

The explainer page ("LatentMoE: NVIDIA's Latent Mixture of Experts Explained
Through Equations, Architecture, Code and ...", its feed-forward section)
says a gated activation such as SwiGLU adds a gate matrix next to W1 and
changes nothing else; the shaping paper ("Shaping Latent
Mixture-of-Experts ...", its rank tables) names an expert's three matrices
W_g, W_u, W_o.  The reading taken: h = silu(a W_g) * (a W1), out = h W2, for
routed and shared experts alike, with silu(v) = v / (1 + e^-v).

Pins that do not retype the oracle's formula:
  * the dense brute force (every expert on every token, torch's silu);
  * silu(v) - silu(-v) = v and silu(v) + silu(-v) = v tanh(v / 2) (exact
    identities of the logistic function): flipping the sign of every gate
    matrix leaves the routing alone, so y(W_g) - y(-W_g) is the layer with
    the bilinear expert (a W_g) * (a W1), and y(W_g) + y(-W_g) the layer with
    (a W_g) tanh(a W_g / 2) * (a W1) -- both written here with plain matmuls
    and numpy's tanh; the two together fix silu completely;
  * a zero gate bank switches the routed experts off exactly.
"""

import numpy as np
import pytest

from oracle import dense, oracle
from synth import make_workload
from synth.generate import Workload
from tests.helpers import random_fp8_workload, random_workload, shape


def _gshape(**kw):
    base = dict(T=11, d=16, l=8, m=12, n_experts=6, top_k=3, n_shared=2, m_shared=8, dtype="bf16",
                expert_act="swiglu")
    base.update(kw)
    return shape(**base)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


@pytest.mark.parametrize("kw", [dict(), dict(dtype="f32"), dict(n_shared=0), dict(top_k=6, n_experts=6),
                                dict(top_k=1)])
def test_gated_oracle_matches_dense_brute_force(kw):
    wl = random_workload(_gshape(**kw), seed=3)
    r = oracle.forward(wl, want=("y", "u", "z", "logits"))
    ref = dense.layer_dense_from_workload(wl)
    for k in ("logits", "z", "u", "y"):
        assert _rel(getattr(r, k), ref[k]) < 1e-12, k


def test_gated_fp8_oracle_matches_dense_brute_force():
    wl = random_fp8_workload(_gshape(expert_dtype="fp8"), seed=5)
    assert wl.tensors["w1g"].dtype == np.uint8 and "w1g_scale" in wl.tensors
    r = oracle.forward(wl, want=("y", "u"))
    ref = dense.layer_dense_from_workload(wl)
    assert _rel(r.u, ref["u"]) < 1e-12
    assert _rel(r.y, ref["y"]) < 1e-12


def _negated_gates(wl: Workload) -> Workload:
    """The same workload with every gate matrix negated (a sign flip of each
    bf16 / float32 / E4M3 value: exact)."""
    t = dict(wl.tensors)
    for k in ("w1g", "w1g_s"):
        a = t[k]
        if a.dtype == np.uint16:
            t[k] = a ^ np.uint16(0x8000)
        elif a.dtype == np.uint8:
            t[k] = a ^ np.uint8(0x80)
        else:
            t[k] = -a
    return Workload(wl.shape, t)


def _layer_with_act(wl, r, phi):
    """y for the oracle's routing and gates (r.idx, r.gate) with the gated
    activation replaced by phi(g, v) (g = a W_g, v = a W1): plain matmuls."""
    x = wl.f64("x")
    w1 = dense.expert_bank_f64(wl, "w1")
    w2 = dense.expert_bank_f64(wl, "w2")
    wg = dense.expert_bank_f64(wl, "w1g")
    z = x @ wl.f64("w_down")
    u = np.zeros_like(z)
    for t in range(x.shape[0]):
        for k in range(wl.shape.top_k):
            e = r.idx[t, k]
            u[t] += r.gate[t, k] * (phi(z[t] @ wg[e], z[t] @ w1[e]) @ w2[e])
    y = u @ wl.f64("w_up")
    for j in range(wl.shape.n_shared):
        y += phi(x @ wl.f64("w1g_s")[j], x @ wl.f64("w1_s")[j]) @ wl.f64("w2_s")[j]
    return y


@pytest.mark.parametrize("fp8", [False, True])
def test_gate_sign_flip_odd_and_even_parts(fp8):
    sh = _gshape(expert_dtype="fp8" if fp8 else None)
    wl = random_fp8_workload(sh, seed=7) if fp8 else random_workload(sh, seed=7, scale=2.0)
    neg = _negated_gates(wl)
    a = oracle.forward(wl, want=("y", "idx", "gate"))
    b = oracle.forward(neg, want=("y", "idx", "gate"))
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.gate, b.gate)  # the router ignores W_g
    odd = _layer_with_act(wl, a, lambda g, v: g * v)
    even = _layer_with_act(wl, a, lambda g, v: g * np.tanh(g / 2.0) * v)
    assert _rel(a.y - b.y, odd) < 1e-10
    assert _rel(a.y + b.y, even) < 1e-10


def test_zero_gate_bank_switches_routed_experts_off():
    wl = random_workload(_gshape(), seed=11)
    t = dict(wl.tensors)
    t["w1g"] = np.zeros_like(t["w1g"])
    r = oracle.forward(Workload(wl.shape, t), want=("h", "u", "y", "hs"))
    assert np.all(r.h == 0.0) and np.all(r.u == 0.0)
    # y is then the shared experts alone
    x = wl.f64("x")
    ys = sum(dense.silu_torch(x @ wl.f64("w1g_s")[j]) * (x @ wl.f64("w1_s")[j]) @ wl.f64("w2_s")[j]
             for j in range(wl.shape.n_shared))
    assert _rel(r.y, ys) < 1e-12


def test_relu2_workloads_unchanged_by_the_gate_children():
    # the gate banks use seed children 9 and 10 of the recipe; the first nine
    # children, and so every tensor of a non-gated workload, do not depend on
    # how many children are spawned
    for seed in (0, 1, 5):
        a = np.random.SeedSequence(seed).spawn(9)
        b = np.random.SeedSequence(seed).spawn(11)
        for i in range(9):
            assert np.array_equal(a[i].generate_state(4), b[i].generate_state(4))
    sh = shape(T=4, d=64, l=32, m=64, n_experts=16, top_k=2, n_shared=1, m_shared=64, dtype="bf16", seed=9)
    plain = make_workload(sh)
    gated = make_workload(shape(T=4, d=64, l=32, m=64, n_experts=16, top_k=2, n_shared=1, m_shared=64,
                                dtype="bf16", seed=9, expert_act="swiglu"))
    assert "w1g" not in plain.tensors
    for k in ("x", "w_router", "w_down", "w1", "w2", "w_up", "w1_s", "w2_s"):
        assert np.array_equal(plain.tensors[k], gated.tensors[k]), k
    assert gated.tensors["w1g"].shape == (16, 32, 64) and gated.tensors["w1g_s"].shape == (1, 64, 64)
