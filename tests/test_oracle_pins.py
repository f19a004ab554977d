"""Pins of the CPU oracle against facts outside the oracle itself.

Each test checks the fp64 C oracle (and where useful the numpy dense brute
force) against a hand-derived worked example, a closed form, a special case
that reduces to a library routine, or an invariant of the layer defined on
the explainer page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained
Through Equations, Architecture, Code and ..." (Figures 3, 6, 8, 9 and its
MoE / LatentMoE code blocks).
"""

import json
import os
import zlib

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import dense, oracle
from tests.helpers import near_tie_mask, random_workload, shape, workload_from_arrays


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------
# hand-derived worked example
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def hand(golden_dir):
    with open(os.path.join(golden_dir, "handworked_tiny.json")) as f:
        fx = json.load(f)
    s = fx["shape"]
    sh = shape(T=len(fx["x"]), d=s["d"], l=s["l"], m=s["m"], n_experts=s["n_experts"],
               top_k=s["top_k"], n_shared=s["n_shared"], m_shared=s["m_shared"],
               alpha=s["alpha"])
    return fx, workload_from_arrays(sh, fx)


def test_handworked_c_oracle(hand):
    fx, wl = hand
    r = oracle.forward(wl, want=("idx", "gate", "z", "u", "y"))
    ex = fx["expected"]
    assert np.array_equal(r.idx, np.array(ex["idx"]))
    for k in ("gate", "z", "u", "y"):
        np.testing.assert_allclose(getattr(r, k), np.array(ex[k]), rtol=1e-14, atol=1e-14)


def test_handworked_dense(hand):
    fx, wl = hand
    r = dense.layer_dense_from_workload(wl)
    ex = fx["expected"]
    assert np.array_equal(dense.select_lexsort(r["logits"], wl.shape.top_k), np.array(ex["idx"]))
    np.testing.assert_allclose(r["y"], np.array(ex["y"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(r["u"], np.array(ex["u"]), rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# independent formulation: dense evaluation of every expert, masked
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [
    dict(T=16, d=8, l=4, m=6, n_experts=4, top_k=2, n_shared=1, m_shared=5),
    dict(T=9, d=16, l=4, m=12, n_experts=12, top_k=3, n_shared=2, m_shared=7, alpha=4),
    dict(T=5, d=6, l=6, m=3, n_experts=3, top_k=3, n_shared=0, m_shared=0, alpha=1),
    dict(T=7, d=8, l=8, m=5, n_experts=1, top_k=1, n_shared=1, m_shared=4, alpha=1),
    dict(T=12, d=16, l=8, m=8, n_experts=8, top_k=4, n_shared=1, m_shared=8, dtype="bf16"),
    dict(T=11, d=16, l=8, m=8, n_experts=8, top_k=2, n_shared=1, m_shared=8, zipf_s=1.1),
])
def test_c_oracle_matches_dense_bruteforce(cfg):
    sh = shape(**cfg)
    wl = random_workload(sh, seed=zlib.crc32(repr(sorted(cfg.items())).encode()) % 1000)
    r = oracle.forward(wl, want=("logits", "idx", "gate", "z", "u", "y"))
    d = dense.layer_dense_from_workload(wl)
    np.testing.assert_allclose(r.logits, d["logits"], rtol=1e-12, atol=1e-13)
    assert np.array_equal(r.idx, dense.select_lexsort(d["logits"], sh.top_k))
    G = np.take_along_axis(d["G"], r.idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(r.gate, G, rtol=1e-12, atol=1e-15)
    assert _rel(r.z, d["z"]) < 1e-12
    assert _rel(r.u, d["u"]) < 1e-12
    assert _rel(r.y, d["y"]) < 1e-12


def test_c_oracle_matches_dense_on_tiny_config_tokens():
    from synth import get_config, make_workload
    wl = make_workload(get_config("tiny_f32"))
    toks = np.arange(0, 256, 7)
    r = oracle.forward(wl, tokens=toks, want=("idx", "y"))
    d = dense.layer_dense_from_workload(wl, tokens=toks)
    assert np.array_equal(r.idx, dense.select_lexsort(d["logits"], wl.shape.top_k))
    assert _rel(r.y, d["y"]) < 1e-12


# --------------------------------------------------------------------------
# closed forms and special cases
# --------------------------------------------------------------------------
def _identity_layer(T, d, n_shared, rng):
    sh = shape(T=T, d=d, l=d, m=d, n_experts=1, top_k=1, n_shared=n_shared,
               m_shared=d if n_shared else 0, alpha=1)
    I = np.eye(d, dtype=np.float32)
    arr = {"x": rng.standard_normal((T, d)).astype(np.float32),
           "w_router": rng.standard_normal((d, 1)).astype(np.float32),
           "w_down": I, "w1": I[None], "w2": I[None], "w_up": I,
           "w1_s": np.stack([I] * n_shared) if n_shared else np.zeros((0, d, 1), np.float32),
           "w2_s": np.stack([I] * n_shared) if n_shared else np.zeros((0, 1, d), np.float32)}
    return workload_from_arrays(sh, arr), arr["x"].astype(np.float64)


@pytest.mark.parametrize("n_shared", [0, 1, 2])
def test_identity_weights_give_squared_relu(n_shared):
    """One expert, K'=1, every matrix the identity: y = (1 + S) relu(x)^2."""
    wl, x = _identity_layer(10, 6, n_shared, np.random.default_rng(3))
    r = oracle.forward(wl, want=("gate", "y"))
    assert np.all(r.gate == 1.0)
    np.testing.assert_allclose(r.y, (1 + n_shared) * np.maximum(x, 0) ** 2, rtol=1e-15, atol=0)


def test_top1_gate_is_exactly_one_and_argmax():
    sh = shape(T=20, d=8, l=4, m=6, n_experts=7, top_k=1, n_shared=1, m_shared=3)
    wl = random_workload(sh, seed=11)
    r = oracle.forward(wl, want=("logits", "idx", "gate"))
    assert np.all(r.gate == 1.0)
    assert np.array_equal(r.idx[:, 0], np.argmax(r.logits, axis=1))


def test_all_experts_selected_gives_softmax_mixture():
    """K' = N': the gates are the full softmax (scipy), in score order."""
    sh = shape(T=15, d=8, l=4, m=6, n_experts=5, top_k=5, n_shared=1, m_shared=3)
    wl = random_workload(sh, seed=12)
    r = oracle.forward(wl, want=("logits", "idx", "gate", "o", "u"))
    p = sp_softmax(r.logits, axis=1)
    np.testing.assert_allclose(r.gate, np.take_along_axis(p, r.idx.astype(np.int64), 1),
                               rtol=1e-13, atol=1e-16)
    # u is then the softmax-weighted sum of every expert's output
    np.testing.assert_allclose(r.u, np.einsum("tk,tkl->tl", r.gate, r.o), rtol=1e-12)


def test_zero_router_selects_first_experts_uniformly():
    sh = shape(T=6, d=8, l=4, m=6, n_experts=9, top_k=4, n_shared=1, m_shared=3)
    rng = np.random.default_rng(5)
    from tests.helpers import random_arrays
    arr = random_arrays(sh, rng)
    arr["w_router"] = np.zeros_like(arr["w_router"])
    r = oracle.forward(workload_from_arrays(sh, arr), want=("idx", "gate"))
    assert np.array_equal(r.idx, np.tile(np.arange(4, dtype=np.int32), (6, 1)))
    np.testing.assert_allclose(r.gate, 0.25, rtol=1e-15)


def test_standard_moe_reduction():
    """alpha = 1 with W_down = W_up = I is the standard MoE of the explainer's
    MoE code block: experts at width d, weighted sum, plus shared experts.
    The reference here is scipy's softmax plus per-token expert evaluation."""
    d = 6
    sh = shape(T=9, d=d, l=d, m=5, n_experts=6, top_k=2, n_shared=1, m_shared=4, alpha=1)
    rng = np.random.default_rng(8)
    from tests.helpers import random_arrays
    arr = random_arrays(sh, rng)
    arr["w_down"] = np.eye(d, dtype=np.float32)
    arr["w_up"] = np.eye(d, dtype=np.float32)
    wl = workload_from_arrays(sh, arr)
    r = oracle.forward(wl, want=("y",))
    f = {k: np.asarray(v, np.float64) for k, v in arr.items()}
    y = np.zeros((9, d))
    for t in range(9):
        s = f["x"][t] @ f["w_router"]
        top = sorted(range(6), key=lambda e: (-s[e], e))[:2]
        p = sp_softmax(s)[top]
        p = p / p.sum()
        for g, e in zip(p, top):
            y[t] += g * (np.maximum(f["x"][t] @ f["w1"][e], 0) ** 2 @ f["w2"][e])
        y[t] += np.maximum(f["x"][t] @ f["w1_s"][0], 0) ** 2 @ f["w2_s"][0]
    np.testing.assert_allclose(r.y, y, rtol=1e-12, atol=1e-14)


def test_projections_apply_around_the_experts():
    """Rank-one check of where W_down and W_up sit: with one expert whose
    matrices are identities in l, y = relu(x W_down)^2 W_up."""
    d, l = 8, 2
    sh = shape(T=7, d=d, l=l, m=l, n_experts=1, top_k=1, n_shared=0, m_shared=0, alpha=4)
    rng = np.random.default_rng(9)
    I = np.eye(l, dtype=np.float32)
    arr = {"x": rng.standard_normal((7, d)).astype(np.float32),
           "w_router": rng.standard_normal((d, 1)).astype(np.float32),
           "w_down": rng.standard_normal((d, l)).astype(np.float32), "w1": I[None],
           "w2": I[None], "w_up": rng.standard_normal((l, d)).astype(np.float32),
           "w1_s": np.zeros((0, d, 1), np.float32), "w2_s": np.zeros((0, 1, d), np.float32)}
    r = oracle.forward(workload_from_arrays(sh, arr), want=("z", "y"))
    f = {k: v.astype(np.float64) for k, v in arr.items()}
    z = f["x"] @ f["w_down"]
    np.testing.assert_allclose(r.z, z, rtol=1e-14)
    np.testing.assert_allclose(r.y, (np.maximum(z, 0) ** 2) @ f["w_up"], rtol=1e-13)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_degree_two_homogeneity_under_fixed_routing():
    """With the routing fixed, every path is linear -> squared ReLU -> linear,
    so y(c x) = c^2 y(x) for c > 0; a dropped square or a misplaced
    nonlinearity breaks it."""
    sh = shape(T=10, d=8, l=4, m=6, n_experts=5, top_k=2, n_shared=1, m_shared=3)
    from tests.helpers import random_arrays
    arr = random_arrays(sh, np.random.default_rng(21))
    arr["w_router"] = np.zeros_like(arr["w_router"])     # gates fixed at 1/K'
    wl = workload_from_arrays(sh, arr)
    r1 = oracle.forward(wl, want=("idx", "y"))
    x2 = (wl.f32("x") * np.float32(4.0)).astype(np.float32)
    r2 = oracle.forward(wl.with_x(x2), want=("idx", "y"))
    assert np.array_equal(r1.idx, r2.idx)
    np.testing.assert_allclose(r2.y, 16.0 * r1.y, rtol=1e-12, atol=1e-12)


def test_negative_preactivations_vanish():
    """All W1 entries and x nonnegative, W_down nonnegative -> pre-activations
    >= 0 for x >= 0 and <= 0 for x <= 0: the routed and shared paths give
    exactly zero on -x."""
    sh = shape(T=6, d=8, l=4, m=6, n_experts=4, top_k=2, n_shared=1, m_shared=3)
    rng = np.random.default_rng(4)
    from tests.helpers import random_arrays
    arr = random_arrays(sh, rng)
    for k in ("w_down", "w1", "w1_s"):
        arr[k] = np.abs(arr[k])
    arr["x"] = -np.abs(arr["x"])
    r = oracle.forward(workload_from_arrays(sh, arr), want=("u", "y"))
    assert np.all(r.u == 0.0) and np.all(r.y == 0.0)


def test_token_permutation_equivariance():
    sh = shape(T=13, d=8, l=4, m=6, n_experts=6, top_k=3, n_shared=1, m_shared=5)
    wl = random_workload(sh, seed=31)
    perm = np.random.default_rng(1).permutation(13)
    r1 = oracle.forward(wl, want=("y",))
    r2 = oracle.forward(wl.with_x(np.ascontiguousarray(wl.tensors["x"][perm])), want=("y",))
    assert np.array_equal(r2.y, r1.y[perm])
    r3 = oracle.forward(wl, tokens=perm, want=("y",))
    assert np.array_equal(r3.y, r1.y[perm])


def test_expert_relabelling_invariance():
    sh = shape(T=12, d=8, l=4, m=6, n_experts=6, top_k=3, n_shared=1, m_shared=5)
    rng = np.random.default_rng(41)
    from tests.helpers import random_arrays
    arr = random_arrays(sh, rng)
    q = rng.permutation(6)
    arr2 = dict(arr)
    arr2["w_router"] = arr["w_router"][:, q]
    arr2["w1"] = arr["w1"][q]
    arr2["w2"] = arr["w2"][q]
    r1 = oracle.forward(workload_from_arrays(sh, arr), want=("idx", "y"))
    r2 = oracle.forward(workload_from_arrays(sh, arr2), want=("idx", "y"))
    assert np.array_equal(q[r2.idx], r1.idx)
    np.testing.assert_allclose(r2.y, r1.y, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_routing_invariants(dtype):
    sh = shape(T=64, d=16, l=8, m=8, n_experts=16, top_k=5, n_shared=1, m_shared=8, dtype=dtype)
    wl = random_workload(sh, seed=51)
    r = oracle.forward(wl, want=("logits", "idx", "gate"))
    np.testing.assert_allclose(r.gate.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(r.gate, axis=1) <= 1e-15)          # slots in score order
    for t in range(sh.T):
        assert len(set(r.idx[t])) == sh.top_k
        s = r.logits[t]
        sel = r.idx[t]
        assert np.min(s[sel]) >= np.max(np.delete(s, sel))


# --------------------------------------------------------------------------
# selection with ties and the dispatch order
# --------------------------------------------------------------------------
def test_select_with_ties_matches_lexsort():
    rng = np.random.default_rng(61)
    s = rng.integers(-3, 4, size=(200, 24)).astype(np.float64)   # many exact ties
    for K in (1, 3, 8, 24):
        assert np.array_equal(oracle.select(s, K), dense.select_lexsort(s, K))


def test_select_signed_zero_is_a_tie():
    s = np.array([[-0.0, 0.0, -1.0, 0.0]])
    assert np.array_equal(oracle.select(s, 2), np.array([[0, 1]]))


def test_gates_match_scipy_renormalised_softmax():
    rng = np.random.default_rng(62)
    s = rng.standard_normal((50, 32)) * 3
    idx = dense.select_lexsort(s, 6)
    p = sp_softmax(s, axis=1)
    ref = np.take_along_axis(p, idx.astype(np.int64), 1)
    ref /= ref.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(oracle.gates(s, idx), ref, rtol=1e-13)


def _random_idx(rng, T, K, N):
    return np.stack([rng.choice(N, size=K, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,K,N", [(1, 1, 1), (7, 3, 5), (64, 6, 256), (300, 16, 40), (33, 4, 4)])
def test_dispatch_matches_stable_argsort_and_definition(T, K, N):
    rng = np.random.default_rng(T * 1000 + K)
    idx = _random_idx(rng, T, K, N)
    dp = oracle.dispatch(idx, N)
    c, o, p, pm = dense.dispatch_argsort(idx, N)
    assert np.array_equal(dp.counts, c) and np.array_equal(dp.offsets, o)
    assert np.array_equal(dp.pos, p) and np.array_equal(dp.perm, pm)
    # the definition, brute force: pos = offsets[e] + #{t' < t : e in idx[t']}
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            assert dp.pos[t, k] == dp.offsets[e] + int(np.sum(idx[:t] == e))
    # a bijection onto [0, T*K) with perm[pos[t,k]] = t
    assert np.array_equal(np.sort(dp.pos.reshape(-1)), np.arange(T * K))
    assert np.all(dp.perm[dp.pos] == np.arange(T)[:, None])
    assert dp.offsets[-1] == T * K and np.all(np.diff(dp.offsets) >= 0)


def test_dispatch_rejects_bad_indices():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 0]], dtype=np.int32), 4)
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 4]], dtype=np.int32), 4)
