"""GPU parity of the backward pass: latentmoe_backward (through the C ABI)
against the fp64 oracle's orc_backward on the same seeded inputs and the
same dy (never anything the GPU computed).

dy is zero on tokens whose K'-th and (K'+1)-th oracle scores are closer
than 1e-3, so a routing decision that fp32 scores may take differently
contributes to no gradient on either side.

Bars (|d| / (|ref| + RMS(ref)) elementwise, the forward's stage metric):
  * f32 layers: 1e-4 (measured: 1e-5 and below);
  * bf16 layers: one bar per gradient (tests/tolerances.py), each at least
    twice the error that an exact emulation of the backward's bf16 rounding
    points (dY, dH, dA, dz, ds and the recomputed forward's intermediates
    rounded once each, sums exact) reaches on these shapes and seeds;
    tests/test_tolerance_derivation.py recomputes them.
"""

import ctypes

import numpy as np
import pytest
import torch

from mixture_experts_layer_latentmoe_amd import _abi
from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
from oracle import oracle
from synth import get_config, make_workload
from synth.generate import bf16_bits_to_f32, f32_to_bf16_bits
from tests import cases as C
from tests import gpu_util as G
from tests import tolerances as TOL
from tests.helpers import near_tie_mask, random_workload, shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


def _dy(wl, seed=17):
    sh = wl.shape
    r = oracle.forward(wl, want=("logits",))
    keep = ~near_tie_mask(r.logits, sh.top_k, 1e-3)
    dy = np.random.default_rng(seed).standard_normal((sh.T, sh.d)).astype(np.float32) * keep[:, None]
    if sh.dtype == "bf16":
        store = f32_to_bf16_bits(dy)
        return store, bf16_bits_to_f32(store).astype(np.float64)
    return dy, dy.astype(np.float64)


def _gpu_grads(wl, dy_store, layer=None):
    sh = wl.shape
    own = layer is None
    if own:
        layer = LatentMoE.from_workload(wl)
    x = to_device(wl.tensors["x"], sh.dtype, "cuda:0")
    dyt = to_device(dy_store, sh.dtype, "cuda:0")
    g = layer.backward(x, dyt)
    torch.cuda.synchronize()
    out = {k: v.float().cpu().numpy() for k, v in g.items()}
    if own:
        layer.close()
    return out


def _check(wl, experts=None):
    sh = wl.shape
    G.say(f"[gpu] backward {sh.name}: T={sh.T} d={sh.d} N'={sh.n_experts} K'={sh.top_k} {sh.dtype} {sh.expert_act}")
    dy_store, dy64 = _dy(wl)
    ex = list(range(sh.n_experts)) if experts is None else experts
    ref = oracle.backward(wl, dy64, experts=ex)
    got = _gpu_grads(wl, dy_store)
    names = {"dw1g": "dw1_gate", "dw1g_s": "dw1_shared_gate", "dw1_s": "dw1_shared", "dw2_s": "dw2_shared"}
    errs = {}
    for k, v in ref.items():
        gk = names.get(k, k)
        if v.size == 0 or gk not in got:
            continue
        g = got[gk]
        bank = k in ("dw1", "dw2", "dw1g")
        if bank:
            g = g[ex]
        errs[gk] = G.elem_err(g, v)
        assert errs[gk] <= TOL.backward_bar(sh, gk), (gk, errs[gk])
    G.say("[gpu]   gradient errors, max |d| / (|ref| + RMS): " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    expected = {"dx", "dw_router", "dw_down", "dw1", "dw2", "dw_up"}
    if sh.n_shared > 0:
        expected |= {"dw1_shared", "dw2_shared"}
    if sh.expert_act == "swiglu":
        expected |= {"dw1_gate"} | ({"dw1_shared_gate"} if sh.n_shared > 0 else set())
    if sh.has_bias:
        expected |= {"db_router"}
    assert expected <= set(errs), expected - set(errs)


def test_backward_tiny_f32():
    _check(make_workload(get_config("tiny_f32")))


@pytest.mark.parametrize("cfg", C.BACKWARD_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_shapes(cfg, dtype):
    # 300 rows: tiled x-pass and grouped GEMMs; 40 and 9: the few-row kernel;
    # 130: split-K; a router bias; no shared expert; K' = N'
    _check(C.backward_workload(cfg, dtype))


@pytest.mark.parametrize("T", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_one_and_two_tokens(T, dtype):
    # every expert but K' (or 2 K') has no rows: their bank gradients are zeros
    cfg = dict(T=T, d=256, l=128, m=128, n_experts=16, top_k=4, n_shared=1, m_shared=192, alpha=2)
    _check(random_workload(shape(dtype=dtype, **cfg), seed=40 + T))


@pytest.mark.parametrize("T", [300, 64])
def test_backward_readme_widths(T):
    _check(make_workload(get_config("readme_acc"), T=T), experts=[0, 7, 100, 255])


def test_backward_gated_shape_widths():
    _check(make_workload(get_config("shape_swiglu"), T=130), experts=[0, 9, 511])


def test_backward_full_size_readme_dx_sample():
    # 4096 tokens, 98304 dispatch rows on the GPU; dx of a token depends on
    # that token alone, so the oracle runs on a sample of 64 of them
    wl = make_workload(get_config("readme_acc"))
    dy_store, dy64 = _dy(wl)
    got = _gpu_grads(wl, dy_store)
    toks = G.sample_tokens(wl.shape.T, 64, seed=5)
    sub = wl.with_x(wl.tensors["x"][toks])
    ref = oracle.backward(sub, dy64[toks], experts=[])
    err = G.elem_err(got["dx"][toks], ref["dx"])
    G.say(f"[gpu] backward readme_acc full size: dx on {len(toks)} sampled tokens, max |d| / (|ref| + RMS) = {err:.2e}")
    assert err <= TOL.backward_bar(wl.shape, "dx"), err
    for k, v in got.items():
        assert np.all(np.isfinite(v)), k


def test_backward_deterministic_and_repeatable():
    wl = make_workload(get_config("readme_acc"), T=200)
    dy_store, _ = _dy(wl)
    layer = LatentMoE.from_workload(wl)
    try:
        a = _gpu_grads(wl, dy_store, layer)
        x = to_device(wl.tensors["x"], "bf16", "cuda:0")
        y1 = layer.forward(x).float().cpu().numpy()  # a forward between backward calls
        b = _gpu_grads(wl, dy_store, layer)
        y2 = layer.forward(x).float().cpu().numpy()
    finally:
        layer.close()
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(y1, y2)


def test_backward_argument_errors():
    wl = make_workload(get_config("tiny_f32"))
    layer = LatentMoE.from_workload(wl)
    L = _abi.lib()
    try:
        x = to_device(wl.tensors["x"], "f32", "cuda:0")
        g = _abi.latentmoe_grads()
        assert L.latentmoe_backward(ctypes.c_void_p(layer.handle), None, ctypes.c_void_p(x.data_ptr()), 4, None,
                                    ctypes.byref(g)) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
        assert L.latentmoe_backward(ctypes.c_void_p(layer.handle), ctypes.c_void_p(x.data_ptr()),
                                    ctypes.c_void_p(x.data_ptr()), 0, None, ctypes.byref(g)) == \
            _abi.LATENTMOE_ERR_INVALID_ARGUMENT
        db = torch.empty(16, device="cuda:0")
        g.db_router = db.data_ptr()  # tiny_f32 has no router bias
        assert L.latentmoe_backward(ctypes.c_void_p(layer.handle), ctypes.c_void_p(x.data_ptr()),
                                    ctypes.c_void_p(x.data_ptr()), 4, None, ctypes.byref(g)) == \
            _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    finally:
        layer.close()
    fp8 = LatentMoE.from_workload(make_workload(get_config("decode_eff_fp8"), T=4))
    try:
        x = torch.zeros(4, 2048, dtype=torch.bfloat16, device="cuda:0")
        g = _abi.latentmoe_grads()
        assert L.latentmoe_backward(ctypes.c_void_p(fp8.handle), ctypes.c_void_p(x.data_ptr()),
                                    ctypes.c_void_p(x.data_ptr()), 4, None, ctypes.byref(g)) == \
            _abi.LATENTMOE_ERR_UNSUPPORTED
    finally:
        fp8.close()
