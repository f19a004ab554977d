"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle on
the same seeded inputs.

  * routing, every token: the GPU's experts, slot order and gates equal the
    oracle's selection rule and renormalised gates applied to the GPU's own
    fp32 scores (experts bit for bit, gates to an fp32 rounding bound); the
    scores within DELTA/2 of the oracle's fp64 scores; on every token whose
    oracle top-(K'+1) scores are DELTA apart, the oracle's fp64 routing;
  * dispatch: bit-exact against the oracle's counting sort of the GPU's
    expert choices, and its defining properties;
  * every intermediate (z, h_s, H, Y, u) on decided tokens, to the bars of
    tests/tolerances.py (each derived from the bf16 rounding points);
  * the layer output: max (|y - y_oracle| - half an output ulp) <= 2e-2
    RMS(y_oracle) for bf16, 1e-4 for fp32, excluding tokens whose K'-th and
    (K'+1)-th oracle scores are closer than 1e-3.
Full-size workloads are checked on every token (readme_acc, decode_eff) or
on at least 1024 tokens (wide_prefill, zipf_skew, shape_swiglu).
"""

import numpy as np
import pytest
import torch

from mixture_experts_layer_latentmoe_amd import _abi
from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
from oracle import oracle
from synth import get_config, make_workload
from tests import cases as C
from tests import gpu_util as G
from tests.helpers import random_arrays, random_workload, shape, workload_from_arrays

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()  # the HIP library must be there; raises otherwise


def _full_check(wl, n_sample=None):
    return G.full_check(wl, n_sample)


def test_tiny_f32_all_tokens():
    _full_check(make_workload(get_config("tiny_f32")))


def test_readme_weights_ragged_tokens():
    """300 tokens: 19 router chunks of 16 tokens, the last one ragged."""
    _full_check(make_workload(get_config("readme_acc"), T=300))


def test_zipf_bias_ragged_tokens():
    _full_check(make_workload(get_config("zipf_skew"), T=231))


@pytest.mark.parametrize("T", [64, 40])
def test_zipf_decode_multi_tile_experts(T):
    """Decode batches whose biased router gives several experts up to T rows:
    two 32-row tiles per such expert (the second ragged at T = 40 and for the
    experts with 63 rows), through the per-tile A-row table of the first
    grouped GEMM."""
    wl = make_workload(get_config("zipf_skew"), T=T)
    counts = np.bincount(G.oracle_routing(wl).idx.ravel(), minlength=wl.shape.n_experts)
    assert counts.max() > 32
    _full_check(wl)


@pytest.mark.parametrize("name,n_sample", [("readme_acc", None), ("decode_eff", None),
                                           ("wide_prefill", 1024), ("zipf_skew", 1024)])
def test_full_size(name, n_sample):
    """Full-size workloads: routing and dispatch on every token; the output
    and every intermediate on every token (readme_acc, decode_eff) or on
    1024 seeded tokens including the first and the last."""
    _full_check(make_workload(get_config(name)), n_sample=n_sample)


def test_large_ragged_token_count():
    """4059 tokens at the README widths: the x-pass on 256x256 tiles and the
    up-projection on 128x256 tiles (both with the software-pipelined fragment
    reads) end in a ragged row tile (219 and 91 rows); output and every
    intermediate on 1024 seeded tokens including the first and the last."""
    _full_check(make_workload(get_config("readme_acc"), T=4059), n_sample=1024)


def test_single_token():
    _full_check(make_workload(get_config("readme_acc"), T=1))


def test_one_handle_many_token_counts():
    wl = make_workload(get_config("tiny_f32"))
    layer = LatentMoE.from_workload(wl, max_tokens=256)
    try:
        for T in (256, 17, 1, 100):
            sub = wl.with_x(np.ascontiguousarray(wl.tensors["x"][:T]))
            out = G.run_gpu(sub, layer=layer)
            G.check_routing(out, sub, G.oracle_routing(sub))
            toks = np.arange(T)
            ref = oracle.forward(sub, want=("logits", "y"))
            G.check_output(out, sub, ref, toks)
    finally:
        layer.close()


def test_zero_router_ties_fill_first_experts():
    """W_r = 0: every score ties, so every token takes experts 0..K'-1 with
    gates 1/K' and four experts hold all 1000 tokens (many tiles each)."""
    sh = shape(T=1000, d=256, l=128, m=192, n_experts=32, top_k=4, n_shared=1, m_shared=128,
               dtype="bf16")
    arr = random_arrays(sh, np.random.default_rng(3))
    arr["w_router"] = np.zeros_like(arr["w_router"])
    wl = workload_from_arrays(sh, arr)
    out = G.run_gpu(wl)
    # exact ties everywhere: the index rule decides, on both sides
    assert np.all(out["logits"] == 0.0)
    assert np.all(out["idx"] == np.arange(4, dtype=np.int32)[None, :])
    assert np.all(out["gate"] == np.float32(0.25))
    G.check_dispatch_properties(out, 4, 32)
    ref_route = G.oracle_routing(wl)
    assert np.array_equal(ref_route.idx, out["idx"])
    dp = oracle.dispatch(ref_route.idx, 32)
    assert np.array_equal(out["pos"], dp.pos) and np.array_equal(out["perm_token"], dp.perm)
    toks = np.arange(1000)
    ref = oracle.forward(wl, tokens=toks, want=("logits", "idx", "gate", "z", "h", "o", "u", "hs", "y"))
    G.check_stages(out, wl, ref, toks, np.ones(len(toks), dtype=bool))


@pytest.mark.parametrize("T", C.TILE_ROWS)
def test_expert_rows_at_tile_boundaries(T):
    """W_r = 0 on a bf16 prefill shape: experts 0..3 hold exactly T rows each
    and the other 12 none.  The bf16 forward's grouped GEMMs take 256-row
    tiles whose last one per expert holds up to 320 rows: full tiles, one row
    short or long, the 320-row maximum and one past it.  Every token is
    checked, stage by stage."""
    sh = C.tile_rows_shape(T)
    arr = random_arrays(sh, np.random.default_rng(T))
    arr["w_router"] = np.zeros_like(arr["w_router"])
    wl = workload_from_arrays(sh, arr)
    out = G.run_gpu(wl)
    assert np.all(out["idx"] == np.arange(4, dtype=np.int32)[None, :])
    assert np.array_equal(out["counts"], np.array([T] * 4 + [0] * 12, dtype=out["counts"].dtype))
    toks = np.arange(T)
    ref = oracle.forward(wl, tokens=toks, want=("logits", "idx", "gate", "z", "h", "o", "u", "hs", "y"))
    G.check_stages(out, wl, ref, toks, np.ones(T, dtype=bool))


@pytest.mark.parametrize("zero_router,T", [(True, 1300), (False, 2048)])
def test_grouped_gemm2_320_column_tiles(zero_router, T):
    """l = 640 with more than 320 rows per expert on average: the 256-row tile
    table without extra rows, where grouped GEMM 2 (N = l) takes 256x320
    tiles, two per row block instead of three 256-column ones.  A zero
    router gives experts 0..3 exactly 1300 rows (5 full tiles and one of 20
    rows); a random one about 512 rows each.  Every token, stage by stage."""
    sh = shape(T=T, d=1280, l=640, m=192, n_experts=16, top_k=4, n_shared=1, m_shared=128, dtype="bf16")
    arr = random_arrays(sh, np.random.default_rng(T))
    if zero_router:
        arr["w_router"] = np.zeros_like(arr["w_router"])
    wl = workload_from_arrays(sh, arr)
    if not zero_router:
        out = _full_check(wl)
        assert out["counts"].min() > 320
        return
    out = G.run_gpu(wl)
    assert np.array_equal(out["counts"], np.array([T] * 4 + [0] * 12, dtype=out["counts"].dtype))
    toks = np.arange(T)
    ref = oracle.forward(wl, tokens=toks, want=("logits", "idx", "gate", "z", "h", "o", "u", "hs", "y"))
    G.check_stages(out, wl, ref, toks, np.ones(T, dtype=bool))


def test_expert_rows_straddle_tile_height():
    """2048 tokens over 16 experts with K' = 2: about 256 rows per expert,
    some just under and some just over one 256-row tile."""
    sh = shape(T=2048, d=256, l=128, m=192, n_experts=16, top_k=2, n_shared=1, m_shared=128, dtype="bf16")
    out = _full_check(random_workload(sh, seed=11))
    assert out["counts"].min() < 256 < out["counts"].max()


# --------------------------------------------------------------------------
# fused expert MLP: H stays on chip; Y is compared stage by stage (the debug
# H output comes from grouped GEMM 1 run beside it)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("l,T", C.FUSED_TILE_ROWS)
def test_fused_mlp_rows_at_tile_boundaries(l, T):
    """Zero router, K' = N' = 16: every expert holds exactly T rows, so its
    last fused tile (128 rows at l = 512, 64 at l = 1024) is full, one row
    short or one row long; every token, stage by stage."""
    sh = C.fused_tile_rows_shape(l, T)
    arr = random_arrays(sh, np.random.default_rng(T))
    arr["w_router"] = np.zeros_like(arr["w_router"])
    wl = workload_from_arrays(sh, arr)
    out = G.run_gpu(wl)
    assert np.all(out["idx"] == np.arange(16, dtype=np.int32)[None, :])
    assert np.array_equal(out["counts"], np.full(16, T, dtype=out["counts"].dtype))
    toks = np.arange(T)
    ref = oracle.forward(wl, tokens=toks, want=("logits", "idx", "gate", "z", "h", "o", "u", "hs", "y"))
    G.check_stages(out, wl, ref, toks, np.ones(T, dtype=bool))


@pytest.mark.parametrize("cfg", C.FUSED_SHAPES)
def test_fused_mlp_random_routing(cfg):
    _full_check(C.fused_workload(cfg))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_score_ties_follow_index_order(dtype):
    """Router weights in {-1/4, 0, 1/4} and x in {-1, 0, 1}: every score is a
    multiple of 1/4, exact in fp32 and fp64 alike, with many exact ties.  The
    selection, its slot order (ties to the lower index) and the dispatch
    permutation must equal the oracle's on every token."""
    sh = shape(T=200, d=256, l=128, m=128, n_experts=64, top_k=8, n_shared=1, m_shared=128, dtype=dtype)
    rng = np.random.default_rng(17)
    arr = random_arrays(sh, rng)
    arr["w_router"] = (rng.integers(-1, 2, size=(256, 64)) * 0.25).astype(np.float32)
    arr["x"] = rng.integers(-1, 2, size=(200, 256)).astype(np.float32)
    wl = workload_from_arrays(sh, arr)
    out = G.run_gpu(wl)
    ref = G.oracle_routing(wl)
    assert np.array_equal(out["logits"].astype(np.float64), ref.logits)
    srt = -np.sort(-ref.logits, axis=1)
    assert np.mean(np.any(srt[:, :8] == srt[:, 1:9], axis=1)) > 0.5   # ties are common
    assert np.array_equal(out["idx"], ref.idx)
    np.testing.assert_allclose(out["gate"], ref.gate, rtol=1e-5, atol=1e-7)
    G.check_dispatch_properties(out, 8, 64)
    dp = oracle.dispatch(ref.idx, 64)
    assert np.array_equal(out["pos"], dp.pos) and np.array_equal(out["perm_token"], dp.perm)
    assert np.array_equal(out["counts"], dp.counts) and np.array_equal(out["offsets"], dp.offsets)


@pytest.mark.parametrize("cfg", C.EDGE_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shape_edge_cases(cfg, dtype):
    """K' = 1, K' = N', no shared expert, odd tile multiples, alpha = 1, the
    largest expert count."""
    _full_check(C.edge_workload(cfg, dtype))


@pytest.mark.parametrize("T", [512, 64, 5])
def test_deterministic_bits(T):
    # T = 64 and 5 take the split-K dense GEMMs: partial sums are added in
    # split order, so the bits must not depend on the order the splits finish
    wl = make_workload(get_config("readme_acc"), T=T)
    layer = LatentMoE.from_workload(wl)
    try:
        a = G.run_gpu(wl, layer=layer)
        b = G.run_gpu(wl, layer=layer)
        c = G.run_gpu(wl, layer=layer)
    finally:
        layer.close()
    for k in ("idx", "gate", "pos", "perm_token", "y", "h", "u"):
        assert np.array_equal(a[k], c[k]), k
    for k in ("idx", "gate", "pos", "perm_token", "y", "h", "u"):
        assert np.array_equal(a[k], b[k]), k


def test_forward_argument_errors():
    wl = make_workload(get_config("tiny_f32"), T=8)
    layer = LatentMoE.from_workload(wl, max_tokens=8)
    try:
        x = to_device(wl.tensors["x"], "f32", "cuda:0")
        y = torch.empty_like(x)
        s = torch.cuda.current_stream().cuda_stream
        L = _abi.lib()
        import ctypes
        for T in (0, 9, -1):
            assert L.latentmoe_forward(ctypes.c_void_p(layer.handle), ctypes.c_void_p(x.data_ptr()),
                                       ctypes.c_void_p(y.data_ptr()), T, ctypes.c_void_p(s), None) == \
                _abi.LATENTMOE_ERR_INVALID_ARGUMENT
        # in place (x and y overlap) is rejected
        assert L.latentmoe_forward(ctypes.c_void_p(layer.handle), ctypes.c_void_p(x.data_ptr()),
                                   ctypes.c_void_p(x.data_ptr()), 8, ctypes.c_void_p(s), None) == \
            _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    finally:
        layer.close()


def test_profile_stage_mask_times_only_selected_stages():
    wl = make_workload(get_config("tiny_f32"), T=64)
    layer = LatentMoE.from_workload(wl, max_tokens=64)
    try:
        x = to_device(wl.tensors["x"], "f32", "cuda:0")
        y = torch.empty_like(x)
        names = [_abi.latentmoe_stage_name(i) for i in range(_abi.LATENTMOE_MAX_STAGES)]
        names = [n for n in names if n]
        sel = names.index("grouped_gemm1_relu2")
        L = _abi.lib()
        import ctypes
        assert L.latentmoe_profile_begin(ctypes.c_void_p(layer.handle), 4, 0) == \
            _abi.LATENTMOE_ERR_INVALID_ARGUMENT  # empty mask
        _abi.latentmoe_profile_begin(layer.handle, 4, 1 << sel)
        for _ in range(3):
            layer.forward(x, y)
        st = _abi.latentmoe_profile_end(layer.handle)
        assert st["grouped_gemm1_relu2"][1] == 3 and st["grouped_gemm1_relu2"][0] > 0
        assert all(n == 0 for k, (ms, n) in st.items() if k != "grouped_gemm1_relu2")
        # the mask changes no result
        ref = G.run_gpu(wl)["y"]
        layer.forward(x, y)
        assert np.array_equal(y.cpu().numpy(), ref)
    finally:
        layer.close()


# --------------------------------------------------------------------------
# FP8 (E4M3) expert banks with per-column scales
# --------------------------------------------------------------------------
def test_fp8_decode_full_size():
    # 64 tokens: the 32-row grouped tiles with E4M3 weight tiles
    _full_check(make_workload(get_config("decode_eff_fp8")), 64)


@pytest.mark.parametrize("T", [300, 7])
def test_fp8_readme_widths(T):
    # 300 tokens x 6 slots: the 128x128 grouped tiles; 7 tokens: a single
    # partial tile per expert
    _full_check(make_workload(get_config("decode_eff_fp8"), T=T))


@pytest.mark.parametrize("cfg", C.FP8_SHAPES)
def test_fp8_shape_edge_cases(cfg):
    _full_check(C.fp8_workload(cfg))


# --------------------------------------------------------------------------
# gated (SwiGLU) experts: gate and value columns interleaved by 8 in the B
# operands, silu(gate) * value in every epilogue
# --------------------------------------------------------------------------
def test_swiglu_full_size():
    _full_check(make_workload(get_config("shape_swiglu")), n_sample=1024)


@pytest.mark.parametrize("T", [300, 130, 64, 7])
def test_swiglu_token_counts(T):
    # 300: 128x128 tiles (staged gated epilogue); 130: split-K x-pass (its
    # reduce pairs the gate and value groups); 64 and 7: the few-row kernel
    # with 64 and 32 rows, and the 32-row grouped tiles
    _full_check(C.swiglu_tokens_workload(T))


@pytest.mark.parametrize("cfg", C.SWIGLU_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_swiglu_shape_edge_cases(cfg, dtype):
    _full_check(C.swiglu_workload(cfg, dtype))


@pytest.mark.parametrize("cfg", C.FP8_SHAPES)
def test_swiglu_fp8_banks(cfg):
    _full_check(C.swiglu_fp8_workload(cfg))
