"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, validates configs on the host, and its host-side cost counts agree
with the oracle's closed forms."""

import ctypes
import os
import re

import pytest

from mixture_experts_layer_latentmoe_amd import _abi
from oracle import cost as ocost
from synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "latentmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(latentmoe_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = _abi.lib()
    names = _header_functions()
    assert "latentmoe_create" in names and "latentmoe_forward" in names and "latentmoe_destroy" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_abi.EXPORTED)


def _cfg(sh, **over):
    kw = dict(d=sh.d, l=sh.l, m=sh.m, n_experts=sh.n_experts, top_k=sh.top_k, alpha=sh.alpha,
              n_shared=sh.n_shared, m_shared=sh.m_shared, variant=sh.variant, dtype=sh.dtype,
              max_tokens=sh.T, has_router_bias=sh.has_bias, expert_dtype=sh.expert_dtype,
              expert_act=sh.expert_act)
    kw.update(over)
    return _abi.make_config(**kw)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_named_configs_validate(name):
    assert _abi.latentmoe_validate_config(_cfg(CONFIGS[name])) == _abi.LATENTMOE_OK
    assert _abi.latentmoe_workspace_bytes(_cfg(CONFIGS[name])) > 0


@pytest.mark.parametrize("over,status", [
    (dict(l=500), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),         # l * alpha != d
    (dict(top_k=0), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),
    (dict(top_k=300), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),      # K' > N'
    (dict(top_k=22), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),       # acc needs alpha | K'
    (dict(n_experts=258), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),  # alpha must divide N'
    (dict(max_tokens=0), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),
    (dict(n_shared=-1), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),
    (dict(m_shared=0), _abi.LATENTMOE_ERR_INVALID_ARGUMENT),     # S > 0 needs m_s
    (dict(m=1400), _abi.LATENTMOE_ERR_UNSUPPORTED),              # not a multiple of 64
    (dict(n_experts=2048, top_k=24), _abi.LATENTMOE_ERR_UNSUPPORTED),
    (dict(n_experts=4, top_k=4), _abi.LATENTMOE_ERR_UNSUPPORTED),   # N' % 16
    (dict(top_k=68, n_experts=256), _abi.LATENTMOE_ERR_UNSUPPORTED),
    (dict(max_tokens=1 << 27), _abi.LATENTMOE_ERR_UNSUPPORTED),  # T K' overflows int32
])
def test_invalid_configs_are_rejected(over, status):
    assert _abi.latentmoe_validate_config(_cfg(CONFIGS["readme_acc"], **over)) == status


def test_expert_format_checks():
    c = _cfg(CONFIGS["readme_acc"])
    c.expert_format = 7
    assert _abi.latentmoe_validate_config(c) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    # E4M3 expert banks need a bf16 layer
    c = _cfg(CONFIGS["tiny_f32"], expert_dtype="fp8")
    assert _abi.latentmoe_validate_config(c) == _abi.LATENTMOE_ERR_UNSUPPORTED
    assert _abi.latentmoe_validate_config(_cfg(CONFIGS["decode_eff_fp8"])) == _abi.LATENTMOE_OK


def test_fp8_create_needs_scales_before_any_gpu_call():
    L = _abi.lib()
    cfg = _cfg(CONFIGS["decode_eff_fp8"])
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the check comes first
    w = _abi.latentmoe_weights(fake, None, fake, fake, fake, fake, fake, fake, None, None)
    h = ctypes.c_void_p(0)
    assert L.latentmoe_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h)) == \
        _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    assert h.value is None


def test_expert_act_checks():
    c = _cfg(CONFIGS["readme_acc"])
    c.expert_act = 2
    assert _abi.latentmoe_validate_config(c) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    assert _abi.latentmoe_validate_config(_cfg(CONFIGS["readme_acc"], expert_act="swiglu")) == _abi.LATENTMOE_OK
    assert _abi.latentmoe_validate_config(_cfg(CONFIGS["decode_eff_fp8"], expert_act="swiglu")) == _abi.LATENTMOE_OK
    # the gated bank of one expert ([W_g | W1], 2 l m elements) must stay under 2 GiB
    big = _cfg(CONFIGS["readme_acc"], d=32768, l=8192, m=65536, n_experts=16, top_k=4, n_shared=0, max_tokens=8)
    assert _abi.latentmoe_validate_config(big) == _abi.LATENTMOE_OK
    big.expert_act = _abi.LATENTMOE_ACT_SWIGLU
    assert _abi.latentmoe_validate_config(big) == _abi.LATENTMOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("fp8,shared", [(False, True), (False, False), (True, True)])
def test_gated_create_needs_gate_banks_before_any_gpu_call(fp8, shared):
    L = _abi.lib()
    sh = CONFIGS["decode_eff_fp8" if fp8 else "readme_acc"]
    cfg = _cfg(sh, expert_act="swiglu", **({} if shared else dict(n_shared=0)))
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the checks come first
    sc = fake if fp8 else None
    full = dict(w_router=fake, w_down=fake, w1=fake, w2=fake, w_up=fake, w1_shared=fake if shared else None,
                w2_shared=fake if shared else None, w1_scale=sc, w2_scale=sc, w1_gate=fake,
                w1_shared_gate=fake if shared else None, w1_gate_scale=sc)
    missing = ["w1_gate"] + (["w1_shared_gate"] if shared else []) + (["w1_gate_scale"] if fp8 else [])
    for k in missing:
        kw = dict(full)
        kw[k] = None
        w = _abi.latentmoe_weights(**kw)
        h = ctypes.c_void_p(0)
        assert L.latentmoe_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h)) == \
            _abi.LATENTMOE_ERR_INVALID_ARGUMENT, k
        assert h.value is None


def test_gated_cost_counts_three_matrices():
    # a gated expert holds a gate matrix next to W1 (the explainer page's
    # feed-forward paragraph near Figure 9): every expert term scales by 3/2,
    # the projections and the router do not
    sh = CONFIGS["readme_acc"]
    a = _abi.latentmoe_cost(_cfg(sh))
    b = _abi.latentmoe_cost(_cfg(sh, expert_act="swiglu"))
    for k in ("latent_expert_params", "routed_pool_params", "shared_params", "baseline_expert_params",
              "expert_bytes_per_token_fp8"):
        assert b[k] == pytest.approx(1.5 * a[k], rel=1e-15), k
    for k in ("projection_params", "router_params", "a2a_bytes_per_token", "log10_combinations"):
        assert b[k] == a[k], k
    assert b["active_params_per_token"] - a["active_params_per_token"] == pytest.approx(
        0.5 * (a["active_params_per_token"] - a["projection_params"]), rel=1e-15)


def test_eff_variant_allows_any_topk():
    assert _abi.latentmoe_validate_config(_cfg(CONFIGS["readme_acc"], top_k=22, variant="eff")) == 0


def test_bad_dtype_and_variant_rejected():
    c = _cfg(CONFIGS["readme_acc"])
    c.dtype = 7
    assert _abi.latentmoe_validate_config(c) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    c = _cfg(CONFIGS["readme_acc"])
    c.variant = 3
    assert _abi.latentmoe_validate_config(c) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT


def test_null_arguments_rejected_before_any_gpu_call():
    L = _abi.lib()
    assert L.latentmoe_validate_config(None) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    h = ctypes.c_void_p(0)
    cfg = _cfg(CONFIGS["tiny_f32"])
    assert L.latentmoe_create(ctypes.byref(cfg), None, None, ctypes.byref(h)) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    assert h.value is None
    w = _abi.latentmoe_weights()
    assert L.latentmoe_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h)) == \
        _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    assert L.latentmoe_create(ctypes.byref(cfg), ctypes.byref(w), None, None) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    assert L.latentmoe_forward(None, None, None, 1, None, None) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    assert L.latentmoe_forward_noalloc(None, None, None, 1, None) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT
    assert L.latentmoe_destroy(None) == _abi.LATENTMOE_OK
    assert L.latentmoe_profile_begin(None, 1, 0xFFFF) == _abi.LATENTMOE_ERR_INVALID_ARGUMENT


def test_status_strings():
    for s in range(6):
        assert _abi.status_string(s) and _abi.status_string(s) != "unknown status"
    assert _abi.status_string(99) == "unknown status"
    assert _abi.latentmoe_stage_name(0) == "gemm_x_router_down_shared1"
    assert _abi.latentmoe_stage_name(1) == "router_select"
    assert _abi.latentmoe_stage_name(99) == ""


@pytest.mark.parametrize("name", list(CONFIGS))
def test_host_cost_matches_oracle_closed_forms(name):
    sh = CONFIGS[name]
    got = _abi.latentmoe_cost(_cfg(sh))
    ref = ocost.layer_cost(sh.d, sh.l, sh.m, sh.n_experts, sh.top_k, sh.alpha, sh.variant,
                           sh.n_shared, sh.m_shared, matrices=3 if sh.expert_act == "swiglu" else 2)
    pairs = [("latent_expert_params", ref.latent_expert_params),
             ("routed_pool_params", ref.routed_pool_params),
             ("projection_params", ref.projection_params),
             ("router_params", ref.router_params),
             ("layer_params_excl_router", ref.layer_params_excl_router),
             ("active_params_per_token", ref.active_params_per_token),
             ("flops_per_token", ref.flops_per_token),
             ("baseline_expert_params", ref.baseline_expert_params),
             ("baseline_layer_params_excl_router", ref.baseline_layer_params_excl_router),
             ("baseline_active_params_per_token", ref.baseline_active_params_per_token),
             ("expert_bytes_per_token_fp8", ref.expert_weight_bytes_per_token(1.0)),
             ("a2a_bytes_per_token", ocost.all_to_all_bytes_per_token(sh.top_k, sh.l, 0.5, 2.0))]
    for k, v in pairs:
        assert got[k] == pytest.approx(v, rel=1e-12), k
    for k, v in [("log10_combinations", ref.log10_combinations),
                 ("baseline_log10_combinations", ref.baseline_log10_combinations),
                 ("log10_combination_bound", ref.log10_combination_bound)]:
        assert got[k] == pytest.approx(v, abs=1e-9), k


def test_host_cost_reproduces_explainer_running_example():
    # d 4096, l 1024, m 2688, 512 experts, 24 active, 2 shared experts of width 2688
    c = _abi.latentmoe_cost(_abi.make_config(4096, 1024, 2688, 512, 24, 4, 2, 2688, "acc", "bf16", 1))
    assert round(c["layer_params_excl_router"] / 1e6, 1) == 2871.0
    assert round(c["baseline_layer_params_excl_router"] / 1e6, 1) == 2862.6
    assert round(c["active_params_per_token"] / 1e6, 1) == 184.5
    assert round(c["baseline_active_params_per_token"] / 1e6, 1) == 176.2
    assert round(c["expert_bytes_per_token_fp8"] / 1e6) == 132
    assert c["a2a_bytes_per_token"] == 60 * 1024
    assert round(c["log10_combinations"]) == 41
