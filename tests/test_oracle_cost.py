"""The closed-form cost counts against every worked number the explainer page
prints for its running example (tests/golden/explainer_worked_numbers.json,
each entry naming the figure or section it comes from)."""

import json
import os
from math import comb, log10

import numpy as np
import pytest

from oracle import cost


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "explainer_worked_numbers.json")) as f:
        return json.load(f)


def _computed(g):
    r = g["running_example"]
    d, l, m, N, K, a = r["d"], r["l"], r["m"], r["N"], r["K"], r["alpha"]
    S, ms, bw, peak, L = r["n_shared"], r["m_shared"], r["bandwidth_B_per_s"], r["peak_fp4_flops"], r["n_layers"]
    acc = cost.layer_cost(d, l, m, r["n_prime"], r["k_prime_acc"], a, "acc", S, ms)
    eff = cost.layer_cost(d, l, m, r["n_prime"], r["k_prime_eff"], a, "eff", S, ms)
    sup = cost.layer_cost(d, l, m, r["n_prime"], r["k_prime_super"], a, "acc", S, ms)
    fp8 = 1.0
    ridge = cost.ridge_flop_per_byte(peak, bw)
    return {
        "dense_ffn_matrix_params": d * m,
        "standard_expert_params": acc.baseline_expert_params,
        "baseline_routed_pool_params": acc.baseline_routed_pool_params,
        "baseline_active_routed_params": acc.baseline_top_k * acc.baseline_expert_params,
        "w_down_params": acc.projection_params / 2,
        "projection_params": acc.projection_params,
        "projection_overhead_percent": 100.0 * acc.projection_params / acc.routed_pool_params,
        "router_params": acc.router_params,
        "latent_expert_matrix_params": acc.latent_expert_params / 2,
        "latent_expert_params": acc.latent_expert_params,
        "latent_routed_pool_params": acc.routed_pool_params,
        "baseline_layer_params_excl_router": acc.baseline_layer_params_excl_router,
        "latent_layer_params_excl_router": acc.layer_params_excl_router,
        "baseline_active_params": acc.baseline_active_params_per_token,
        "latent_acc_active_params": acc.active_params_per_token,
        "latent_eff_active_params": eff.active_params_per_token,
        "decode_bytes_acc": acc.expert_weight_bytes_per_token(fp8),
        "decode_time_acc_us": acc.expert_weight_bytes_per_token(fp8) / bw * 1e6,
        "decode_bytes_super": sup.expert_weight_bytes_per_token(fp8),
        "decode_bytes_eff": eff.expert_weight_bytes_per_token(fp8),
        "a2a_bytes_acc_KiB": cost.all_to_all_bytes_per_token(r["k_prime_acc"], l, 0.5, 2) / 1024,
        "a2a_bytes_super_KiB": cost.all_to_all_bytes_per_token(r["k_prime_super"], l, 0.5, 2) / 1024,
        "a2a_bytes_eff_KiB": cost.all_to_all_bytes_per_token(r["k_prime_eff"], l, 0.5, 2) / 1024,
        "a2a_out_bytes_per_expert_d": cost.all_to_all_bytes_per_token(1, d, 0.5, 0),
        "a2a_back_bytes_per_expert_d": cost.all_to_all_bytes_per_token(1, d, 0, 2),
        "model_decode_bytes_acc": L * acc.expert_weight_bytes_per_token(fp8),
        "model_decode_bytes_eff": L * eff.expert_weight_bytes_per_token(fp8),
        "model_decode_time_acc_ms": L * acc.expert_weight_bytes_per_token(fp8) / bw * 1e3,
        "model_decode_time_eff_ms": L * eff.expert_weight_bytes_per_token(fp8) / bw * 1e3,
        "combinations_baseline": cost.exact_comb(N, K),
        "log10_combinations_baseline": acc.baseline_log10_combinations,
        "log10_combinations_latent": acc.log10_combinations,
        "log10_combination_bound": acc.log10_combination_bound,
        "orders_of_magnitude_gain": acc.log10_combinations - acc.baseline_log10_combinations,
        "roofline_ridge_flop_per_byte": ridge,
        "tokens_per_expert_to_ridge": cost.tokens_to_ridge(ridge, fp8),
        "iso_cost_identity_product": r["k_prime_acc"] * l,
    }


def _half_unit(printed: str) -> float:
    dec = len(printed.split(".")[1]) if "." in printed else 0
    return 0.5 * 10.0 ** (-dec)


def test_every_printed_number_reproduces(golden):
    got = _computed(golden)
    assert set(got) == {n["name"] for n in golden["numbers"]}
    bad = []
    for n in golden["numbers"]:
        v = got[n["name"]] / n["scale"]
        if abs(v - float(n["printed"])) > _half_unit(n["printed"]) + 1e-12:
            bad.append((n["name"], v, n["printed"]))
    assert not bad, bad


def test_iso_cost_identity_is_exact(golden):
    r = golden["running_example"]
    assert r["k_prime_acc"] * r["l"] == r["K"] * r["d"]


def test_combination_count_against_exact_integer():
    assert abs(cost.log10_comb(512, 24) - log10(comb(512, 24))) < 1e-9
    assert abs(cost.log10_comb(128, 6) - log10(comb(128, 6))) < 1e-12


def test_counts_match_the_tensors_a_token_touches():
    """Parameter and FLOP counts against the shapes of generated tensors."""
    from synth import get_config, make_workload
    sh = get_config("tiny_f32")
    wl = make_workload(sh, T=4)
    t = wl.tensors
    c = cost.layer_cost(sh.d, sh.l, sh.m, sh.n_experts, sh.top_k, sh.alpha, sh.variant,
                        sh.n_shared, sh.m_shared)
    assert c.routed_pool_params == t["w1"].size + t["w2"].size
    assert c.projection_params == t["w_down"].size + t["w_up"].size
    assert c.router_params == t["w_router"].size
    assert c.layer_params_excl_router == (t["w1"].size + t["w2"].size + t["w_down"].size
                                          + t["w_up"].size + t["w1_s"].size + t["w2_s"].size)
    per_expert = t["w1"][0].size + t["w2"][0].size
    macs = (t["w_router"].size + t["w_down"].size + sh.top_k * per_expert + t["w_up"].size
            + t["w1_s"].size + t["w2_s"].size)
    assert c.flops_per_token == 2 * macs
    assert c.active_params_per_token == macs - t["w_router"].size
