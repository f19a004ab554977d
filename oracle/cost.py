"""Closed-form cost quantities of a LatentMoE layer and its baseline MoE.

TEST INFRASTRUCTURE ONLY (the GPU library has its own host-side
``latentmoe_cost``; this file is the independent check of it).

The pages never print the cost table as formulas (the Latent-MoE README's
"Inspect the asymptotic cost quantities from Table 1" section only lists a
``cost_summary()`` call).  The formulas below are the plain counts of the
matrices a layer holds and a token touches; every worked number on the
explainer page "LatentMoE: NVIDIA's Latent Mixture of Experts Explained
Through Equations, Architecture, Code and ..." (its MoE section, Figure 9,
the parameter totals after the LatentMoE code block, Figures 11-13 and the
expert-combination count) reproduces from them; tests/golden holds those
numbers with their places on the page.

Symbols: d model width, l = d/alpha latent width, m expert hidden width,
N' routed experts (N = N'/alpha in the baseline), K' active (K = K'/alpha for
variant acc, K = K' for eff), S shared experts of hidden width m_s.
b_w bytes per expert weight; b_out / b_back bytes per element sent to /
returned from an expert.  FLOPs count 2 per multiply-add.  Gated experts
(the explainer's feed-forward section: a gated activation such as SwiGLU
adds a gate matrix next to W1 and changes nothing else) hold and touch
three expert matrices instead of two: ``matrices=3``.
"""

from dataclasses import dataclass
from math import comb, lgamma, log


def log10_comb(n: int, k: int) -> float:
    return (lgamma(n + 1) - lgamma(k + 1) - lgamma(n - k + 1)) / log(10.0)


@dataclass
class LayerCost:
    # latent layer
    latent_expert_params: int
    routed_pool_params: int
    projection_params: int
    router_params: int
    layer_params_excl_router: int
    active_params_per_token: int
    flops_per_token: int
    log10_combinations: float
    # baseline MoE with the same d, m, S, m_s and N = N'/alpha
    baseline_n_experts: int
    baseline_top_k: int
    baseline_expert_params: int
    baseline_routed_pool_params: int
    baseline_layer_params_excl_router: int
    baseline_active_params_per_token: int
    baseline_log10_combinations: float
    log10_combination_bound: float   # alpha * log10 C(N, K)

    def expert_weight_bytes_per_token(self, b_w: float) -> float:
        return self.active_routed_params * b_w

    @property
    def active_routed_params(self) -> int:
        return self.active_params_per_token - self.projection_params - self._shared_params

    _shared_params: int = 0


def layer_cost(d: int, l: int, m: int, n_experts: int, top_k: int, alpha: int,
               variant: str, n_shared: int, m_shared: int, matrices: int = 2) -> LayerCost:
    N, K = n_experts // alpha, (top_k // alpha if variant == "acc" else top_k)
    mm = matrices
    latent_expert = mm * l * m
    shared = n_shared * mm * d * m_shared
    proj = 2 * d * l
    pool = n_experts * latent_expert
    base_expert = mm * d * m
    c = LayerCost(
        latent_expert_params=latent_expert,
        routed_pool_params=pool,
        projection_params=proj,
        router_params=d * n_experts,
        layer_params_excl_router=pool + shared + proj,
        active_params_per_token=top_k * latent_expert + shared + proj,
        flops_per_token=2 * (d * n_experts + 2 * d * l + top_k * mm * l * m + n_shared * mm * d * m_shared),
        log10_combinations=log10_comb(n_experts, top_k),
        baseline_n_experts=N,
        baseline_top_k=K,
        baseline_expert_params=base_expert,
        baseline_routed_pool_params=N * base_expert,
        baseline_layer_params_excl_router=N * base_expert + shared,
        baseline_active_params_per_token=K * base_expert + shared,
        baseline_log10_combinations=log10_comb(N, K),
        log10_combination_bound=alpha * log10_comb(N, K),
    )
    c._shared_params = shared
    return c


def all_to_all_bytes_per_token(top_k: int, width: int, b_out: float, b_back: float) -> float:
    """One round trip per selected expert, ``width`` numbers each way."""
    return top_k * width * (b_out + b_back)


def exact_comb(n: int, k: int) -> int:
    return comb(n, k)


def ridge_flop_per_byte(peak_flops: float, bandwidth: float) -> float:
    return peak_flops / bandwidth


def tokens_to_ridge(ridge: float, b_w: float) -> float:
    """Each weight byte is read once and used in 2*t_exp FLOPs per 1/b_w
    weights: FLOP/byte = 2 t_exp / b_w."""
    return ridge * b_w / 2.0
