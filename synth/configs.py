"""The five named LatentMoE layer workloads (shapes, dtype, seeds).

Shapes follow the pages:
  * ``tiny_f32``      -- the transformer demo shape of the Latent-MoE README
                         ("Transformer Usage": d_model 256, d_ff 256, 8 experts,
                         top-2, alpha 2, one shared expert), run in float32.
  * ``readme_acc``    -- the layer of the Latent-MoE README "Usage" section
                         (d 2048, m 1408, N 64, K 6, alpha 4, two shared experts,
                         variant acc  ->  N' 256, K' 24), 4096 tokens, bf16.
  * ``decode_eff``    -- the same weights, variant eff (K' = K = 6 of 256),
                         64 tokens: the weight-streaming decode regime the
                         explainer page analyses in its byte-count section.
  * ``wide_prefill``  -- the explainer's running example widths (d 4096,
                         l 1024, N' 512) with a synthetic m 1024, K' 16,
                         one shared expert of width 4096, 8192 tokens.
  * ``zipf_skew``     -- the 8B "deeper" regime of Table 1 on the
                         "Shaping Latent Mixture-of-Experts" page (l 640,
                         m 512, N 512, K 16, m_s 1024) with a synthetic
                         d 2560, 16384 tokens, and a router bias
                         b_e = 2 ln(Zipf_1.1 weight of rank e+1) that makes
                         expert loads heavily imbalanced.
  * ``decode_eff_fp8`` -- decode_eff with W1/W2 quantized to FP8 E4M3 (the
                         explainer's byte-count section prices expert weights
                         in FP8): half the expert bytes per decoded token.
"""

from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class LayerShape:
    name: str
    T: int            # tokens (batch x seq flattened)
    d: int            # model width
    l: int            # latent width, d / alpha
    m: int            # routed-expert hidden width
    n_experts: int    # N' (already scaled by alpha)
    top_k: int        # K'
    n_shared: int     # S always-on shared experts (width d in and out)
    m_shared: int     # shared-expert hidden width m_s
    alpha: int
    variant: str      # "acc" or "eff"
    dtype: str        # "f32" or "bf16"
    seed: int         # seed of the weights
    x_seed: Optional[int] = None   # seed of x if it differs from ``seed``
    zipf_s: Optional[float] = None  # router bias exponent (None: no bias)
    expert_dtype: Optional[str] = None  # "fp8": W1/W2 as E4M3 bytes + per-column scales
    expert_act: str = "relu2"  # "swiglu": gated experts silu(W_g a) * (W1 a), routed and shared

    @property
    def P(self) -> int:
        return self.T * self.top_k

    @property
    def has_bias(self) -> bool:
        return self.zipf_s is not None

    def with_tokens(self, T: int) -> "LayerShape":
        kw = dict(self.__dict__)
        kw["T"] = T
        return LayerShape(**kw)


CONFIGS = {
    "tiny_f32": LayerShape("tiny_f32", T=256, d=256, l=128, m=256, n_experts=16,
                           top_k=4, n_shared=1, m_shared=256, alpha=2,
                           variant="acc", dtype="f32", seed=0),
    "readme_acc": LayerShape("readme_acc", T=4096, d=2048, l=512, m=1408,
                             n_experts=256, top_k=24, n_shared=2, m_shared=1408,
                             alpha=4, variant="acc", dtype="bf16", seed=1),
    "decode_eff": LayerShape("decode_eff", T=64, d=2048, l=512, m=1408,
                             n_experts=256, top_k=6, n_shared=2, m_shared=1408,
                             alpha=4, variant="eff", dtype="bf16", seed=1,
                             x_seed=2),
    "wide_prefill": LayerShape("wide_prefill", T=8192, d=4096, l=1024, m=1024,
                               n_experts=512, top_k=16, n_shared=1,
                               m_shared=4096, alpha=4, variant="acc",
                               dtype="bf16", seed=3),
    "zipf_skew": LayerShape("zipf_skew", T=16384, d=2560, l=640, m=512,
                            n_experts=512, top_k=16, n_shared=1, m_shared=1024,
                            alpha=4, variant="acc", dtype="bf16", seed=4,
                            zipf_s=1.1),
    # decode_eff with the routed-expert banks in FP8 (E4M3, one scale per
    # expert and output column), the format the explainer's byte count uses
    "decode_eff_fp8": LayerShape("decode_eff_fp8", T=64, d=2048, l=512, m=1408,
                                 n_experts=256, top_k=6, n_shared=2, m_shared=1408,
                                 alpha=4, variant="eff", dtype="bf16", seed=1,
                                 x_seed=2, expert_dtype="fp8"),
    # gated (SwiGLU) experts at the shaping paper's 8B "deeper" expert widths
    # (its Table 1: l = 640, m = 512, K'/N' = 16/512, shared width 1024),
    # synthetic d = 2560, uniform routing
    "shape_swiglu": LayerShape("shape_swiglu", T=8192, d=2560, l=640, m=512,
                               n_experts=512, top_k=16, n_shared=1, m_shared=1024,
                               alpha=4, variant="acc", dtype="bf16", seed=5,
                               expert_act="swiglu"),
}

CONFIG_ORDER = ["tiny_f32", "readme_acc", "decode_eff", "wide_prefill", "zipf_skew"]


def get_config(name: str) -> LayerShape:
    return CONFIGS[name]
