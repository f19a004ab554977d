"""Shapes and seeds of the synthetic edge-case layers, shared by the GPU
parity tests and the CPU test that derives their tolerances from an
emulation of the bf16 rounding points (so both run on the same inputs).

No layer arithmetic here.
"""

from synth import get_config, make_workload
from tests.helpers import random_fp8_workload, random_workload, shape

# test_shape_edge_cases: K' = 1, K' = N', no shared expert, odd tile
# multiples, alpha = 1, the dispatch and selection limits.  Seed = T.
EDGE_SHAPES = [
    dict(T=70, d=128, l=64, m=128, n_experts=16, top_k=1, n_shared=1, m_shared=64, alpha=2, variant="eff"),
    dict(T=45, d=128, l=64, m=64, n_experts=16, top_k=16, n_shared=1, m_shared=64, alpha=2, variant="eff"),
    dict(T=64, d=128, l=64, m=128, n_experts=32, top_k=4, n_shared=0, m_shared=0, alpha=2),
    dict(T=99, d=256, l=64, m=320, n_experts=64, top_k=8, n_shared=3, m_shared=192, alpha=4),
    dict(T=40, d=128, l=128, m=64, n_experts=16, top_k=2, n_shared=1, m_shared=64, alpha=1),
    # dispatch at its limits: 1024 experts over 64 chunks (one-workgroup path),
    # then 65 chunks and 1008 experts (two-kernel path, a partial last batch)
    dict(T=1024, d=128, l=64, m=64, n_experts=1024, top_k=8, n_shared=1, m_shared=64, alpha=2),
    dict(T=1040, d=128, l=64, m=64, n_experts=1008, top_k=6, n_shared=0, m_shared=0, alpha=2, variant="eff"),
    # decode-sized batches at the selection's limits: 64 tokens, 1024 experts,
    # K' = 64; and 48 experts (a partial group of 64 scores per lane)
    dict(T=64, d=128, l=64, m=64, n_experts=1024, top_k=64, n_shared=1, m_shared=64, alpha=2),
    dict(T=33, d=128, l=64, m=64, n_experts=48, top_k=6, n_shared=1, m_shared=64, alpha=2),
]

# test_fp8_shape_edge_cases (seed = T) and test_swiglu_fp8_banks (seed = T + 2)
FP8_SHAPES = [
    dict(T=96, d=128, l=64, m=192, n_experts=16, top_k=4, n_shared=1, m_shared=64, alpha=2),
    dict(T=33, d=256, l=128, m=64, n_experts=32, top_k=8, n_shared=0, m_shared=0, alpha=2),
]

# test_swiglu_shape_edge_cases (seed = T + 1)
SWIGLU_SHAPES = [
    # x-pass gated columns from 144: the 128-column tile [128, 256) holds
    # both plain z columns and gated pairs (direct epilogue)
    dict(T=300, d=256, l=128, m=128, n_experts=16, top_k=4, n_shared=1, m_shared=192, alpha=2),
    dict(T=70, d=256, l=128, m=128, n_experts=16, top_k=4, n_shared=1, m_shared=192, alpha=2),
    dict(T=40, d=256, l=128, m=128, n_experts=16, top_k=4, n_shared=1, m_shared=192, alpha=2),
    dict(T=9, d=128, l=64, m=64, n_experts=32, top_k=8, n_shared=0, m_shared=0, alpha=2),
]

# test_backward_shapes (seed = T + 3)
BACKWARD_SHAPES = [
    dict(T=300, d=256, l=128, m=128, n_experts=16, top_k=4, n_shared=1, m_shared=192, alpha=2),
    dict(T=300, d=256, l=128, m=128, n_experts=16, top_k=4, n_shared=1, m_shared=192, alpha=2, expert_act="swiglu"),
    dict(T=40, d=256, l=128, m=128, n_experts=16, top_k=4, n_shared=1, m_shared=192, alpha=2, zipf_s=1.1),
    dict(T=9, d=128, l=64, m=64, n_experts=32, top_k=8, n_shared=0, m_shared=0, alpha=2),
    dict(T=130, d=128, l=64, m=192, n_experts=16, top_k=16, n_shared=2, m_shared=64, alpha=2, variant="eff"),
]


# test_expert_rows_at_tile_boundaries: a zero router, four experts holding T
# rows each (seed = T).  The bf16 forward's 256-row tiles take up to 320 rows
# in an expert's last tile: 255..320 rows are one tile, 321 two (256 + 65),
# 513 two (256 + 257), 577 three (256 + 256 + 65).
TILE_ROWS = [255, 256, 257, 320, 321, 513, 577]


def tile_rows_shape(T):
    return shape(T=T, d=256, l=128, m=192, n_experts=16, top_k=4, n_shared=1, m_shared=128, dtype="bf16")


def edge_workload(cfg, dtype):
    return random_workload(shape(dtype=dtype, **cfg), seed=cfg["T"])


def fp8_workload(cfg):
    return random_fp8_workload(shape(dtype="bf16", expert_dtype="fp8", **cfg), seed=cfg["T"])


def swiglu_workload(cfg, dtype):
    return random_workload(shape(dtype=dtype, expert_act="swiglu", **cfg), seed=cfg["T"] + 1)


def swiglu_fp8_workload(cfg):
    return random_fp8_workload(shape(dtype="bf16", expert_dtype="fp8", expert_act="swiglu", **cfg),
                               seed=cfg["T"] + 2)


def backward_workload(cfg, dtype):
    return random_workload(shape(dtype=dtype, **cfg), seed=cfg["T"] + 3)


def swiglu_tokens_workload(T):
    """test_swiglu_token_counts: the gated workload at T tokens."""
    return make_workload(get_config("shape_swiglu"), T=T)


# The fused expert MLP (bf16 layers with l = 512: 128-row tiles, l = 1024:
# 64-row tiles; at least 32 rows per expert on average).
# test_fused_mlp_rows_at_tile_boundaries: a zero router with K' = N' = 16, so
# every expert holds exactly T rows (seed = T).
FUSED_TILE_ROWS = [(512, 128), (512, 129), (512, 255), (512, 257), (1024, 64), (1024, 65), (1024, 127), (1024, 129)]
# test_fused_mlp_random_routing: scattered rows over many experts (seed = T + 5)
FUSED_SHAPES = [
    dict(T=1024, d=1024, l=512, m=384, n_experts=32, top_k=8, n_shared=1, m_shared=256, alpha=2),
    dict(T=512, d=2048, l=1024, m=256, n_experts=32, top_k=8, n_shared=1, m_shared=256, alpha=2),
    dict(T=700, d=2048, l=512, m=128, n_experts=64, top_k=16, n_shared=0, m_shared=0, alpha=4),
]


def fused_tile_rows_shape(l, T):
    return shape(T=T, d=2 * l, l=l, m=256, n_experts=16, top_k=16, n_shared=1, m_shared=128, alpha=2, dtype="bf16")


def fused_workload(cfg):
    return random_workload(shape(dtype="bf16", **cfg), seed=cfg["T"] + 5)
