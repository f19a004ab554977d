"""The seeded input generator: determinism, shapes, and bf16 rounding
checked against torch's own float32 -> bfloat16 conversion (nearest-even)."""

import numpy as np
import torch

from synth import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_workload
from synth.generate import make_x, zipf_router_bias


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        # exact halfway cases between two bf16 values
                        ((np.arange(1, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)])
    ours = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_shaped():
    sh = get_config("tiny_f32")
    a = make_workload(sh)
    b = make_workload(sh)
    for k, v in a.tensors.items():
        if v is not None:
            assert np.array_equal(v, b.tensors[k])
    t = a.tensors
    assert t["x"].shape == (256, 256) and t["w_router"].shape == (256, 16)
    assert t["w1"].shape == (16, 128, 256) and t["w2"].shape == (16, 256, 128)
    assert t["w1_s"].shape == (1, 256, 256) and t["w2_s"].shape == (1, 256, 256)
    assert t["b_router"] is None


def test_x_prefix_is_stable_across_token_counts():
    sh = get_config("tiny_f32")
    assert np.array_equal(make_x(sh, 17), make_x(sh, 256)[:17])


def test_decode_shares_readme_weights():
    a, b = get_config("readme_acc"), get_config("decode_eff")
    assert (a.d, a.l, a.m, a.n_experts, a.seed) == (b.d, b.l, b.m, b.n_experts, b.seed)
    assert b.x_seed != a.seed and b.top_k == 6 and b.T == 64


def test_zipf_bias_ranks_and_normalisation():
    b = zipf_router_bias(512, 1.1).astype(np.float64)
    assert np.all(np.diff(b) < 0)
    w = np.exp(b / 2.0)
    assert abs(w.sum() - 1.0) < 1e-5
    assert abs((b[0] - b[1]) / 2.0 - 1.1 * np.log(2.0)) < 1e-5


def test_config_shapes_are_consistent():
    for sh in CONFIGS.values():
        assert sh.l * sh.alpha == sh.d
        assert sh.n_experts % sh.alpha == 0
        if sh.variant == "acc":
            assert sh.top_k % sh.alpha == 0
