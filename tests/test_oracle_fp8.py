"""Pins of the oracle's FP8 expert banks (E4M3 bytes with one float32 scale
per expert and output column; W = decode(q) * scale).

The explainer page ("LatentMoE: NVIDIA's Latent Mixture of Experts Explained
Through Equations, Architecture, Code and ...", byte-count section) prices
expert weights in FP8 and fixes no scale convention; the reading taken is
the per-output-column scale.  The decode follows the OCP 8-bit floating
point definition of E4M3 (bias 7, subnormals at exponent field 0, NaN at
exponent 15 with mantissa 7, no infinities, largest finite value 448).
"""

import math

import numpy as np
import pytest
import torch

from oracle import dense, oracle
from synth.generate import f32_to_bf16_bits, quantize_e4m3_columns
from tests.helpers import random_fp8_workload, shape, workload_from_arrays


# --------------------------------------------------------------------------
# the decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("byte,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x3F, 1.875), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0),
    (0x81, -(2.0 ** -9)), (0xB8, -1.0), (0xFE, -448.0),
])
def test_e4m3_format_values(byte, value):
    assert oracle.fp8_decode(np.array([byte], np.uint8))[0] == value


def test_e4m3_signed_zero_and_nan():
    v = oracle.fp8_decode(np.array([0x00, 0x80, 0x7F, 0xFF], np.uint8))
    assert v[0] == 0.0 and not math.copysign(1.0, v[0]) < 0
    assert v[1] == 0.0 and math.copysign(1.0, v[1]) < 0
    assert np.isnan(v[2]) and np.isnan(v[3])


def test_e4m3_all_bytes_match_torch():
    q = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(q)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


# --------------------------------------------------------------------------
# the forward pass with FP8 banks
# --------------------------------------------------------------------------
def _fp8_shape(**kw):
    base = dict(T=9, d=16, l=8, m=12, n_experts=6, top_k=3, n_shared=1, m_shared=8, dtype="bf16",
                expert_dtype="fp8")
    base.update(kw)
    return shape(**base)


def test_fp8_banks_equal_bf16_banks_of_the_same_values():
    """Power-of-two scales make decode(q) * scale exact in bf16: the FP8 path
    must then give the bf16 path's numbers (which are pinned elsewhere), so
    a scale applied per row, to the wrong expert or not at all would fail."""
    sh = _fp8_shape()
    wl8 = random_fp8_workload(sh, seed=3, pow2_scales=True)
    t = dict(wl8.tensors)
    for k in ("w1", "w2"):
        dec = oracle.fp8_decode(t[k]) * t.pop(k + "_scale").astype(np.float64)[:, None, :]
        bits = f32_to_bf16_bits(dec.astype(np.float32))
        assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64), dec)
        t[k] = bits
    import dataclasses
    sh16 = dataclasses.replace(sh, expert_dtype=None)
    wl16 = type(wl8)(sh16, t)
    want = ("logits", "idx", "gate", "z", "h", "o", "u", "y")
    a = oracle.forward(wl8, want=want)
    b = oracle.forward(wl16, want=want)
    for k in want:
        assert np.array_equal(getattr(a, k), getattr(b, k)), k


@pytest.mark.parametrize("kw", [dict(), dict(top_k=6, n_shared=0, m_shared=0), dict(dtype="bf16", zipf_s=1.1)])
def test_fp8_oracle_matches_dense_bruteforce(kw):
    sh = _fp8_shape(**kw)
    wl = random_fp8_workload(sh, seed=11)
    r = oracle.forward(wl, want=("logits", "idx", "gate", "z", "u", "y"))
    d = dense.layer_dense_from_workload(wl)
    assert np.array_equal(r.idx, dense.select_lexsort(d["logits"], sh.top_k))
    for k in ("z", "u", "y"):
        ref = d[k]
        assert np.max(np.abs(getattr(r, k) - ref)) <= 1e-12 * np.max(np.abs(ref)), k


def test_fp8_oracle_rejects_missing_scales():
    sh = _fp8_shape()
    wl = random_fp8_workload(sh, seed=1)
    del wl.tensors["w1_scale"]
    with pytest.raises(Exception):
        oracle.forward(wl)


# --------------------------------------------------------------------------
# the input recipe's quantizer (inputs, not the layer)
# --------------------------------------------------------------------------
def test_quantizer_maps_column_maximum_to_448_and_rounds_to_nearest():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((64, 24)).astype(np.float32)
    w[:, 5] = 0.0
    q, sc = quantize_e4m3_columns(w)
    dec = oracle.fp8_decode(q)
    assert sc[5] == 1.0 and np.all(dec[:, 5] == 0.0)
    cols = [j for j in range(24) if j != 5]
    assert np.all(np.max(np.abs(dec[:, cols]), axis=0) == 448.0)
    # nearest: relative error of a normal E4M3 value is at most 2^-4
    r = w / sc[None, :]
    big = np.abs(r) >= 2.0 ** -6
    assert np.all(np.abs(dec[big] - r[big]) <= np.abs(r[big]) * 2.0 ** -4 + 1e-12)
