"""Seeded generation of LatentMoE layer inputs.

Recipe (one numpy ``SeedSequence(seed).spawn(11)`` child per tensor, in the
fixed order x, W_r, b, W_down, W1, W2, W_up, W1_s, W2_s, W_g, W_g_s; the
first nine children do not depend on how many are spawned):

  * x ~ N(0, 1), shape [T, d]
  * every weight ~ N(0, 1/fan_in) with fan_in its input width:
      W_r [d, N'], W_down [d, l], W1_s [S, d, m_s]  -> fan_in d
      W1  [N', l, m], W_up [l, d]                    -> fan_in l
      W2  [N', m, l]                                 -> fan_in m
      W2_s [S, m_s, d]                               -> fan_in m_s
      gated experts only: W_g [N', l, m] -> fan_in l, W_g_s [S, d, m_s] -> fan_in d
    Weights are stored [in, out] row-major, so row i of a matrix holds the
    weights leaving input coordinate i.
  * optional router bias b_e = 2 ln( (e+1)^-s / H_{N', s} )  (Zipf law of
    exponent s over expert ranks 1..N'); its seed child is left unused.

All draws are float32.  For bf16 workloads each tensor is rounded to bf16
(round to nearest, ties to even) once; the rounded values are canonical.
Large expert banks are drawn one expert at a time, in expert order, from the
same generator.

FP8 expert banks (``expert_dtype="fp8"``): each expert's W1 and W2 float32
draw is quantized per output column j: scale_j = max_i |W[i, j]| / 448 (the
largest finite E4M3 value) and q[i, j] = E4M3(W[i, j] / scale_j), rounded to
nearest even by torch's float8_e4m3fn conversion.  The bytes q and the
float32 scales are the canonical inputs; the other tensors stay bf16.  A
gated bank's W_g is quantized the same way.
"""

from dataclasses import dataclass, field
from functools import lru_cache
from typing import Dict, Optional

import numpy as np

from .configs import LayerShape

_ORDER = ("x", "w_router", "b_router", "w_down", "w1", "w2", "w_up", "w1_s", "w2_s", "w1g", "w1g_s")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


@dataclass
class Workload:
    """Canonical inputs of one layer invocation.

    ``tensors`` maps a name from ``_ORDER`` to a numpy array.  For bf16
    workloads the arrays are uint16 bf16 bit patterns, for f32 workloads
    float32 arrays.  ``b_router`` is always float32 (or absent).
    """

    shape: LayerShape
    tensors: Dict[str, np.ndarray] = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.shape.dtype

    def f32(self, name: str) -> np.ndarray:
        """The tensor as float32 (exact widening for bf16)."""
        a = self.tensors[name]
        if a is None:
            return None
        if a.dtype == np.uint8:
            raise TypeError(f"{name} holds FP8 bytes; their values need the per-column scales")
        if a.dtype == np.uint16:
            return bf16_bits_to_f32(a)
        return a

    def f64(self, name: str) -> np.ndarray:
        a = self.f32(name)
        return None if a is None else a.astype(np.float64)

    def with_x(self, x: np.ndarray) -> "Workload":
        t = dict(self.tensors)
        t["x"] = x
        return Workload(self.shape.with_tokens(x.shape[0]), t)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def _normal(rng, shape, fan_in) -> np.ndarray:
    scale = np.float32(1.0 / np.sqrt(float(fan_in)))
    return rng.standard_normal(shape, dtype=np.float32) * scale


def _bank(rng, n, shape, fan_in, dtype) -> np.ndarray:
    """Draw n matrices of ``shape`` one after another (expert order)."""
    out = np.empty((n,) + tuple(shape), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for e in range(n):
        out[e] = _store(_normal(rng, shape, fan_in), dtype)
    return out


def quantize_e4m3_columns(w: np.ndarray):
    """w [in, out] float32 -> (q uint8 [in, out], scale float32 [out]):
    scale_j = max_i |w[i, j]| / 448 (1 for an all-zero column) and
    q = E4M3(w / scale), nearest-even, by torch's float8_e4m3fn conversion."""
    import torch
    w = np.ascontiguousarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=0)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = torch.from_numpy(w / scale[None, :]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(q), scale


def _bank_fp8(rng, n, shape, fan_in):
    """Like _bank, each expert quantized per output column (see the header)."""
    q = np.empty((n,) + tuple(shape), dtype=np.uint8)
    sc = np.empty((n, shape[1]), dtype=np.float32)
    for e in range(n):
        q[e], sc[e] = quantize_e4m3_columns(_normal(rng, shape, fan_in))
    return q, sc


def zipf_router_bias(n_experts: int, s: float) -> np.ndarray:
    r = np.arange(1, n_experts + 1, dtype=np.float64)
    w = r ** (-s)
    w /= w.sum()
    return (2.0 * np.log(w)).astype(np.float32)


def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(len(_ORDER))


@lru_cache(maxsize=4)
def _weights(shape_key: tuple) -> Dict[str, np.ndarray]:
    (d, l, m, n_e, S, m_s, dtype, seed, zipf_s, expert_dtype, expert_act) = shape_key
    ch = _children(seed)
    g = {name: np.random.default_rng(c) for name, c in zip(_ORDER, ch)}
    w = {}
    w["w_router"] = _store(_normal(g["w_router"], (d, n_e), d), dtype)
    w["b_router"] = None if zipf_s is None else zipf_router_bias(n_e, zipf_s)
    w["w_down"] = _store(_normal(g["w_down"], (d, l), d), dtype)
    if expert_dtype == "fp8":
        w["w1"], w["w1_scale"] = _bank_fp8(g["w1"], n_e, (l, m), l)
        w["w2"], w["w2_scale"] = _bank_fp8(g["w2"], n_e, (m, l), m)
    else:
        w["w1"] = _bank(g["w1"], n_e, (l, m), l, dtype)
        w["w2"] = _bank(g["w2"], n_e, (m, l), m, dtype)
    w["w_up"] = _store(_normal(g["w_up"], (l, d), l), dtype)
    w["w1_s"] = _bank(g["w1_s"], S, (d, m_s), d, dtype)
    w["w2_s"] = _bank(g["w2_s"], S, (m_s, d), m_s, dtype)
    if expert_act == "swiglu":
        if expert_dtype == "fp8":
            w["w1g"], w["w1g_scale"] = _bank_fp8(g["w1g"], n_e, (l, m), l)
        else:
            w["w1g"] = _bank(g["w1g"], n_e, (l, m), l, dtype)
        w["w1g_s"] = _bank(g["w1g_s"], S, (d, m_s), d, dtype)
    for a in w.values():
        if a is not None:
            a.setflags(write=False)
    return w


def make_x(shape: LayerShape, T: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    T = shape.T if T is None else T
    s = seed if seed is not None else (shape.x_seed if shape.x_seed is not None else shape.seed)
    rng = np.random.default_rng(_children(s)[0])
    return _store(rng.standard_normal((T, shape.d), dtype=np.float32), shape.dtype)


def make_workload(shape: LayerShape, T: Optional[int] = None,
                  x_seed: Optional[int] = None) -> Workload:
    """Weights from ``shape.seed``; x from ``x_seed`` (default: the shape's)."""
    key = (shape.d, shape.l, shape.m, shape.n_experts, shape.n_shared,
           shape.m_shared, shape.dtype, shape.seed, shape.zipf_s, shape.expert_dtype, shape.expert_act)
    w = _weights(key)
    x = make_x(shape, T, x_seed)
    t = dict(w)
    t["x"] = x
    return Workload(shape.with_tokens(x.shape[0]), t)
