"""ctypes front end of the fp64 C oracle (``latentmoe_oracle.c``).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.  It does not import the GPU package.

The layer it evaluates is the LatentMoE forward pass of the explainer page
"LatentMoE: NVIDIA's Latent Mixture of Experts Explained Through Equations,
Architecture, Code and ..." (Figures 3, 6, 8, 9 and its LatentMoE code
block); the C file's header lists each step and the reading taken where the
page is silent.
"""

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import build_oracle

_i64 = C.c_int64
_i32 = C.c_int32
_vp = C.c_void_p


class _Shape(C.Structure):
    _fields_ = [("d", _i64), ("l", _i64), ("m", _i64), ("m_s", _i64),
                ("n_shared", _i64), ("n_experts", _i64), ("top_k", _i64),
                ("bf16", _i32), ("has_bias", _i32), ("expert_fp8", _i32), ("gated", _i32)]


class _Tensors(C.Structure):
    _fields_ = [(n, _vp) for n in ("x", "w_router", "b_router", "w_down", "w1",
                                   "w2", "w_up", "w1_s", "w2_s", "w1_scale", "w2_scale",
                                   "w1g", "w1g_s", "w1g_scale")]


class _Outputs(C.Structure):
    _fields_ = [(n, _vp) for n in ("logits", "idx", "gate", "z", "h", "o", "u",
                                   "hs", "y")]


_lib = None


def lib():
    """The compiled oracle; LATENTMOE_ORACLE_LIB may name another build of the
    same source (the sanitized one)."""
    global _lib
    if _lib is None:
        path = os.environ.get("LATENTMOE_ORACLE_LIB", build_oracle.LIB)
        if not os.path.exists(path):
            if path != build_oracle.LIB:
                raise FileNotFoundError(path)
            build_oracle.build()
        L = C.CDLL(path)
        L.orc_forward.argtypes = [C.POINTER(_Shape), C.POINTER(_Tensors), _i64, _vp,
                                  _i64, _vp, C.POINTER(_Outputs), C.c_int]
        L.orc_forward.restype = C.c_int
        L.orc_select.argtypes = [_vp, _i64, _i64, _i64, _vp]
        L.orc_select.restype = C.c_int
        L.orc_gates.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp]
        L.orc_gates.restype = C.c_int
        L.orc_dispatch.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
        L.orc_dispatch.restype = C.c_int
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = C.c_int
        L.orc_fp8_decode.argtypes = [_vp, _i64, _vp]
        L.orc_fp8_decode.restype = C.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


@dataclass
class OracleResult:
    tokens: np.ndarray
    logits: Optional[np.ndarray] = None
    idx: Optional[np.ndarray] = None
    gate: Optional[np.ndarray] = None
    z: Optional[np.ndarray] = None
    h: Optional[np.ndarray] = None
    o: Optional[np.ndarray] = None
    u: Optional[np.ndarray] = None
    hs: Optional[np.ndarray] = None
    y: Optional[np.ndarray] = None


def _storage(a: np.ndarray, bf16: bool) -> np.ndarray:
    want = np.uint16 if bf16 else np.float32
    if a.dtype != want:
        raise TypeError(f"expected {want} storage, got {a.dtype}")
    return np.ascontiguousarray(a)


def forward(wl, tokens: Optional[Sequence[int]] = None, want=("y",),
            idx_in: Optional[np.ndarray] = None, n_threads: int = 0) -> OracleResult:
    """Evaluate the layer for ``tokens`` (default: all) of workload ``wl``.

    ``want`` names the per-token outputs to return (logits, idx, gate, z, h,
    o, u, hs, y).  ``idx_in`` ([n, K'] int32) forces the routing.
    """
    sh = wl.shape
    bf16 = sh.dtype == "bf16"
    fp8 = sh.expert_dtype == "fp8"
    gated = sh.expert_act == "swiglu"
    T = sh.T
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n = tok.shape[0]
    N, K, l, m, d = sh.n_experts, sh.top_k, sh.l, sh.m, sh.d
    S, ms = sh.n_shared, sh.m_shared
    t = {k: (None if wl.tensors.get(k) is None else _storage(wl.tensors[k], bf16))
         for k in ("x", "w_router", "w_down", "w_up", "w1_s", "w2_s")}
    t["w1g_s"] = _storage(wl.tensors["w1g_s"], bf16) if (gated and S > 0) else None
    for k in (("w1", "w2", "w1g") if gated else ("w1", "w2")):
        if fp8:
            t[k] = np.ascontiguousarray(wl.tensors[k], dtype=np.uint8)
            sc = np.ascontiguousarray(wl.tensors[k + "_scale"], dtype=np.float32)
            assert sc.shape == (N, l if k == "w2" else m)
            t[k + "_scale"] = sc
        else:
            t[k] = _storage(wl.tensors[k], bf16)
            t[k + "_scale"] = None
    b = wl.tensors.get("b_router")
    if b is not None:
        b = np.ascontiguousarray(b, dtype=np.float32)
    shapes = {"logits": (n, N), "idx": (n, K), "gate": (n, K), "z": (n, l),
              "h": (n, K, m), "o": (n, K, l), "u": (n, l), "hs": (n, S * ms), "y": (n, d)}
    res = OracleResult(tokens=tok)
    outs = _Outputs()
    for name in want:
        arr = np.zeros(shapes[name], dtype=np.int32 if name == "idx" else np.float64)
        setattr(res, name, arr)
        setattr(outs, name, arr.ctypes.data)
    cs = _Shape(d, l, m, ms if S > 0 else 0, S, N, K, 1 if bf16 else 0,
                1 if (sh.has_bias and b is not None) else 0, 1 if fp8 else 0, 1 if gated else 0)
    ct = _Tensors(_ptr(t["x"]), _ptr(t["w_router"]), _ptr(b), _ptr(t["w_down"]),
                  _ptr(t["w1"]), _ptr(t["w2"]), _ptr(t["w_up"]),
                  _ptr(t["w1_s"]) if S > 0 else None, _ptr(t["w2_s"]) if S > 0 else None,
                  _ptr(t["w1_scale"]), _ptr(t["w2_scale"]),
                  _ptr(t.get("w1g")), _ptr(t["w1g_s"]), _ptr(t.get("w1g_scale")))
    forced = None
    if idx_in is not None:
        forced = np.ascontiguousarray(idx_in, dtype=np.int32)
        assert forced.shape == (n, K)
    rc = lib().orc_forward(C.byref(cs), C.byref(ct), T, tok.ctypes.data, n,
                           _ptr(forced), C.byref(outs), int(n_threads))
    if rc != 0:
        raise RuntimeError(f"orc_forward failed with {rc}")
    return res


def select(scores: np.ndarray, K: int) -> np.ndarray:
    """Top-K' indices of every row of ``scores`` in (score desc, index asc) order."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    T, N = s.shape
    idx = np.zeros((T, K), dtype=np.int32)
    rc = lib().orc_select(s.ctypes.data, T, N, K, idx.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"orc_select failed with {rc}")
    return idx


def gates(scores: np.ndarray, idx: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(scores, dtype=np.float64)
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    T, N = s.shape
    K = ix.shape[1]
    g = np.zeros((T, K), dtype=np.float64)
    rc = lib().orc_gates(s.ctypes.data, T, N, ix.ctypes.data, K, g.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"orc_gates failed with {rc}")
    return g


@dataclass
class Dispatch:
    counts: np.ndarray
    offsets: np.ndarray
    pos: np.ndarray
    perm: np.ndarray


def dispatch(idx: np.ndarray, N: int) -> Dispatch:
    """Stable counting sort of (token, slot) pairs by expert, then token."""
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    T, K = ix.shape
    counts = np.zeros(N, dtype=np.int32)
    offsets = np.zeros(N + 1, dtype=np.int32)
    pos = np.zeros((T, K), dtype=np.int32)
    perm = np.zeros(T * K, dtype=np.int32)
    rc = lib().orc_dispatch(ix.ctypes.data, T, K, N, counts.ctypes.data,
                            offsets.ctypes.data, pos.ctypes.data, perm.ctypes.data)
    if rc != 0:
        raise ValueError(f"orc_dispatch rejected the indices ({rc})")
    return Dispatch(counts, offsets, pos, perm)


def max_threads() -> int:
    return int(lib().orc_max_threads())


def fp8_decode(q: np.ndarray) -> np.ndarray:
    """The oracle's own E4M3 decode of every byte of ``q`` (float64)."""
    a = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.zeros(a.shape, dtype=np.float64)
    rc = lib().orc_fp8_decode(a.ctypes.data, a.size, out.ctypes.data)
    if rc != 0:
        raise RuntimeError("orc_fp8_decode failed")
    return out


class _Grads(C.Structure):
    _fields_ = [(n, _vp) for n in ("dx", "dw_router", "db_router", "dw_down", "dw1", "dw2", "dw1g",
                                   "dw_up", "dw1_s", "dw2_s", "dw1g_s")]


def backward(wl, dy: np.ndarray, experts: Optional[Sequence[int]] = None, n_threads: int = 0) -> dict:
    """Gradients of a loss L through the layer of workload ``wl`` given
    dy = dL/dy [T, d] (float64), over all T tokens.  Returns dx and every
    weight gradient in float64, in the weights' [in, out] layouts; the
    expert banks' gradients (dw1, dw2, and dw1g when gated) only for
    ``experts`` (default: all), stacked in that order."""
    sh = wl.shape
    if sh.expert_dtype == "fp8":
        raise ValueError("FP8 expert banks are not differentiated")
    bf16 = sh.dtype == "bf16"
    gated = sh.expert_act == "swiglu"
    T, N, K, l, m, d = sh.T, sh.n_experts, sh.top_k, sh.l, sh.m, sh.d
    S, ms = sh.n_shared, sh.m_shared
    ex = np.arange(N, dtype=np.int32) if experts is None else np.asarray(experts, dtype=np.int32)
    t = {k: (None if wl.tensors.get(k) is None else _storage(wl.tensors[k], bf16))
         for k in ("x", "w_router", "w_down", "w1", "w2", "w_up", "w1_s", "w2_s")}
    t["w1g"] = _storage(wl.tensors["w1g"], bf16) if gated else None
    t["w1g_s"] = _storage(wl.tensors["w1g_s"], bf16) if (gated and S > 0) else None
    b = wl.tensors.get("b_router")
    if b is not None:
        b = np.ascontiguousarray(b, dtype=np.float32)
    dyd = np.ascontiguousarray(dy, dtype=np.float64)
    assert dyd.shape == (T, d)
    shapes = {"dx": (T, d), "dw_router": (d, N), "db_router": (N,), "dw_down": (d, l),
              "dw1": (len(ex), l, m), "dw2": (len(ex), m, l), "dw_up": (l, d),
              "dw1_s": (S, d, ms), "dw2_s": (S, ms, d)}
    if gated:
        shapes.update({"dw1g": (len(ex), l, m), "dw1g_s": (S, d, ms)})
    res = {k: np.zeros(v) for k, v in shapes.items()}
    g = _Grads(*[res[k].ctypes.data if k in res else None for k, _ in _Grads._fields_])
    cs = _Shape(d, l, m, ms if S > 0 else 0, S, N, K, 1 if bf16 else 0,
                1 if (sh.has_bias and b is not None) else 0, 0, 1 if gated else 0)
    ct = _Tensors(_ptr(t["x"]), _ptr(t["w_router"]), _ptr(b), _ptr(t["w_down"]), _ptr(t["w1"]), _ptr(t["w2"]),
                  _ptr(t["w_up"]), _ptr(t["w1_s"]) if S > 0 else None, _ptr(t["w2_s"]) if S > 0 else None,
                  None, None, _ptr(t["w1g"]), _ptr(t["w1g_s"]), None)
    L = lib()
    L.orc_backward.argtypes = [C.POINTER(_Shape), C.POINTER(_Tensors), _i64, _vp, _vp, _i64,
                               C.POINTER(_Grads), C.c_int]
    L.orc_backward.restype = C.c_int
    rc = L.orc_backward(C.byref(cs), C.byref(ct), T, dyd.ctypes.data, ex.ctypes.data, len(ex), C.byref(g),
                        int(n_threads))
    if rc != 0:
        raise RuntimeError(f"orc_backward failed with {rc}")
    return res
