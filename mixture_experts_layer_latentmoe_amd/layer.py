"""Torch-facing wrapper around the C ABI: moves host arrays into device
memory, passes pointers and the current HIP stream, and allocates outputs.
No layer arithmetic happens here."""

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import _abi

_TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """float32 array, or uint16 array of bf16 bits, -> device tensor."""
    a = np.ascontiguousarray(a)
    if not a.flags.writeable:  # torch wants writable memory; the copy is on the host only
        a = a.copy()
    if a.dtype == np.uint16:
        assert dtype == "bf16"
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "bf16":
        raise TypeError("bf16 tensors are passed as uint16 bit patterns")
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass
class Shape:
    d: int
    l: int
    m: int
    n_experts: int
    top_k: int
    alpha: int
    n_shared: int
    m_shared: int
    variant: str
    dtype: str
    has_bias: bool
    expert_dtype: Optional[str] = None  # "fp8": W1/W2 are E4M3 bytes with column scales
    expert_act: str = "relu2"           # "swiglu": gated experts, gate banks w1g / w1g_s


class LatentMoE:
    """One configured layer on one device.

    ``arrays``: x is not needed; w_router [d,N'], b_router [N'] (fp32, or
    None), w_down [d,l], w1 [N',l,m], w2 [N',m,l], w_up [l,d],
    w1_s [S,d,m_s], w2_s [S,m_s,d] as float32 or bf16-bit uint16 arrays;
    with ``expert_dtype == "fp8"`` w1/w2 are uint8 E4M3 bytes and
    w1_scale [N',m], w2_scale [N',l] their float32 column scales.  With
    ``expert_act == "swiglu"`` the gate banks w1g [N',l,m] (like w1, with
    w1g_scale in an FP8 bank) and w1g_s [S,d,m_s] come too.
    """

    def __init__(self, shape: Shape, arrays: Dict[str, np.ndarray], max_tokens: int, device="cuda:0"):
        self.shape = shape
        self.device = torch.device(device)
        self.max_tokens = int(max_tokens)
        self.tdtype = _TORCH[shape.dtype]
        self.cfg = _abi.make_config(shape.d, shape.l, shape.m, shape.n_experts, shape.top_k, shape.alpha,
                                    shape.n_shared, shape.m_shared, shape.variant, shape.dtype,
                                    self.max_tokens, shape.has_bias, shape.expert_dtype, shape.expert_act)
        fp8 = shape.expert_dtype == "fp8"
        gated = shape.expert_act == "swiglu"
        dev = {"w1g": None, "w1g_s": None}
        names = ["w_router", "w_down", "w1", "w2", "w_up", "w1_s", "w2_s"] + (["w1g", "w1g_s"] if gated else [])
        for k in names:
            if k in ("w1_s", "w2_s", "w1g_s") and shape.n_shared == 0:
                dev[k] = None
                continue
            if fp8 and k in ("w1", "w2", "w1g"):
                dev[k] = torch.from_numpy(np.ascontiguousarray(arrays[k], dtype=np.uint8).copy()).to(self.device)
                continue
            dev[k] = to_device(arrays[k], shape.dtype, self.device)
        for k in ("w1_scale", "w2_scale", "w1g_scale"):
            dev[k] = (torch.from_numpy(np.ascontiguousarray(arrays[k], dtype=np.float32).copy()).to(self.device)
                      if fp8 and (gated or k != "w1g_scale") else None)
        b = arrays.get("b_router")
        dev["b_router"] = (torch.from_numpy(np.array(b, np.float32)).to(self.device)
                           if (shape.has_bias and b is not None) else None)

        def ptr(t):
            return None if t is None else t.data_ptr()

        w = _abi.latentmoe_weights(ptr(dev["w_router"]), ptr(dev["b_router"]), ptr(dev["w_down"]),
                                   ptr(dev["w1"]), ptr(dev["w2"]), ptr(dev["w_up"]), ptr(dev["w1_s"]),
                                   ptr(dev["w2_s"]), ptr(dev["w1_scale"]), ptr(dev["w2_scale"]),
                                   ptr(dev["w1g"]), ptr(dev["w1g_s"]), ptr(dev["w1g_scale"]))
        with torch.cuda.device(self.device):
            self.handle = _abi.latentmoe_create(self.cfg, w, _stream_ptr(self.device))
        del dev  # create copied the weights

    @classmethod
    def from_workload(cls, wl, max_tokens: Optional[int] = None, device="cuda:0") -> "LatentMoE":
        sh = wl.shape
        s = Shape(sh.d, sh.l, sh.m, sh.n_experts, sh.top_k, sh.alpha, sh.n_shared, sh.m_shared,
                  sh.variant, sh.dtype, sh.has_bias, sh.expert_dtype, sh.expert_act)
        return cls(s, wl.tensors, max_tokens or sh.T, device)

    def close(self):
        if getattr(self, "handle", None):
            _abi.latentmoe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                dbg: Optional[_abi.latentmoe_debug] = None) -> torch.Tensor:
        assert x.is_contiguous() and x.dtype == self.tdtype and x.device == self.device
        T = x.shape[0]
        assert x.shape == (T, self.shape.d)
        if y is None:
            y = torch.empty_like(x)
        _abi.latentmoe_forward(self.handle, x.data_ptr(), y.data_ptr(), T, _stream_ptr(self.device), dbg)
        return y

    def forward_debug(self, x: torch.Tensor, want=("logits", "idx", "gate", "counts", "offsets",
                                                   "perm_token", "pos", "z", "h_shared", "h", "y_perm",
                                                   "u")):
        """Forward that also returns the intermediate results (device tensors)."""
        s = self.shape
        T = x.shape[0]
        P = T * s.top_k
        i32, f32, E = torch.int32, torch.float32, self.tdtype
        shapes = {"logits": ((T, s.n_experts), f32), "idx": ((T, s.top_k), i32), "gate": ((T, s.top_k), f32),
                  "counts": ((s.n_experts,), i32), "offsets": ((s.n_experts + 1,), i32),
                  "perm_token": ((P,), i32), "pos": ((T, s.top_k), i32), "z": ((T, s.l), E),
                  "h_shared": ((T, s.n_shared * s.m_shared), E), "h": ((P, s.m), E),
                  "y_perm": ((P, s.l), E), "u": ((T, s.l), E)}
        out = {k: torch.empty(*shapes[k][0], dtype=shapes[k][1], device=self.device) for k in want}
        dbg = _abi.latentmoe_debug(*[(out[k].data_ptr() if k in out else None)
                                     for k, _ in _abi.latentmoe_debug._fields_])
        out["y"] = self.forward(x, dbg=dbg)
        return out

    def backward(self, x: torch.Tensor, dy: torch.Tensor, want=None):
        """dx and the weight gradients (fp32, the weights' [in, out] layouts)
        for dy = dL/dy, as device tensors; ``want`` names a subset."""
        s = self.shape
        T = x.shape[0]
        assert x.is_contiguous() and dy.is_contiguous() and dy.shape == x.shape
        f32, E = torch.float32, self.tdtype
        S, ms = s.n_shared, s.m_shared
        shapes = {"dx": ((T, s.d), E), "dw_router": ((s.d, s.n_experts), f32), "dw_down": ((s.d, s.l), f32),
                  "dw1": ((s.n_experts, s.l, s.m), f32), "dw2": ((s.n_experts, s.m, s.l), f32),
                  "dw_up": ((s.l, s.d), f32)}
        if S > 0:
            shapes.update({"dw1_shared": ((S, s.d, ms), f32), "dw2_shared": ((S, ms, s.d), f32)})
        if s.has_bias:
            shapes["db_router"] = ((s.n_experts,), f32)
        if s.expert_act == "swiglu":
            shapes["dw1_gate"] = ((s.n_experts, s.l, s.m), f32)
            if S > 0:
                shapes["dw1_shared_gate"] = ((S, s.d, ms), f32)
        keys = list(shapes) if want is None else [k for k in want if k in shapes]
        out = {k: torch.empty(*shapes[k][0], dtype=shapes[k][1], device=self.device) for k in keys}
        g = _abi.latentmoe_grads(*[(out[k].data_ptr() if k in out else None)
                                   for k, _ in _abi.latentmoe_grads._fields_])
        _abi.latentmoe_backward(self.handle, x.data_ptr(), dy.data_ptr(), T, _stream_ptr(self.device), g)
        return out
