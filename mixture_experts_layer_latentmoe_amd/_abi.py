"""ctypes binding of the C ABI in include/latentmoe.h (same names, same
arguments; marshalling only).  Every step of the layer runs in the HIP
library; importing this module never falls back to anything else: if the
library is missing, loading it raises."""

import ctypes as C
import os

from . import build as _build

_i64, _i32, _vp = C.c_int64, C.c_int32, C.c_void_p

LATENTMOE_OK = 0
LATENTMOE_ERR_INVALID_ARGUMENT = 1
LATENTMOE_ERR_UNSUPPORTED = 2
LATENTMOE_ERR_OUT_OF_MEMORY = 3
LATENTMOE_ERR_HIP = 4
LATENTMOE_ERR_EXCEEDS_SCRATCH = 5
LATENTMOE_NOALLOC_SCRATCH_BYTES = 64 << 20
LATENTMOE_VARIANT_ACC, LATENTMOE_VARIANT_EFF = 0, 1
LATENTMOE_DTYPE_F32, LATENTMOE_DTYPE_BF16 = 0, 1
LATENTMOE_EXPERT_AS_DTYPE, LATENTMOE_EXPERT_FP8_E4M3 = 0, 1
LATENTMOE_ACT_RELU2, LATENTMOE_ACT_SWIGLU = 0, 1
LATENTMOE_MAX_STAGES = 16

EXPORTED = ("latentmoe_create", "latentmoe_forward", "latentmoe_forward_noalloc", "latentmoe_backward",
            "latentmoe_destroy",
            "latentmoe_validate_config",
            "latentmoe_workspace_bytes", "latentmoe_cost", "latentmoe_status_string",
            "latentmoe_last_hip_error", "latentmoe_profile_begin", "latentmoe_profile_end",
            "latentmoe_stage_name")


class latentmoe_config(C.Structure):
    _fields_ = [("d", _i64), ("l", _i64), ("m", _i64), ("m_shared", _i64), ("n_shared", _i64),
                ("n_experts", _i64), ("top_k", _i64), ("alpha", _i64), ("variant", _i32),
                ("dtype", _i32), ("max_tokens", _i64), ("has_router_bias", _i32), ("expert_format", _i32),
                ("expert_act", _i32)]


class latentmoe_weights(C.Structure):
    _fields_ = [(n, _vp) for n in ("w_router", "b_router", "w_down", "w1", "w2", "w_up",
                                   "w1_shared", "w2_shared", "w1_scale", "w2_scale",
                                   "w1_gate", "w1_shared_gate", "w1_gate_scale")]


class latentmoe_debug(C.Structure):
    _fields_ = [(n, _vp) for n in ("logits", "idx", "gate", "counts", "offsets", "perm_token",
                                   "pos", "z", "h_shared", "h", "y_perm", "u")]


class latentmoe_grads(C.Structure):
    _fields_ = [(n, _vp) for n in ("dx", "dw_router", "db_router", "dw_down", "dw1", "dw2", "dw_up",
                                   "dw1_shared", "dw2_shared", "dw1_gate", "dw1_shared_gate")]


_COST_FIELDS = ("latent_expert_params", "routed_pool_params", "projection_params", "router_params",
                "shared_params", "layer_params_excl_router", "active_params_per_token",
                "expert_bytes_per_token_fp8", "expert_bytes_per_token_bf16", "a2a_bytes_per_token",
                "flops_per_token", "log10_combinations", "baseline_n_experts", "baseline_top_k",
                "baseline_expert_params", "baseline_layer_params_excl_router",
                "baseline_active_params_per_token", "baseline_a2a_bytes_per_token",
                "baseline_log10_combinations", "log10_combination_bound")


class latentmoe_cost_out(C.Structure):
    _fields_ = [(n, C.c_double) for n in _COST_FIELDS]


class LatentMoEError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = status_string(status)
        if status == LATENTMOE_ERR_HIP:
            msg += f" (hipError {lib().latentmoe_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")


_lib = None


def lib_path() -> str:
    return _build.LIB


def lib():
    """Load liblatentmoe.so (built in-tree by build()); raise if absent."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run __graft_entry__.build() or "
                              "python -m mixture_experts_layer_latentmoe_amd.build")
        L = C.CDLL(path)
        P = C.POINTER
        L.latentmoe_create.argtypes = [P(latentmoe_config), P(latentmoe_weights), _vp, P(_vp)]
        L.latentmoe_forward.argtypes = [_vp, _vp, _vp, _i64, _vp, P(latentmoe_debug)]
        L.latentmoe_forward_noalloc.argtypes = [_vp, _vp, _vp, _i64, _vp]
        L.latentmoe_backward.argtypes = [_vp, _vp, _vp, _i64, _vp, P(latentmoe_grads)]
        L.latentmoe_destroy.argtypes = [_vp]
        L.latentmoe_validate_config.argtypes = [P(latentmoe_config)]
        L.latentmoe_workspace_bytes.argtypes = [P(latentmoe_config), P(_i64)]
        L.latentmoe_cost.argtypes = [P(latentmoe_config), P(latentmoe_cost_out)]
        L.latentmoe_status_string.argtypes = [C.c_int]
        L.latentmoe_status_string.restype = C.c_char_p
        L.latentmoe_last_hip_error.argtypes = []
        L.latentmoe_profile_begin.argtypes = [_vp, C.c_int, C.c_uint32]
        L.latentmoe_profile_end.argtypes = [_vp, P(C.c_double), P(_i32), P(_i32)]
        L.latentmoe_stage_name.argtypes = [C.c_int]
        L.latentmoe_stage_name.restype = C.c_char_p
        for n in EXPORTED:
            if n not in ("latentmoe_status_string", "latentmoe_stage_name"):
                getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().latentmoe_status_string(int(status)).decode()


def _check(fn, st):
    if st != LATENTMOE_OK:
        raise LatentMoEError(fn, st)


def make_config(d, l, m, n_experts, top_k, alpha, n_shared=0, m_shared=0, variant="acc",
                dtype="bf16", max_tokens=1, has_router_bias=False, expert_dtype=None,
                expert_act="relu2") -> latentmoe_config:
    return latentmoe_config(d, l, m, m_shared, n_shared, n_experts, top_k, alpha,
                            LATENTMOE_VARIANT_ACC if variant == "acc" else LATENTMOE_VARIANT_EFF,
                            LATENTMOE_DTYPE_BF16 if dtype == "bf16" else LATENTMOE_DTYPE_F32,
                            max_tokens, 1 if has_router_bias else 0,
                            LATENTMOE_EXPERT_FP8_E4M3 if expert_dtype == "fp8" else LATENTMOE_EXPERT_AS_DTYPE,
                            LATENTMOE_ACT_SWIGLU if expert_act == "swiglu" else LATENTMOE_ACT_RELU2)


def latentmoe_validate_config(cfg: latentmoe_config) -> int:
    return lib().latentmoe_validate_config(C.byref(cfg))


def latentmoe_workspace_bytes(cfg: latentmoe_config) -> int:
    out = _i64(0)
    _check("latentmoe_workspace_bytes", lib().latentmoe_workspace_bytes(C.byref(cfg), C.byref(out)))
    return out.value


def latentmoe_cost(cfg: latentmoe_config) -> dict:
    out = latentmoe_cost_out()
    _check("latentmoe_cost", lib().latentmoe_cost(C.byref(cfg), C.byref(out)))
    return {n: getattr(out, n) for n in _COST_FIELDS}


def latentmoe_create(cfg: latentmoe_config, weights: latentmoe_weights, stream: int) -> int:
    h = _vp(0)
    _check("latentmoe_create", lib().latentmoe_create(C.byref(cfg), C.byref(weights), _vp(stream), C.byref(h)))
    return h.value


def latentmoe_forward(handle: int, x_ptr: int, y_ptr: int, T: int, stream: int,
                      dbg: latentmoe_debug = None) -> None:
    _check("latentmoe_forward", lib().latentmoe_forward(_vp(handle), _vp(x_ptr), _vp(y_ptr), int(T),
                                                        _vp(stream), C.byref(dbg) if dbg is not None else None))


def latentmoe_forward_noalloc(handle: int, x_ptr: int, y_ptr: int, T: int, stream: int) -> None:
    _check("latentmoe_forward_noalloc",
           lib().latentmoe_forward_noalloc(_vp(handle), _vp(x_ptr), _vp(y_ptr), int(T), _vp(stream)))


def latentmoe_backward(handle: int, x_ptr: int, dy_ptr: int, T: int, stream: int, grads: latentmoe_grads) -> None:
    _check("latentmoe_backward", lib().latentmoe_backward(_vp(handle), _vp(x_ptr), _vp(dy_ptr), int(T),
                                                          _vp(stream), C.byref(grads)))


def latentmoe_destroy(handle: int) -> None:
    _check("latentmoe_destroy", lib().latentmoe_destroy(_vp(handle)))


ALL_STAGES = 0xFFFF


def latentmoe_profile_begin(handle: int, max_forwards: int, stage_mask: int = ALL_STAGES) -> None:
    _check("latentmoe_profile_begin",
           lib().latentmoe_profile_begin(_vp(handle), int(max_forwards), int(stage_mask) & 0xFFFFFFFF))


def latentmoe_profile_end(handle: int) -> dict:
    ms = (C.c_double * LATENTMOE_MAX_STAGES)()
    n = (_i32 * LATENTMOE_MAX_STAGES)()
    ns = _i32(0)
    _check("latentmoe_profile_end", lib().latentmoe_profile_end(_vp(handle), ms, n, C.byref(ns)))
    return {latentmoe_stage_name(i): (ms[i], n[i]) for i in range(ns.value)}


def latentmoe_stage_name(i: int) -> str:
    return lib().latentmoe_stage_name(int(i)).decode()
