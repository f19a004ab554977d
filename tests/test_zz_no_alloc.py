"""latentmoe_forward_noalloc (through the C ABI) against latentmoe_forward on
the same handle and input: the forward with its workspace in the library's
static scratch array instead of the handle's allocation.

Two calls in a row, the second with fewer tokens, so the second runs on what
the first left in the array.  Each is compared with latentmoe_forward's
output: bit for bit where both take the same kernels with the same split-K
partition (always for T <= 64 and T > 256), else to the contract bar.  Also:
a token count whose workspace exceeds the array is refused with
LATENTMOE_ERR_EXCEEDS_SCRATCH before any GPU work, and the array is the
same memory on every handle (one handle's calls leave nothing behind that
breaks the next handle's).
"""

import ctypes

import numpy as np
import pytest
import torch

from mixture_experts_layer_latentmoe_amd import _abi
from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
from synth import get_config, make_workload
from tests import gpu_util as G
from tests import tolerances as TOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


def _both(layer, x):
    s = torch.cuda.current_stream().cuda_stream
    y_ref = torch.empty_like(x)
    _abi.latentmoe_forward(layer.handle, x.data_ptr(), y_ref.data_ptr(), x.shape[0], s)
    y = torch.full_like(x, float("nan"))
    _abi.latentmoe_forward_noalloc(layer.handle, x.data_ptr(), y.data_ptr(), x.shape[0], s)
    torch.cuda.synchronize()
    return G.to_np(y), G.to_np(y_ref)


@pytest.mark.parametrize("name,Ts", [("readme_acc", (300, 40)), ("readme_acc", (200, 7)),
                                     ("tiny_f32", (256, 17)), ("decode_eff_fp8", (64, 5)),
                                     ("shape_swiglu", (130, 64))])
def test_noalloc_matches_forward_two_calls(name, Ts):
    wl = make_workload(get_config(name), T=Ts[0])
    layer = LatentMoE.from_workload(wl, max_tokens=Ts[0])
    try:
        for T in Ts:
            G.say(f"[gpu] noalloc {name} T={T}")
            x = to_device(np.ascontiguousarray(wl.tensors["x"][:T]), wl.shape.dtype, "cuda:0")
            y, y_ref = _both(layer, x)
            assert np.all(np.isfinite(y))
            if T <= 64 or T > 256:
                assert np.array_equal(y, y_ref), T
            else:
                err = TOL.y_err(y, y_ref.astype(np.float64), wl.shape.dtype)
                assert err <= TOL.y_bar(wl.shape), err
    finally:
        layer.close()


def test_noalloc_rejects_too_many_tokens():
    wl = make_workload(get_config("readme_acc"), T=4096)
    layer = LatentMoE.from_workload(wl)
    try:
        x = to_device(wl.tensors["x"], "bf16", "cuda:0")
        y = torch.empty_like(x)
        L = _abi.lib()
        st = L.latentmoe_forward_noalloc(ctypes.c_void_p(layer.handle), ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(y.data_ptr()), 4096, None)
        assert st == _abi.LATENTMOE_ERR_EXCEEDS_SCRATCH
        assert L.latentmoe_forward_noalloc(ctypes.c_void_p(layer.handle), ctypes.c_void_p(x.data_ptr()),
                                           ctypes.c_void_p(x.data_ptr()), 64, None) == \
            _abi.LATENTMOE_ERR_INVALID_ARGUMENT
        # a size that fits still runs on the same handle afterwards
        y2, y2_ref = _both(layer, x[:64].contiguous())
        assert np.array_equal(y2, y2_ref)
    finally:
        layer.close()


def test_noalloc_two_handles_share_the_array():
    a_wl = make_workload(get_config("decode_eff"))
    b_wl = make_workload(get_config("tiny_f32"), T=64)
    a = LatentMoE.from_workload(a_wl)
    b = LatentMoE.from_workload(b_wl)
    try:
        xa = to_device(a_wl.tensors["x"], "bf16", "cuda:0")
        xb = to_device(b_wl.tensors["x"], "f32", "cuda:0")
        for _ in range(2):
            ya, ya_ref = _both(a, xa)
            yb, yb_ref = _both(b, xb)
            assert np.array_equal(ya, ya_ref) and np.array_equal(yb, yb_ref)
    finally:
        a.close()
        b.close()
