"""Device allocation failures reach the callers as LATENTMOE_ERR_OUT_OF_MEMORY
and leave nothing broken behind (the library's LATENTMOE_FAIL_ALLOC_AT test
hook makes the n-th device allocation of the process fail).

The hook counts allocations per process, so the scenario runs in a fresh
child process, in order:
  * create fails at its first allocation (the weight copy), then at its
    second (the workspace): both return OUT_OF_MEMORY and no handle;
  * create succeeds and the forward runs;
  * the first backward call fails at its weight layouts, then (a second
    call) at its workspace: OUT_OF_MEMORY each time, and the handle's forward
    still gives the same bits;
  * with the hook off, the backward runs and the forward is unchanged.
"""

import os
import subprocess
import sys
import textwrap

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = textwrap.dedent("""
    import os, ctypes
    import numpy as np, torch
    from mixture_experts_layer_latentmoe_amd import _abi
    from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
    from synth import get_config, make_workload
    wl = make_workload(get_config("tiny_f32"), T=32)
    def fail_at(n):
        if n:
            os.environ["LATENTMOE_FAIL_ALLOC_AT"] = str(n)
        else:
            os.environ.pop("LATENTMOE_FAIL_ALLOC_AT", None)
    for n in (1, 3):  # allocations 1: weights of the first create; 2, 3: weights, workspace of the second
        fail_at(n)
        try:
            LatentMoE.from_workload(wl)
            raise SystemExit(f"create did not fail at allocation {n}")
        except _abi.LatentMoEError as e:
            assert e.status == _abi.LATENTMOE_ERR_OUT_OF_MEMORY, e
        print("create failed at allocation", n, flush=True)
    fail_at(0)
    layer = LatentMoE.from_workload(wl)   # allocations 4, 5
    x = to_device(wl.tensors["x"], "f32", "cuda:0")
    y0 = layer.forward(x).cpu().numpy()
    dy = torch.ones_like(x)
    for n in (6, 8):  # the backward's weight layouts (6), then its workspace (8, after 7 succeeded)
        fail_at(n)
        try:
            layer.backward(x, dy)
            raise SystemExit(f"backward did not fail at allocation {n}")
        except _abi.LatentMoEError as e:
            assert e.status == _abi.LATENTMOE_ERR_OUT_OF_MEMORY, e
        assert np.array_equal(layer.forward(x).cpu().numpy(), y0)
        print("backward failed at allocation", n, flush=True)
    fail_at(0)
    g = layer.backward(x, dy)
    torch.cuda.synchronize()
    assert all(np.all(np.isfinite(v.cpu().numpy())) for v in g.values())
    assert np.array_equal(layer.forward(x).cpu().numpy(), y0)
    layer.close()
    print("ALLOC_HOOK_OK", flush=True)
""")


def test_allocation_failures_are_reported_and_recovered():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ)
    env.pop("LATENTMOE_FAIL_ALLOC_AT", None)
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0 and "ALLOC_HOOK_OK" in r.stdout
