"""The forward under HIP graph capture (serving loops replay a captured
decode step instead of launching its kernels one by one).

latentmoe_forward allocates nothing, synchronises nothing and records no
memset, so a capture on the caller's stream holds only its kernel launches.
Each replay is checked bit for bit against an eager forward of the same
input, with eager work and synchronisations between the replays, and with the
captured input overwritten between replays (the graph reads the buffer it was
captured with).
"""

import numpy as np
import pytest
import torch

from mixture_experts_layer_latentmoe_amd import _abi
from mixture_experts_layer_latentmoe_amd.layer import LatentMoE, to_device
from synth import get_config, make_workload
from synth.generate import f32_to_bf16_bits
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


@pytest.mark.parametrize("name", ["decode_eff", "decode_eff_fp8", "tiny_f32"])
def test_forward_replays_from_a_hip_graph(name):
    wl = make_workload(get_config(name))
    sh = wl.shape
    G.say(f"[gpu] graph replay {name}: T={sh.T}")
    layer = LatentMoE.from_workload(wl)
    try:
        rng = np.random.default_rng(11)
        draws = [rng.standard_normal((sh.T, sh.d)).astype(np.float32) for _ in range(2)]
        inputs = [wl.tensors["x"]] + [f32_to_bf16_bits(a) if sh.dtype == "bf16" else a for a in draws]
        xs = [to_device(a, sh.dtype, "cuda:0") for a in inputs]
        eager = []
        for x in xs:
            eager.append(layer.forward(x).clone())
        torch.cuda.synchronize()

        x_static = xs[0].clone()
        y_static = torch.empty_like(x_static)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                layer.forward(x_static, y=y_static)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer.forward(x_static, y=y_static)
        torch.cuda.synchronize()

        for rep in range(6):
            i = rep % len(xs)
            x_static.copy_(xs[i])
            y_static.fill_(0)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_static, eager[i]), (rep, i)
            # eager work between the replays
            y2 = layer.forward(xs[(i + 1) % len(xs)])
            torch.cuda.synchronize()
            assert torch.equal(y2, eager[(i + 1) % len(xs)]), rep
    finally:
        layer.close()
