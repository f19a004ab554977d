"""LatentMoE layer forward pass on MI355X (gfx950): hand-written HIP kernels
behind a C ABI (include/latentmoe.h), with a thin ctypes binding.

The library is loaded lazily by ``_abi.lib()`` and raises if it has not been
built; there is no other execution path.
"""

from . import _abi  # noqa: F401
from ._abi import (  # noqa: F401
    LatentMoEError,
    latentmoe_cost,
    latentmoe_create,
    latentmoe_destroy,
    latentmoe_forward,
    latentmoe_validate_config,
    latentmoe_workspace_bytes,
    make_config,
)
