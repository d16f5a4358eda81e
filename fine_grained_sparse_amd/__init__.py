"""Fine-grained MoE feed-forward layer for MI355X (gfx950): HIP kernels behind a C ABI.

The compute path lives in libfgs_moe.so (sources in csrc/, ABI in
include/fgs_moe.h); `binding` marshals torch tensors into it.
"""
from . import binding  # noqa: F401
from .binding import MoeLayer, MoeError, route_outputs, aux_struct  # noqa: F401
