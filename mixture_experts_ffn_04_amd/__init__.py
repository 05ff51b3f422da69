"""libmoe: the routed mixture-of-experts FFN layer on AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI declared in
include/libmoe.h (built into libmoe.so); `binding` is the Python binding.
"""
from . import binding  # noqa: F401
from .binding import MoeLayer, MoeLayerGraph, MoeWeights  # noqa: F401
from .placement import balanced_shares, expert_map  # noqa: F401
