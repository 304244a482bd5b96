"""MI355X (gfx950) Stable LatentMoE layer with MXFP4 routed experts.

The compute lives in the HIP library libmoe_latent.so (C ABI in
include/moe_latent.h); this package is its thin Python binding.
"""
from . import _lib  # noqa: F401
from ._lib import MoeError, MoeShape, load, make_shape  # noqa: F401
from .ops import LatentMoE, shape_of  # noqa: F401
