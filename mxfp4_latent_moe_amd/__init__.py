"""MI355X (gfx950) Stable LatentMoE layer with MXFP4 routed experts.

The compute lives in the HIP library libmoe_latent.so (C ABI in
include/moe_latent.h); this package is its thin Python binding.
"""
from . import _lib  # noqa: F401
from ._lib import (MOE_OPND_BF16, MOE_OPND_BF16X2, MOE_OPND_MX6X3, MOE_OPND_MX8X3, MoeError, MoeShape,  # noqa: F401
                   load, make_shape)
from .ops import LatentMoE, shape_of  # noqa: F401
