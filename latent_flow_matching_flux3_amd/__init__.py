"""flux3_dit: the FLUX.3 Image Klein denoiser transformer on MI355X (gfx950).

The compute path is the HIP library libflux3_dit.so (C ABI in
include/flux3_dit.h); this package is its thin Python binding.
"""
from ._lib import *  # noqa: F401,F403
from ._lib import EXPORTS, LIB_PATH, lib  # noqa: F401
