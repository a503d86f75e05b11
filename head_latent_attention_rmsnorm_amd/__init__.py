"""MI355X (gfx950) eager multi-head latent attention forward path.

The compute lives in libmla.so (HIP kernels behind the C ABI of
include/mla.h); this package is its thin PyTorch binding. Importing it loads
the library and fails loudly if it has not been built.
"""

from . import _lib

_lib.load()

from . import api, pipeline  # noqa: E402,F401
from .api import *  # noqa: E402,F401,F403

__version__ = "0.1.0"
