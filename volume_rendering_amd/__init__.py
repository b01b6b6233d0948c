"""MI355X-native NeRF forward-render hot path.

The work runs in ``libnerf_mi355x.so`` (hand-written HIP for gfx950) behind
the C ABI declared in ``include/nerf_mi355x.h``; this package is its thin
Python binding (``_binding``) plus argument-marshalling helpers
(``weights``).  PyTorch is used for device memory and streams only.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import EXPORTED, NerfError, lib  # noqa: F401
from . import weights  # noqa: F401
