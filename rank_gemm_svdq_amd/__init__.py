"""MI355X-native SVDQuant W4A4 + low-rank linear layer.

The compute lives in a C-ABI shared library (``include/svdq.h``) built from
``csrc/`` for gfx950; this package is its thin ctypes binding.  The library
is loaded on first use and a missing or unloadable library raises at once:
there is no fallback path.
"""

from .binding import *  # noqa: F401,F403
