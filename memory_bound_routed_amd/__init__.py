"""Python binding of libmoe (gfx950 MoE decode-step library).

Argument marshalling only: every entry point forwards to the C ABI declared in
include/moe.h with the same name.  Tensors are passed by ``data_ptr()`` and
the stream is the current torch stream unless one is given.  PyTorch is used
for device memory and streams, nothing else.  There is no CPU fallback: if
libmoe.so is missing or fails to load, importing this package raises.

Build the library in-tree first:  python -m memory_bound_routed_amd._build
"""
from __future__ import annotations

import os
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

# While `python -m memory_bound_routed_amd._build` locates its target, the
# interpreter imports this package with sys.argv == ['-m'] (argv[0] becomes
# the script path only once the module is found).  That import loads nothing:
# the command builds the library, which may be missing or older than the
# binding.
_BUILDING = sys.argv[:1] == ["-m"]
if not os.path.exists(LIB_PATH) and not _BUILDING:
    raise ImportError("libmoe.so is not built at %s; run `python -m memory_bound_routed_amd._build`" % LIB_PATH)
if not _BUILDING:
    from ._binding import *  # noqa: F401,F403  (the entry points, Layer, constants)
    from ._binding import _lib  # noqa: F401  (the loaded library, for the ABI tests)
