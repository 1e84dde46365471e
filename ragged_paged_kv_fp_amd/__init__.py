"""MI355X-native ForwardPass attention step on a paged KV pool.

The computation lives in libfp.so (hand-written HIP for gfx950, C ABI in
include/fp.h). This package is its thin Python binding: `api` marshals
arguments, `runner` owns the device buffers of one pass, `build` compiles the
library in-tree.
"""

from . import _lib  # noqa: F401
from ._lib import FpError  # noqa: F401

__all__ = ["api", "runner", "build", "FpError"]


def __getattr__(name):
    # torch-dependent modules load lazily so that the ctypes layer imports without torch
    if name in ("api", "runner"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
