"""MI355X-native (gfx950) 4-bit zig-zag block decode of OPT-style decoders.

The compute lives in libfg.so (hand-written HIP kernels behind the C ABI of
include/fg.h); ``_lib`` is its ctypes binding and ``model`` drives a whole
decoder through it.  Importing the binding fails if the library is not built.
"""
from . import _lib  # noqa: F401  (raises ImportError when libfg.so is missing)
from ._lib import FG_FMT_F16, FG_FMT_Q4G64, FgError  # noqa: F401
