"""MI355X-native (gfx950) Q8_0 prefill forward: HIP kernels behind a C ABI, a ctypes binding."""
from . import binding  # noqa: F401
from .binding import MiError, lib  # noqa: F401
