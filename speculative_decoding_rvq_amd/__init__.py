"""MI355X-native CodePredictor speculative decoding.

The work runs in libcpspec.so (HIP kernels for gfx950 behind the C ABI of
include/cp_spec.h); ``binding`` is its ctypes wrapper.
"""
from . import binding  # noqa: F401
from .binding import Handle, get_stats, new_stats_tensor, weights_to_device  # noqa: F401
