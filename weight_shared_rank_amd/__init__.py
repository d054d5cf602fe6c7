"""MI355X-native weightless linear: theta bundles evaluated by HIP kernels
behind the C ABI in include/weightless.h (see binding.py for the Python
entry points)."""
from .binding import ThetaBundle, WlError, lib, make_spec, theta_bundle_arena_bytes  # noqa: F401
