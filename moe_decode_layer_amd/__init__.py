"""MI355X-native decode step of a DeepSeek-V4.1-style MoE layer half.

The computation runs in libmonolayer.so (hand-written HIP for gfx950, C ABI in
include/mono.h); this package is its ctypes binding. Importing it does not
require a GPU; calling a compute entry point does, and there is no CPU path.
"""

from ._binding import *  # noqa: F401,F403
from ._binding import (EXPORTS, FMT, LIB_PATH, Experts, Head, Layer, MonoError, Shape,  # noqa: F401
                       lib, make_experts, make_head, make_layer, make_shape, ptr)
