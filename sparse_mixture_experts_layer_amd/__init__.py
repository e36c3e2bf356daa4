"""MI355X (gfx950) sparse mixture-of-experts FFN layer.

The layer runs in hand-written HIP kernels behind the C ABI declared in
include/moe_layer.h (library: lib/libmoe_mi355x.so in this package); this
package is the thin Python binding over it.  Build with
`python -m sparse_mixture_experts_layer_amd.build`.
"""
from ._binding import MoeError, LIB_PATH, load  # noqa: F401


def __getattr__(name):
    if name in ("MoELayer", "Route"):
        from . import layer
        return getattr(layer, name)
    raise AttributeError(name)
