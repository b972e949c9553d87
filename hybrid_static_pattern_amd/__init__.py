"""SAF hybrid causal attention for AMD MI355X (gfx950): Python side of libsaf.

The compute path is the C-ABI library libsaf.so (hand-written HIP kernels, declared in
include/saf.h); `saf` is its ctypes binding and `inputs` the seeded synthetic workloads.
"""
from . import inputs  # noqa: F401


def lib():
    """The ctypes binding module (imports torch on first use)."""
    from . import saf
    return saf
