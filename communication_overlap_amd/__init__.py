"""Tile-centric overlap of communication with computation on MI355X.

The compute path lives in libovl.so (HIP kernels for gfx950 behind the C-ABI
of include/ovl.h); `ovl` is its ctypes binding.  Import the binding with
`from communication_overlap_amd import ovl`; loading it requires the built
library and fails loudly without it.
"""

__all__ = ["ovl", "build"]
