"""Delta-prefetched sparse FFN for AMD Instinct MI355X (gfx950).

The compute path is the HIP library libnp.so (C ABI in include/np.h);
`binding` marshals Python arguments into it. Build with
`python -m delta_prefetched_ffn_amd.build`.
"""
from . import binding  # noqa: F401
from .binding import (MASK_INTERSECT, MASK_SINGLE, MASK_UNION, MODES, Layer, NPError,  # noqa: F401
                      decode_step, decode_use_graphs, lib, probe_copy, probe_read)
