"""MI355X (gfx950) GuidedQuant Fisher + LNQ hot path.

The compute runs in the HIP library `libgq.so` (C ABI declared in include/gq.h);
`binding` marshals torch tensors to it.  Nothing here computes on the CPU.
"""
from .binding import (  # noqa: F401
    GQError, library, abi_version, fisher, lnq_codebook_update, lnq_assign_sweep,
    lnq_objective, lnq_quantize, lnq_options,
)
