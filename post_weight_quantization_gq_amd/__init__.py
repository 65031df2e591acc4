"""MI355X (gfx950) GuidedQuant Fisher + LNQ hot path.

The compute runs in the HIP library `_lib/libgq.so` (C ABI declared in
include/gq.h); `binding` marshals torch tensors to it.  Nothing here computes
on the CPU, and nothing here imports the oracle.
"""
from .binding import (  # noqa: F401
    GQError, library, abi_version, options, fisher, gq_fisher_accumulate, lnq_codebook_update,
    lnq_assign_sweep, lnq_objective, lnq_quantize, lnq_quantize_static, lnq_static_scratch_bytes,
    grid_quantize, lut_packed_row_words,
    lut_pack_codes, lut_gemv, gq_fisher_accumulate_host, fisher_stream_workspace_size,
    ganq_workspace_size, ganq_quantize, ganq_factor_damped,
    fisher_workspace_size,
    lnq_workspace_size, gq_timing_enable, gq_timing_read, EXPORTS, GQ_F32, GQ_BF16,
    GQ_INIT_QUANTILE, GQ_INIT_GIVEN, GQ_INIT_UNIFORM, GQ_GRAM_AUTO, GQ_GRAM_DENSE,
    GQ_ENOTPD, GQ_ENONFINITE, GQ_ECHECK, GQ_ESHAPE, GQ_EINVAL, DEFAULT_BLOCK,
)
