"""MI355X (gfx950) Mamba-2 SSD core: forward and analytic backward, plus the
conv1d+SiLU and RMSNorm-gated block-shell ops and the dt activation
(softplus of dt_raw + dt_bias) in front of the core.

Thin Python binding over the C ABI in include/ssd.h (libssd_mi355x.so, built
by ``selective_state_space_mamba_amd.build``).  The binding only marshals
arguments: it checks devices, dtypes, shapes and contiguity, allocates outputs
and the workspace with PyTorch, and passes raw pointers plus the current HIP
stream.  Every step of the computation runs in the library's HIP kernels; if
the library is missing the calls raise.
"""
from ._binding import (  # noqa: F401
    SSDError,
    cast_bf16,
    conv1d_silu_bwd,
    conv1d_silu_fwd,
    dt_softplus_bwd,
    dt_softplus_fwd,
    gemm,
    library_path,
    load_library,
    profile_enable,
    profile_kernel_ms,
    profile_only,
    rmsnorm_gated_bwd,
    rmsnorm_gated_fwd,
    ssd_bwd,
    ssd_bwd_noalloc,
    NOALLOC_SCRATCH_BYTES,
    ssd_fwd,
    ssd_fwd_ex,
    ssd_workspace_bytes,
    version,
)
from .autograd import mamba2_block, mamba2_block_core, ssd_scan  # noqa: F401,E402
