"""libfat5attn for MI355X: exact attention with T5 relative-position bias,
ALiBi, RoPE or a dense bias matrix, dense or packed, forward and backward,
in hand-written HIP kernels for gfx950 behind a C ABI (include/fat5attn.h).

Importing this package does not load the library; the first call does, and it
raises if ``libfat5attn.so`` has not been built (there is no fallback path).
"""
from .api import (  # noqa: F401
    ALiBi,
    DenseBias,
    FireBias,
    fire_theta_size,
    T5Bias,
    alibi_slopes,
    attention,
    cross_entropy,
    fa_bwd,
    fa_bwd_noalloc,
    fa_ce_bwd,
    fa_ce_fwd,
    fa_fwd,
    fa_fwd_workspace_size,
    fa_rmsnorm_bwd,
    fa_rmsnorm_fwd,
    fa_t5_buckets,
    fa_varlen_bwd,
    fa_varlen_fwd,
    rms_norm,
    varlen_attention,
)
from ._lib import LIB_PATH, FaError, load  # noqa: F401

__version__ = "0.1.0"
