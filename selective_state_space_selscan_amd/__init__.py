"""MI355X (gfx950) S6 selective scan: Python binding of libselscan.

The work runs in the HIP kernels behind the C ABI in ``include/selscan.h``.
This module only marshals torch tensors (device memory) and the current HIP
stream into that ABI.  Nothing here computes any step of the scan, and there
is no CPU fallback.  If ``libselscan.so`` is missing, every call raises.

    y = selscan_fwd(u, delta, A, Bm, Cm, D_skip, z, delta_bias)
    y, h_last = selscan_fwd(..., return_last_state=True)
    y = selscan_fwd_ex(..., flags=SELSCAN_FLAG_REVERSE | SELSCAN_FLAG_ZOH_EXACT,
                       conv_weight=w, conv_bias=b)
    grads = selscan_bwd(u, delta, A, Bm, Cm, dy, D_skip, z, delta_bias, h0=h0,
                        dh_last=dh_last)
    grads = selscan_bwd_ex(..., flags=..., conv_weight=w, conv_bias=b)
    y = selscan_state_update(state, u, delta, A, Bm, Cm, D_skip, z, delta_bias)
"""
from ._abi import (  # noqa: F401
    SELSCAN_BF16,
    SELSCAN_F32,
    SELSCAN_FLAG_REUSE_FWD_STATE,
    SELSCAN_FLAG_KEEP_CHECKPOINTS,
    SELSCAN_FLAG_REVERSE,
    SELSCAN_FLAG_ZOH_EXACT,
    SELSCAN_MAX_CONV_WIDTH,
    SelscanError,
    lib,
    lib_path,
    selscan_bwd,
    selscan_bwd_ex,
    selscan_bwd_workspace_bytes,
    selscan_fwd,
    selscan_fwd_ex,
    selscan_fwd_noalloc,
    selscan_fwd_status,
    selscan_fwd_workspace_bytes,
    selscan_state_update,
    status_string,
)
