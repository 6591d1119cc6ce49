"""Causal kernelized linear attention (phi = elu + 1) on MI355X / gfx950.

The computation lives in the HIP library ``liblinattn.so`` (C ABI in
``include/linattn.h``); this package holds its ctypes binding, the in-tree
build script and the seeded synthetic workloads.  Importing the package does
not load the library; the first call does, and raises if it is missing.
"""
from .binding import (  # noqa: F401
    bwd,
    decode_step,
    fwd,
    decode_step_features,
    fwd_chunked,
    fwd_features,
    fwd_vdecay,
    fwd_gated,
    linattn_bwd,
    linattn_bwd_workspace_size,
    linattn_decode_step,
    linattn_decode_step_ex,
    linattn_fwd_chunked,
    linattn_fwd_ex,
    linattn_fwd_features,
    linattn_fwd_features_workspace_size,
    linattn_fwd_vdecay,
    linattn_fwd_vdecay_workspace_size,
    linattn_decode_step_vdecay,
    linattn_fwd_gated,
    linattn_fwd_workspace_size,
    linattn_set_profile_events,
    linattn_status_string,
    workspace_bytes,
)
