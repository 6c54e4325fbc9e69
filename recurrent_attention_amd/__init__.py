"""MI355X-native causal linear attention (unified recurrence) for gfx950.

The compute lives in the HIP library ``liblinattn.so`` (built in-tree from
``csrc/``) behind the C ABI declared in ``include/la.h``.  This package only
marshals arguments to it; importing it does not load the library, the first
call does, and a missing library is an error (there is no CPU fallback).
"""
from .api import (  # noqa: F401
    LA_GATE_NONE, LA_GATE_GAMMA, LA_GATE_DIAG, LA_GATE_SCALAR, LA_PHI_IDENTITY, LA_PHI_ELU1,
    LA_F32, LA_BF16, LaError, chunk_bwd, chunk_bwd_workspace_bytes, chunk_fwd, chunk_fwd_train,
    chunk_fwd_varlen, chunk_fwd_workspace_bytes,
    decode_step, delta_decode_step, delta_fwd, library_path, load_library,
)
