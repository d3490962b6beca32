"""Chunked delta-rule memory operator (DeltaNet, Gated DeltaNet, Kimi Delta Attention,
Gated DeltaNet-2) for AMD MI355X (gfx950): hand-written HIP kernels behind a C ABI
(include/gdr.h), with this package as a thin ctypes binding.

    from gated_delta_rule_73_amd import gdr_forward, gdr_backward, gdr_decode
"""
from .binding import (  # noqa: F401
    GdrError, GdrGrads, GdrInputs, GdrProblem, LIB_PATH, VARIANTS, gdr_backward, gdr_decode, gdr_forward,
    gdr_forward_noalloc, gdr_saved_size, gdr_workspace_size, load_library, make_problem,
)
