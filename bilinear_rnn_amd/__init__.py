"""Comba mixer hot path for AMD Instinct MI355X (gfx950).

The chunk-wise parallel forward and the recurrent (decode) step of Comba,
a bilinear RNN with a scalar-plus-low-rank state transition and output
correction, as hand-written HIP kernels behind a C ABI (include/comba.h).
This package is the thin Python binding over that library.
"""
from .api import (CombaError, bwd_cached_workspace_size, bwd_workspace_size, check_inputs,  # noqa: F401
                  chunk_bwd, chunk_fwd, chunk_fwd_noalloc,
                  chunk_states_size, lds_probe, lib, library_path,
                  mfma_peak_probe, recurrent_step, segmented_workspace_size, varlen_order, workspace_size)

__all__ = ["chunk_fwd", "chunk_bwd", "bwd_workspace_size", "bwd_cached_workspace_size", "chunk_states_size",
           "recurrent_step", "varlen_order", "workspace_size", "segmented_workspace_size", "mfma_peak_probe",
           "lds_probe", "check_inputs", "CombaError"]
