"""Mamba selective scan, native on AMD Instinct MI355X (gfx950).

The scan runs in hand-written HIP kernels behind the C ABI of
``libmssm.so`` (declared in ``include/mssm.h``); this package is the thin
Python binding over it.  PyTorch supplies device memory and streams only.
"""
from .binding import (  # noqa: F401
    LIB_PATH, MAX_DCONV, MSSM_BF16, MSSM_F32, EXPORTS, MssmError, Problem, bwd_workspace_bytes,
    conv_bwd, conv_scan_fwd, conv_scan_fwd_train, conv_step, ctx_bytes, fwd_workspace_bytes, lib, problem, scan_bwd, scan_bwd_saved,
    scan_fwd, scan_fwd_noalloc, scan_fwd_train, ssd_bwd, ssd_bwd_saved, ssd_fwd, ssd_fwd_train, step, Stepper,
)

__all__ = ["scan_fwd", "scan_fwd_noalloc", "scan_fwd_train", "conv_scan_fwd", "conv_scan_fwd_train", "conv_bwd", "scan_bwd", "scan_bwd_saved",
           "ctx_bytes", "step", "Stepper", "conv_step", "ssd_fwd", "ssd_bwd", "ssd_fwd_train", "ssd_bwd_saved", "fwd_workspace_bytes", "bwd_workspace_bytes",
           "MssmError", "Problem", "problem", "lib", "LIB_PATH"]
