"""Fused selective state-space scan, forward and backward, for MI355X (gfx950).

The scan itself runs in the HIP library ``libssmscan.so`` behind the C ABI of
``include/ssm_scan.h``; this package is its thin binding (``selective_scan_fwd``,
``selective_scan_bwd`` and the raw ``ssm_*`` calls), the build script and the
seeded synthetic input generators.
"""
from ._binding import (EXPORTED, SSM_COMBINE_WALK, SSM_COMBINE_WAVE_SCAN, SSM_ERR_ALIAS, SSM_ERR_DEVICE_MISMATCH, SSM_ERR_HIP, SSM_ERR_INVALID_ARG,
                       SSM_ERR_NO_DEVICE, SSM_ERR_SCRATCH, SSM_ERR_UNSUPPORTED, SSM_IO_BF16, SSM_IO_F32, SSM_OK,
                       SSM_SCAN_NOALLOC_SCRATCH_BYTES, SsmScanError, auto_time_parts, bwd_chunk_len,
                       bwd_workspace_bytes, chunk_len, error_string, lib, library_path, selective_scan_bwd,
                       selective_scan_fwd, ssm_scan_bwd_io, ssm_scan_create, ssm_scan_destroy, ssm_scan_dims,
                       ssm_scan_fwd_extras, ssm_selective_scan_bwd, ssm_selective_scan_fwd, ssm_selective_scan_fwd_ex,
                       ssm_selective_scan_fwd_noalloc, workspace_bytes)

__all__ = [
    "selective_scan_fwd", "ssm_scan_create", "ssm_scan_destroy", "ssm_selective_scan_fwd", "ssm_scan_dims",
    "ssm_selective_scan_fwd_ex", "ssm_scan_fwd_extras", "chunk_len", "auto_time_parts", "workspace_bytes",
    "selective_scan_bwd", "ssm_selective_scan_bwd", "ssm_scan_bwd_io", "bwd_chunk_len", "bwd_workspace_bytes",
    "SsmScanError", "error_string", "lib", "library_path", "EXPORTED", "SSM_OK", "SSM_ERR_INVALID_ARG",
    "SSM_ERR_UNSUPPORTED", "SSM_ERR_ALIAS", "SSM_ERR_HIP", "SSM_ERR_NO_DEVICE", "SSM_ERR_DEVICE_MISMATCH",
    "SSM_COMBINE_WALK", "SSM_COMBINE_WAVE_SCAN", "SSM_ERR_SCRATCH", "SSM_IO_F32", "SSM_IO_BF16", "SSM_SCAN_NOALLOC_SCRATCH_BYTES", "ssm_selective_scan_fwd_noalloc",
]
