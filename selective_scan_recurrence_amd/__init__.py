"""Selective state-space scan for AMD Instinct MI355X (gfx950).

The compute lives in libssm.so (hand-written HIP kernels behind the C ABI of
include/ssm.h); this package is its Python binding.  There is no CPU or
PyTorch fallback: if the library is not built, every call raises.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, SSM_BF16, SSM_DEVERR_IDS, SSM_DT_SOFTPLUS, SSM_ERR_ALIGN, SSM_ERR_DTYPE,
    SSM_ERR_HIP, SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_UNSUPPORTED, SSM_ERR_WORKSPACE, SSM_F32,
    SSM_DEVERR_RELAY, SSM_DEVERR_SEQLENS, SSM_HAS_D, SSM_OK, SsmError, SsmScanDesc, SsmScanExt, load, make_ext, selective_scan_bwd, selective_scan_bwd_conv, selective_scan_fwd,
    selective_scan_fwd_ext, selective_scan_fwd_static, selective_state_update, ssm_scan_ext_out_bytes,
    ssm_conv_bwd, ssm_conv_bwd_workspace_bytes, ssm_conv_fwd, ssm_get_device_error,
    ssm_scan_dgrad_layout, ssm_scan_fwd_plan, ssm_scan_out_bytes,
    ssm_scan_state_offset_bytes, ssm_scan_workspace_bytes, ssm_status_str, ssm_version,
)
