// Selective-scan backward kernels for gfx950 (reverse-time adjoint).
#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {

size_t bwd_workspace_bytes(const Shape&) { return 0; }

int launch_scan_bwd(const BwdArgs&, hipStream_t) { return SSM_ERR_UNSUPPORTED; }

}  // namespace ssm
