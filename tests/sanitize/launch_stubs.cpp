// Stand-ins for the kernel launchers, for the host-only sanitizer build of the C
// ABI (which has no device code). The sanitizer driver only passes arguments
// that the host checks reject, or empty batches that return before launching, so
// none of these is ever reached; each reports SSM_EHIP if it is, which the driver
// counts as a failure.
#include <cstdio>

#include "internal.h"

namespace ssm {

static ssm_status unreachable(char *err, size_t errlen, const char *who) {
    std::snprintf(err, errlen, "%s reached in a host-only build", who);
    return SSM_EHIP;
}

// Like the real launchers, each returns at once for an empty batch.
ssm_status scan_launch(const ssm_scan_args &a, const ScanPlan &, hipStream_t, int, char *err, size_t n) {
    if (a.batch == 0) return SSM_OK;
    return unreachable(err, n, "scan_launch");
}
ssm_status ssd_launch(const ssm_ssd_args &a, const SSDPlan &, hipStream_t, char *err, size_t n) {
    if (a.batch == 0) return SSM_OK;
    return unreachable(err, n, "ssd_launch");
}
ssm_status ssd_bwd_launch(const ssm_ssd_bwd_args &a, const SSDBwdPlan &, hipStream_t, char *err, size_t n) {
    if (a.batch == 0) return SSM_OK;
    return unreachable(err, n, "ssd_bwd_launch");
}
ssm_status scan_bwd_launch(const ssm_scan_bwd_args &a, const ScanBwdPlan &, hipStream_t, char *err,
                           size_t n) {
    if (a.batch == 0) return SSM_OK;
    return unreachable(err, n, "scan_bwd_launch");
}
ssm_status step_launch(const ssm_scan_step_args &a, hipStream_t, char *err, size_t n) {
    if (a.batch == 0) return SSM_OK;
    return unreachable(err, n, "step_launch");
}
ssm_status ssd_step_launch(const ssm_ssd_step_args &a, hipStream_t, char *err, size_t n) {
    if (a.batch == 0) return SSM_OK;
    return unreachable(err, n, "ssd_step_launch");
}
ssm_status conv_launch(const ssm_conv_args &a, hipStream_t, char *err, size_t n) {
    if (a.batch == 0) return SSM_OK;
    return unreachable(err, n, "conv_launch");
}

}  // namespace ssm
