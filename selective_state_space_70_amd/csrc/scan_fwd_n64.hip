// Selective-scan kernels for N = 64 states (the templates are in scan_kernels.h;
// one state size per translation unit so that the sizes compile in parallel).
#include "scan_kernels.h"

namespace ssm {

ssm_status scan_launch_n64(const ScanK &k, hipStream_t s, int passes, bool bf16) {
    return bf16 ? launch_sp<uint16_t, 64>(k, s, passes) : launch_sp<float, 64>(k, s, passes);
}

}  // namespace ssm
