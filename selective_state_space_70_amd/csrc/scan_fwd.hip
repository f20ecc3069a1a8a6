// Selective scan (Mamba-1 form): the host dispatcher of one call (the kernels are
// in scan_kernels.h, instantiated per state size in scan_fwd_n*.hip).
#include "scan_kernels.h"

namespace ssm {
namespace {

// L == 0: the final state is the initial one.
__global__ __launch_bounds__(256) void copy_state_kernel(const float *h0, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

}  // namespace

ssm_status scan_launch(const ssm_scan_args &a, const ScanPlan &plan, hipStream_t s, int passes,
                       char *err, size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    if (a.seqlen == 0) {
        if (a.h_final && (passes & 2)) {
            const int64_t n = a.batch * a.dim * a.dstate;
            hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               s, a.h0, a.h_final, n);
        }
    } else {
        ScanK k{};
        k.x = a.x; k.delta = a.delta; k.z = a.z; k.Bm = a.Bm; k.Cm = a.Cm;
        k.A = a.A; k.bias = a.delta_bias; k.Dskip = a.Dskip; k.h0 = a.h0;
        k.y = a.y; k.h_final = a.h_final;
        k.agg = plan.chunks > 1 ? (float *)((char *)a.workspace + plan.agg_offset) : nullptr;
        k.pre = plan.chunks > kWalkChunks ? (float *)((char *)a.workspace + plan.pre_offset) : nullptr;
        k.L = a.seqlen; k.chunk_len = plan.chunk_len; k.D = (int32_t)a.dim;
        k.batch = (int32_t)a.batch; k.chunks = (int32_t)plan.chunks;
        k.dblocks = (int32_t)((a.dim + 63) / 64);
        k.softplus = a.delta_softplus ? 1 : 0;
        k.G = a.ngroups > 1 ? (int32_t)a.ngroups : 1;
        k.dpg = (int32_t)(a.dim / k.G);
        const bool bf = a.dtype == SSM_BF16;
        switch (a.dstate) {
            case 16: scan_launch_n16(k, s, passes, bf); break;
            case 32: scan_launch_n32(k, s, passes, bf); break;
            case 64: scan_launch_n64(k, s, passes, bf); break;
            default: return SSM_ENOTSUP;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(err, errlen, "selective_scan_fwd: kernel launch failed: %s",
                      hipGetErrorString(e));
        return SSM_EHIP;
    }
    return SSM_OK;
}

}  // namespace ssm
