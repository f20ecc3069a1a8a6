// selective_scan_fwd_noalloc: the selective scan with its scratch space (the time
// split's chunk maps and their prefixes) in a fixed file-scope device array
// instead of a caller workspace, so that the call allocates nothing. The kernels
// are those of selective_scan_fwd; they receive the array's device address like
// any workspace pointer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "internal.h"
#include "ssm.h"

// One copy per GPU the library runs on, held until the process ends. Host code
// must not use this name as a device address: it stands for the array only in
// device code and in hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];   // device address per device, once known
std::mutex g_scratch_mu;

// The scratch array's address on the current device, looked up once per device
// with that device current.
ssm_status scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return ssm::set_last_error(SSM_EHIP, "selective_scan_fwd_noalloc: no usable current device (%d)", dev);
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr)
                return ssm::set_last_error(SSM_EHIP,
                                           "selective_scan_fwd_noalloc: hipGetSymbolAddress on device %d: %s",
                                           dev, hipGetErrorString(e));
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return SSM_OK;
}

}  // namespace

extern "C" ssm_status selective_scan_fwd_noalloc(const ssm_scan_args *a, hipStream_t stream) {
    // every argument check first (host only), as in selective_scan_fwd
    const ssm_status st = selective_scan_validate(a);
    if (st != SSM_OK) return st;
    const size_t need = selective_scan_workspace_bytes(a);
    if (need > SSM_NOALLOC_SCRATCH_BYTES)
        return ssm::set_last_error(SSM_ENOTSUP,
                                   "selective_scan_fwd_noalloc: this call needs %zu bytes of scratch, "
                                   "more than the %zu of the fixed array (use selective_scan_fwd with "
                                   "a workspace)", need, (size_t)SSM_NOALLOC_SCRATCH_BYTES);
    void *ptr = nullptr;
    if (need > 0) {
        const ssm_status sa = scratch_address(&ptr);
        if (sa != SSM_OK) return sa;
    }
    ssm_scan_args b = *a;
    b.workspace = ptr;
    b.workspace_bytes = need > 0 ? (size_t)SSM_NOALLOC_SCRATCH_BYTES : 0;
    return selective_scan_fwd(&b, stream);
}
