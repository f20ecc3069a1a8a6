// C ABI of libssm.so: argument checks (host only, before any HIP call), plans,
// and dispatch to the kernel launchers. See include/ssm.h for the contract.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"
#include "ssm.h"

namespace {

thread_local char g_err[512] = "";

ssm_status fail(ssm_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t esize(ssm_dtype t) { return t == SSM_BF16 ? 2 : 4; }

// The dtype field as the int a C caller stored. A C enum object may hold any int;
// loading a value outside ssm_dtype's range through the C++ enum type is undefined,
// so the checks read the bits, and only checked values are read as ssm_dtype.
static_assert(sizeof(ssm_dtype) == sizeof(int), "ssm_dtype is int-sized");
int dtype_bits(const ssm_dtype &f) {
    int v;
    std::memcpy(&v, &f, sizeof v);
    return v;
}
bool dtype_ok(const ssm_dtype &f) {
    const int v = dtype_bits(f);
    return v == SSM_F32 || v == SSM_BF16;
}

constexpr int64_t kMaxRowBytes = (int64_t)1 << 31;
// A launch's threads along one grid dimension (blocks * block size) must fit 32 bits;
// the element-wise kernels use one thread per element (up to 256 per block).
constexpr int64_t kMaxLaunchThreads = ((int64_t)1 << 32) - 256;

int64_t groups(int64_t g) { return g <= 1 ? 1 : g; }

// Sizes, dtype and supported shapes only (what the workspace query depends on).
ssm_status check_scan_sizes(const ssm_scan_args *a) {
    if (!a) return fail(SSM_EINVAL, "selective_scan: args is NULL");
    if (a->batch < 0 || a->seqlen < 0 || a->dim <= 0 || a->dstate <= 0)
        return fail(SSM_EINVAL, "selective_scan: need batch >= 0, seqlen >= 0, dim > 0, dstate > 0 "
                    "(got %lld, %lld, %lld, %lld)", (long long)a->batch, (long long)a->seqlen,
                    (long long)a->dim, (long long)a->dstate);
    if (!dtype_ok(a->dtype))
        return fail(SSM_EINVAL, "selective_scan: unknown dtype %d", dtype_bits(a->dtype));
    if (a->dstate != 16 && a->dstate != 32 && a->dstate != 64)
        return fail(SSM_ENOTSUP, "selective_scan: dstate %lld not supported (16, 32, 64)",
                    (long long)a->dstate);
    if (a->ngroups < 0 || a->dim % groups(a->ngroups))
        return fail(SSM_EINVAL, "selective_scan: ngroups %lld must be >= 0 and divide dim %lld",
                    (long long)a->ngroups, (long long)a->dim);
    if (groups(a->ngroups) > 1 && (a->dim / groups(a->ngroups)) % 64)
        return fail(SSM_ENOTSUP, "selective_scan: with several groups, dim / ngroups must be a "
                    "multiple of 64");
    // every operand is bounded before it enters a product, so no product below overflows
    if (a->batch > 65535 || a->dim > (1 << 30) || a->seqlen >= kMaxRowBytes)
        return fail(SSM_ENOTSUP, "selective_scan: batch <= 65535, dim <= 2^30 and seqlen < 2^31 supported");
    const size_t es = esize(a->dtype);
    if (a->seqlen * a->dim * (int64_t)es >= kMaxRowBytes)
        return fail(SSM_ENOTSUP, "selective_scan: seqlen*dim*elem_size must be < 2^31 bytes");
    if (a->seqlen * groups(a->ngroups) * a->dstate * (int64_t)es >= kMaxRowBytes)
        return fail(SSM_ENOTSUP, "selective_scan: seqlen*ngroups*dstate*elem_size must be < 2^31 bytes");
    if (a->batch * a->dim * a->dstate > kMaxLaunchThreads)
        return fail(SSM_ENOTSUP, "selective_scan: batch*dim*dstate must be < 2^32 (one thread per state element)");
    return SSM_OK;
}

ssm_status check_scan(const ssm_scan_args *a) {
    const ssm_status st = check_scan_sizes(a);
    if (st != SSM_OK) return st;
    const size_t es = esize(a->dtype);
    if (a->batch == 0) return SSM_OK;
    if (!a->A) return fail(SSM_EINVAL, "selective_scan: A is NULL");
    if (!aligned(a->A, 4) || !aligned(a->delta_bias, 4) || !aligned(a->Dskip, 4) ||
        !aligned(a->h0, 4) || !aligned(a->h_final, 4))
        return fail(SSM_EINVAL, "selective_scan: fp32 parameter/state pointers must be 4-byte aligned");
    if (a->seqlen == 0) return SSM_OK;
    if (!a->x || !a->delta || !a->Bm || !a->Cm || !a->y)
        return fail(SSM_EINVAL, "selective_scan: x, delta, Bm, Cm and y are required");
    if (!aligned(a->x, es) || !aligned(a->delta, es) || !aligned(a->z, es) || !aligned(a->y, es))
        return fail(SSM_EINVAL, "selective_scan: x, delta, z, y must be aligned to the element size");
    // B/C rows are fetched with scalar loads of whole dwords
    if (!aligned(a->Bm, 4) || !aligned(a->Cm, 4))
        return fail(SSM_EINVAL, "selective_scan: Bm and Cm must be 4-byte aligned");
    return SSM_OK;
}

ssm_status check_ssd_sizes(const ssm_ssd_args *a) {
    if (!a) return fail(SSM_EINVAL, "ssd_chunked: args is NULL");
    if (a->batch < 0 || a->seqlen < 0 || a->nheads <= 0 || a->headdim <= 0 || a->dstate <= 0 ||
        a->chunk <= 0)
        return fail(SSM_EINVAL, "ssd_chunked: need batch, seqlen >= 0 and nheads, headdim, "
                    "dstate, chunk > 0");
    if (!dtype_ok(a->dtype))
        return fail(SSM_EINVAL, "ssd_chunked: unknown dtype %d", dtype_bits(a->dtype));
    if (a->dtype != SSM_BF16)
        return fail(SSM_ENOTSUP, "ssd_chunked: only bf16 storage is implemented (matrix cores)");
    if (a->headdim != 64)
        return fail(SSM_ENOTSUP, "ssd_chunked: headdim %lld not supported (64)", (long long)a->headdim);
    if (a->dstate != 64 && a->dstate != 128 && a->dstate != 256)
        return fail(SSM_ENOTSUP, "ssd_chunked: dstate %lld not supported (64, 128, 256)",
                    (long long)a->dstate);
    if (a->chunk != 64 && a->chunk != 128 && a->chunk != 256)
        return fail(SSM_ENOTSUP, "ssd_chunked: chunk %lld not supported (64, 128, 256)",
                    (long long)a->chunk);
    if (a->ngroups < 0 || a->nheads % groups(a->ngroups))
        return fail(SSM_EINVAL, "ssd_chunked: ngroups %lld must be >= 0 and divide nheads %lld",
                    (long long)a->ngroups, (long long)a->nheads);
    // every operand is bounded before it enters a product, so no product below overflows
    if (a->batch > 65535 || a->nheads > 65535 || a->seqlen >= kMaxRowBytes)
        return fail(SSM_ENOTSUP, "ssd_chunked: batch and nheads must be <= 65535, seqlen < 2^31");
    if (a->seqlen * a->nheads * a->headdim * 2 >= kMaxRowBytes)
        return fail(SSM_ENOTSUP, "ssd_chunked: seqlen*nheads*headdim*2 must be < 2^31 bytes");
    if ((a->seqlen + a->chunk - 1) / a->chunk > 65535)
        return fail(SSM_ENOTSUP, "ssd_chunked: at most 65535 chunks");
    // threads of the output kernel: 4 * chunk per (batch, chunk, pair of heads),
    // the (batch, chunk) count rounded up to a multiple of 8. The chunk-state kernel's
    // one-dimensional grid is no larger: 256 threads per (batch, chunk, 4 heads of a
    // group), at most 256 * nheads per (batch, chunk).
    if ((a->batch * ((a->seqlen + a->chunk - 1) / a->chunk) + 7) * a->nheads * a->chunk * 4 >
        kMaxLaunchThreads)
        return fail(SSM_ENOTSUP, "ssd_chunked: batch * chunks * heads too large for one launch");
    // the state pass and the state copies run one thread per (4) state element(s)
    if (a->batch * a->nheads * a->headdim * a->dstate > kMaxLaunchThreads)
        return fail(SSM_ENOTSUP, "ssd_chunked: batch*nheads*headdim*dstate must be < 2^32");
    return SSM_OK;
}

ssm_status check_ssd(const ssm_ssd_args *a) {
    const ssm_status st = check_ssd_sizes(a);
    if (st != SSM_OK) return st;
    if (a->batch == 0) return SSM_OK;
    if (!a->A) return fail(SSM_EINVAL, "ssd_chunked: A is NULL");
    if (!aligned(a->A, 4) || !aligned(a->dt_bias, 4) || !aligned(a->Dskip, 4) ||
        !aligned(a->h0, 4) || !aligned(a->h_final, 4))
        return fail(SSM_EINVAL, "ssd_chunked: fp32 parameter/state pointers must be 4-byte aligned");
    if (a->seqlen == 0) return SSM_OK;
    if (!a->x || !a->dt || !a->Bm || !a->Cm || !a->y)
        return fail(SSM_EINVAL, "ssd_chunked: x, dt, Bm, Cm and y are required");
    // matrix-core tiles read 16-byte vectors of x, z, B and C and write 4-byte pairs of y
    if (!aligned(a->x, 16) || !aligned(a->z, 16) || !aligned(a->Bm, 16) || !aligned(a->Cm, 16) ||
        !aligned(a->y, 16) || !aligned(a->dt, 2))
        return fail(SSM_EINVAL, "ssd_chunked: x, z, y, Bm, Cm must be 16-byte aligned, dt 2-byte");
    return SSM_OK;
}

ssm_ssd_args ssd_sizes_of(const ssm_ssd_bwd_args *a) {
    ssm_ssd_args f{};
    f.batch = a->batch; f.seqlen = a->seqlen; f.nheads = a->nheads; f.headdim = a->headdim;
    f.dstate = a->dstate; f.chunk = a->chunk; f.ngroups = a->ngroups;
    std::memcpy(&f.dtype, &a->dtype, sizeof f.dtype);   // checked by check_ssd_sizes
    return f;
}

ssm_status check_ssd_bwd_sizes(const ssm_ssd_bwd_args *a) {
    if (!a) return fail(SSM_EINVAL, "ssd_chunked_bwd: args is NULL");
    const ssm_ssd_args f = ssd_sizes_of(a);
    const ssm_status st = check_ssd_sizes(&f);
    if (st != SSM_OK) return st;

    // dB and dC partial sums are reduced one thread per element
    if (a->batch * a->seqlen * groups(a->ngroups) * a->dstate > kMaxLaunchThreads)
        return fail(SSM_ENOTSUP, "ssd_chunked_bwd: batch*seqlen*ngroups*dstate must be < 2^32");
    return SSM_OK;
}

ssm_status check_ssd_bwd(const ssm_ssd_bwd_args *a) {
    const ssm_status st = check_ssd_bwd_sizes(a);
    if (st != SSM_OK) return st;
    if (a->batch == 0) return SSM_OK;
    if (!a->A || !a->dA) return fail(SSM_EINVAL, "ssd_chunked_bwd: A and dA are required");
    if (!aligned(a->A, 4) || !aligned(a->dt_bias, 4) || !aligned(a->Dskip, 4) || !aligned(a->h0, 4) ||
        !aligned(a->dh_final, 4) || !aligned(a->dA, 4) || !aligned(a->dDskip, 4) ||
        !aligned(a->ddt_bias, 4) || !aligned(a->dh0, 4))
        return fail(SSM_EINVAL, "ssd_chunked_bwd: fp32 parameters, states and their gradients must be 4-byte aligned");
    if (a->seqlen == 0) return SSM_OK;
    if (!a->x || !a->dt || !a->Bm || !a->Cm || !a->dy || !a->dx || !a->ddt || !a->dB || !a->dC)
        return fail(SSM_EINVAL, "ssd_chunked_bwd: x, dt, Bm, Cm, dy, dx, ddt, dB, dC are required");
    if (a->z && !a->dz) return fail(SSM_EINVAL, "ssd_chunked_bwd: dz is required when z is given");
    if (!aligned(a->x, 16) || !aligned(a->z, 16) || !aligned(a->Bm, 16) || !aligned(a->Cm, 16) ||
        !aligned(a->dy, 16) || !aligned(a->dx, 16) || !aligned(a->dz, 16) || !aligned(a->dt, 2) ||
        !aligned(a->ddt, 2) || !aligned(a->dB, 16) || !aligned(a->dC, 16))
        return fail(SSM_EINVAL, "ssd_chunked_bwd: x, z, Bm, Cm, dy, dx, dz, dB, dC must be 16-byte aligned, "
                    "dt and ddt 2-byte");
    return SSM_OK;
}

bool step_dstate_ok(int64_t n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }

ssm_status check_step(const ssm_scan_step_args *a) {
    if (!a) return fail(SSM_EINVAL, "selective_state_update: args is NULL");
    if (a->batch < 0 || a->dim <= 0 || a->dstate <= 0)
        return fail(SSM_EINVAL, "selective_state_update: need batch >= 0, dim > 0, dstate > 0");
    if (!dtype_ok(a->dtype))
        return fail(SSM_EINVAL, "selective_state_update: unknown dtype %d", dtype_bits(a->dtype));
    if (!step_dstate_ok(a->dstate))
        return fail(SSM_ENOTSUP, "selective_state_update: dstate %lld not supported (16..256, power of 2)",
                    (long long)a->dstate);
    if (a->ngroups < 0 || a->dim % groups(a->ngroups))
        return fail(SSM_EINVAL, "selective_state_update: ngroups must be >= 0 and divide dim");
    // batch * dim <= 2^34, tested by division so that the test itself cannot overflow
    if (a->dim > (1 << 30) || a->batch > ((int64_t)1 << 34) / a->dim)
        return fail(SSM_ENOTSUP, "selective_state_update: dim <= 2^30 and batch*dim <= 2^34 supported");
    // one thread per 4 states of a channel (and the rest of its last block)
    if (a->batch * a->dim * a->dstate / 4 + 256 > kMaxLaunchThreads)
        return fail(SSM_ENOTSUP, "selective_state_update: batch*dim*dstate must be < 2^34");
    if (a->batch == 0) return SSM_OK;
    if (!a->x || !a->delta || !a->Bm || !a->Cm || !a->A || !a->state || !a->y)
        return fail(SSM_EINVAL, "selective_state_update: x, delta, Bm, Cm, A, state and y are required");
    const size_t es = esize(a->dtype);
    if (!aligned(a->x, es) || !aligned(a->delta, es) || !aligned(a->z, es) || !aligned(a->Bm, es) ||
        !aligned(a->Cm, es) || !aligned(a->y, es))
        return fail(SSM_EINVAL, "selective_state_update: x, delta, z, Bm, Cm, y must be aligned to the element size");
    if (!aligned(a->A, 4) || !aligned(a->delta_bias, 4) || !aligned(a->Dskip, 4))
        return fail(SSM_EINVAL, "selective_state_update: fp32 parameters must be 4-byte aligned");
    if (!aligned(a->state, 16))
        return fail(SSM_EINVAL, "selective_state_update: state must be 16-byte aligned");
    return SSM_OK;
}

ssm_status check_ssd_step(const ssm_ssd_step_args *a) {
    if (!a) return fail(SSM_EINVAL, "ssd_state_update: args is NULL");
    if (a->batch < 0 || a->nheads <= 0 || a->headdim <= 0 || a->dstate <= 0)
        return fail(SSM_EINVAL, "ssd_state_update: need batch >= 0 and nheads, headdim, dstate > 0");
    if (!dtype_ok(a->dtype))
        return fail(SSM_EINVAL, "ssd_state_update: unknown dtype %d", dtype_bits(a->dtype));
    if (!step_dstate_ok(a->dstate))
        return fail(SSM_ENOTSUP, "ssd_state_update: dstate %lld not supported (16..256, power of 2)",
                    (long long)a->dstate);
    if (a->ngroups < 0 || a->nheads % groups(a->ngroups))
        return fail(SSM_EINVAL, "ssd_state_update: ngroups must be >= 0 and divide nheads");
    // batch * nheads * headdim <= 2^34, tested by division so that the test cannot overflow
    if (a->nheads > (1 << 20) || a->headdim > (1 << 20) || a->nheads * a->headdim > (1 << 30) ||
        a->batch > ((int64_t)1 << 34) / (a->nheads * a->headdim))
        return fail(SSM_ENOTSUP, "ssd_state_update: nheads*headdim <= 2^30 and batch*nheads*headdim <= 2^34");
    if (a->batch * a->nheads * a->headdim * a->dstate / 4 + 256 > kMaxLaunchThreads)
        return fail(SSM_ENOTSUP, "ssd_state_update: batch*nheads*headdim*dstate must be < 2^34");
    if (a->batch == 0) return SSM_OK;
    if (!a->x || !a->dt || !a->Bm || !a->Cm || !a->A || !a->state || !a->y)
        return fail(SSM_EINVAL, "ssd_state_update: x, dt, Bm, Cm, A, state and y are required");
    const size_t es = esize(a->dtype);
    if (!aligned(a->x, es) || !aligned(a->dt, es) || !aligned(a->z, es) || !aligned(a->Bm, es) ||
        !aligned(a->Cm, es) || !aligned(a->y, es))
        return fail(SSM_EINVAL, "ssd_state_update: x, dt, z, Bm, Cm, y must be aligned to the element size");
    if (!aligned(a->A, 4) || !aligned(a->dt_bias, 4) || !aligned(a->Dskip, 4))
        return fail(SSM_EINVAL, "ssd_state_update: fp32 parameters must be 4-byte aligned");
    if (!aligned(a->state, 16))
        return fail(SSM_EINVAL, "ssd_state_update: state must be 16-byte aligned");
    return SSM_OK;
}

ssm_status check_conv(const ssm_conv_args *a) {
    if (!a) return fail(SSM_EINVAL, "causal_conv1d: args is NULL");
    if (a->batch < 0 || a->seqlen < 0 || a->dim <= 0 || a->width <= 0)
        return fail(SSM_EINVAL, "causal_conv1d: need batch, seqlen >= 0 and dim, width > 0");
    if (!dtype_ok(a->dtype))
        return fail(SSM_EINVAL, "causal_conv1d: unknown dtype %d", dtype_bits(a->dtype));
    if (a->width < 2 || a->width > 4)
        return fail(SSM_ENOTSUP, "causal_conv1d: width %lld not supported (2, 3, 4)", (long long)a->width);
    if (a->batch > 65535 || a->dim > (1 << 30) || a->seqlen >= ((int64_t)1 << 31))
        return fail(SSM_ENOTSUP, "causal_conv1d: batch <= 65535, dim <= 2^30, seqlen < 2^31 supported");
    if (a->batch == 0) return SSM_OK;
    if (!a->weight) return fail(SSM_EINVAL, "causal_conv1d: weight is NULL");
    if (a->seqlen > 0 && (!a->x || !a->y))
        return fail(SSM_EINVAL, "causal_conv1d: x and y are required");
    const size_t es = esize(a->dtype);
    if (!aligned(a->x, es) || !aligned(a->y, es) || !aligned(a->init_state, es) ||
        !aligned(a->final_state, es))
        return fail(SSM_EINVAL, "causal_conv1d: x, y and the states must be aligned to the element size");
    if (!aligned(a->weight, 4) || !aligned(a->bias, 4))
        return fail(SSM_EINVAL, "causal_conv1d: weight and bias must be 4-byte aligned");
    if (a->final_state && (a->final_state == a->init_state || a->final_state == a->x))
        return fail(SSM_EINVAL, "causal_conv1d: final_state must not alias init_state or x");
    return SSM_OK;
}

ssm_status check_bwd_sizes(const ssm_scan_bwd_args *a) {
    if (!a) return fail(SSM_EINVAL, "selective_scan_bwd: args is NULL");
    ssm_scan_args f{};
    f.batch = a->batch; f.seqlen = a->seqlen; f.dim = a->dim; f.dstate = a->dstate;
    f.ngroups = a->ngroups;
    std::memcpy(&f.dtype, &a->dtype, sizeof f.dtype);   // checked by check_scan_sizes
    const ssm_status st = check_scan_sizes(&f);
    if (st != SSM_OK) return st;
    // chunks of 64 steps index the second grid dimension of the chunk kernels
    if ((a->seqlen + 63) / 64 > 65535)
        return fail(SSM_ENOTSUP, "selective_scan_bwd: seqlen must be <= 65535 * 64");
    if (a->batch * a->seqlen * groups(a->ngroups) * a->dstate > kMaxLaunchThreads)
        return fail(SSM_ENOTSUP, "selective_scan_bwd: batch*seqlen*ngroups*dstate must be < 2^32 "
                    "(dB and dC are cleared one thread per element)");
    return SSM_OK;
}

ssm_status check_bwd(const ssm_scan_bwd_args *a) {
    const ssm_status st = check_bwd_sizes(a);
    if (st != SSM_OK) return st;
    if (a->batch == 0) return SSM_OK;
    if (!a->A || !a->dA) return fail(SSM_EINVAL, "selective_scan_bwd: A and dA are required");
    if (a->seqlen > 0 && (!a->x || !a->delta || !a->Bm || !a->Cm || !a->dy || !a->dx || !a->ddelta ||
                          !a->dB || !a->dC))
        return fail(SSM_EINVAL, "selective_scan_bwd: x, delta, Bm, Cm, dy, dx, ddelta, dB, dC are required");
    if (a->z && !a->dz) return fail(SSM_EINVAL, "selective_scan_bwd: dz is required when z is given");
    const size_t es = esize(a->dtype);
    if (!aligned(a->x, es) || !aligned(a->delta, es) || !aligned(a->z, es) || !aligned(a->Bm, es) ||
        !aligned(a->Cm, es) || !aligned(a->dy, es) || !aligned(a->dx, es) || !aligned(a->ddelta, es) ||
        !aligned(a->dz, es))
        return fail(SSM_EINVAL, "selective_scan_bwd: tensors must be aligned to the element size");
    if (!aligned(a->A, 4) || !aligned(a->delta_bias, 4) || !aligned(a->Dskip, 4) || !aligned(a->h0, 4) ||
        !aligned(a->dh_final, 4) || !aligned(a->dB, 4) || !aligned(a->dC, 4) || !aligned(a->dA, 4) ||
        !aligned(a->dDskip, 4) || !aligned(a->ddelta_bias, 4) || !aligned(a->dh0, 4))
        return fail(SSM_EINVAL, "selective_scan_bwd: fp32 tensors must be 4-byte aligned");
    return SSM_OK;
}

ssm_status check_workspace(void *ws, size_t have, size_t need, const char *who) {
    if (need == 0) return SSM_OK;
    if (!ws) return fail(SSM_EINVAL, "%s: workspace of %zu bytes required", who, need);
    if (have < need)
        return fail(SSM_EINVAL, "%s: workspace too small (%zu < %zu bytes)", who, have, need);
    if (!aligned(ws, 256)) return fail(SSM_EINVAL, "%s: workspace must be 256-byte aligned", who);
    return SSM_OK;
}

}  // namespace

namespace ssm {
ssm_status set_last_error(ssm_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}
}  // namespace ssm

extern "C" {

ssm_status selective_scan_validate(const ssm_scan_args *a) {
    const ssm_status s = check_scan(a);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

size_t selective_scan_workspace_bytes(const ssm_scan_args *a) {
    if (check_scan_sizes(a) != SSM_OK) return 0;
    return ssm::scan_plan(*a).bytes;
}

static ssm_status scan_passes(const ssm_scan_args *a, hipStream_t stream, int passes) {
    ssm_status s = check_scan(a);
    if (s != SSM_OK) return s;
    const ssm::ScanPlan plan = ssm::scan_plan(*a);
    if (a->batch > 0 && a->seqlen > 0) {
        s = check_workspace(a->workspace, a->workspace_bytes, plan.bytes, "selective_scan");
        if (s != SSM_OK) return s;
    }
    s = ssm::scan_launch(*a, plan, stream, passes, g_err, sizeof g_err);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

ssm_status selective_scan_fwd(const ssm_scan_args *a, hipStream_t stream) {
    return scan_passes(a, stream, 3);
}

ssm_status selective_scan_chunk_states(const ssm_scan_args *a, hipStream_t stream) {
    return scan_passes(a, stream, 1);
}

ssm_status selective_scan_apply(const ssm_scan_args *a, hipStream_t stream) {
    return scan_passes(a, stream, 2);
}

ssm_status ssd_chunked_validate(const ssm_ssd_args *a) {
    const ssm_status s = check_ssd(a);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

size_t ssd_chunked_workspace_bytes(const ssm_ssd_args *a) {
    if (check_ssd_sizes(a) != SSM_OK) return 0;
    return ssm::ssd_plan(*a).bytes;
}

ssm_status ssd_chunked_fwd(const ssm_ssd_args *a, hipStream_t stream) {
    ssm_status s = check_ssd(a);
    if (s != SSM_OK) return s;
    const ssm::SSDPlan plan = ssm::ssd_plan(*a);
    if (a->batch > 0 && a->seqlen > 0) {
        s = check_workspace(a->workspace, a->workspace_bytes, plan.bytes, "ssd_chunked");
        if (s != SSM_OK) return s;
    }
    s = ssm::ssd_launch(*a, plan, stream, g_err, sizeof g_err);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

ssm_status selective_state_update(const ssm_scan_step_args *a, hipStream_t stream) {
    ssm_status s = check_step(a);
    if (s != SSM_OK) return s;
    s = ssm::step_launch(*a, stream, g_err, sizeof g_err);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

ssm_status ssd_state_update(const ssm_ssd_step_args *a, hipStream_t stream) {
    ssm_status s = check_ssd_step(a);
    if (s != SSM_OK) return s;
    s = ssm::ssd_step_launch(*a, stream, g_err, sizeof g_err);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

ssm_status causal_conv1d_fwd(const ssm_conv_args *a, hipStream_t stream) {
    ssm_status s = check_conv(a);
    if (s != SSM_OK) return s;
    s = ssm::conv_launch(*a, stream, g_err, sizeof g_err);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

size_t selective_scan_bwd_workspace_bytes(const ssm_scan_bwd_args *a) {
    if (check_bwd_sizes(a) != SSM_OK) return 0;
    return ssm::scan_bwd_plan(*a).bytes;
}

ssm_status selective_scan_bwd(const ssm_scan_bwd_args *a, hipStream_t stream) {
    ssm_status s = check_bwd(a);
    if (s != SSM_OK) return s;
    const ssm::ScanBwdPlan plan = ssm::scan_bwd_plan(*a);
    if (a->batch > 0 && a->seqlen > 0) {
        s = check_workspace(a->workspace, a->workspace_bytes, plan.bytes, "selective_scan_bwd");
        if (s != SSM_OK) return s;
    }
    s = ssm::scan_bwd_launch(*a, plan, stream, g_err, sizeof g_err);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

size_t ssd_chunked_bwd_workspace_bytes(const ssm_ssd_bwd_args *a) {
    if (check_ssd_bwd_sizes(a) != SSM_OK) return 0;
    return ssm::ssd_bwd_plan(*a).bytes;
}

ssm_status ssd_chunked_bwd(const ssm_ssd_bwd_args *a, hipStream_t stream) {
    ssm_status s = check_ssd_bwd(a);
    if (s != SSM_OK) return s;
    const ssm::SSDBwdPlan plan = ssm::ssd_bwd_plan(*a);
    if (a->batch > 0 && a->seqlen > 0) {
        s = check_workspace(a->workspace, a->workspace_bytes, plan.bytes, "ssd_chunked_bwd");
        if (s != SSM_OK) return s;
    }
    s = ssm::ssd_bwd_launch(*a, plan, stream, g_err, sizeof g_err);
    if (s == SSM_OK) g_err[0] = 0;
    return s;
}

const char *ssm_status_str(ssm_status s) {
    switch (s) {
        case SSM_OK: return "SSM_OK";
        case SSM_EINVAL: return "SSM_EINVAL";
        case SSM_ENOTSUP: return "SSM_ENOTSUP";
        case SSM_EHIP: return "SSM_EHIP";
    }
    return "SSM_UNKNOWN";
}

const char *ssm_last_error(void) { return g_err; }

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

}  // extern "C"
