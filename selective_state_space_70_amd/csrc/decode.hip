// Decode step (sequence length 1) of both forms, the state updated in place.
//
// One step reads the fp32 state once and writes it once, so the step is bound by
// HBM on the state (8 N bytes per channel). Lanes are laid out so that those two
// streams are fully coalesced: a channel's N states are split over N/4 adjacent
// lanes, each holding 4 consecutive states (one 16-byte load and store), and the
// readout sum over n is finished with a butterfly over those lanes. Everything
// per channel (x, dt, z, the step size, the gate) is recomputed by each of its
// lanes, which costs ALU that the memory-bound step has to spare.
//
// The per-channel form has its own decay exp(dt A[d,n]) per state; the per-head
// (SSD) form shares dt and the scalar A of head h = d / P over the P channels of
// the head and all n [Mamba-2 page, Background and Core idea step 3: scalar A per
// head].
#include <cstdio>

#include "device_common.h"
#include "internal.h"

namespace ssm {
namespace {

struct StepK {
    const void *x, *dt, *z, *Bm, *Cm;
    const float *A, *dt_bias, *Dskip;
    float *state;
    void *y;
    int64_t channels;   // batch * D
    int32_t D;          // channels per batch row (dim, or H * P)
    int32_t P;          // channels per head (1 for the per-channel form)
    int32_t softplus;
    int32_t G;          // groups of B, C
    int32_t ppg;        // parameter rows (channels or heads) per group
};

typedef __attribute__((ext_vector_type(4))) float f32x4;

// Each thread updates the same lane position of U channel groups, U blocks of
// channels apart, so U independent state loads are in flight per lane.
template <typename T, int N, bool HEADS, int U>
__global__ __launch_bounds__(256) void state_update_kernel(const StepK k) {
    constexpr int G = N / 4;               // lanes per channel
    constexpr int CPB = 256 / G;           // channels per block
    const int tid = threadIdx.x, q = tid % G;
    const T *x = (const T *)k.x, *dtp = (const T *)k.dt, *z = (const T *)k.z;
    int64_t cs[U];
    bool ok[U];
    float xv[U], dtx[U], dtv[U], dsk[U], zv[U];
    f32x4 st[U], bv[U], cv[U], av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = ((int64_t)blockIdx.x * U + u) * CPB + tid / G;
        ok[u] = c < k.channels;            // whole channel groups drop out together
        cs[u] = ok[u] ? c : 0;
    }
    // Every load of the U channels first, then the arithmetic. C, D and z are loaded
    // here too: the state stores below may alias any of them as far as the compiler
    // knows, so a load placed after a store would wait for it to complete.
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = cs[u];
        const int64_t b = c / k.D;
        const int d = (int)(c % k.D);
        const int h = HEADS ? d / k.P : d;     // parameter index: head or channel
        const int64_t dt_idx = HEADS ? b * (k.D / k.P) + h : c;
        const int64_t row = (b * k.G + h / k.ppg) * N + 4 * q;     // (b, group, 4q..)
        const T *Bm = (const T *)k.Bm + row, *Cm = (const T *)k.Cm + row;
        // optional inputs are read from a valid stand-in when absent (A has an entry
        // for every head or channel, x one for every channel) and the value is dropped
        // afterwards: the loads stay unconditional, with no branch whose join would
        // wait for every load in flight
        const float *biasp = k.dt_bias ? k.dt_bias : k.A, *dskp = k.Dskip ? k.Dskip : k.A;
        const T *zp = z ? z : x;
        const float bias = biasp[h], dskv = dskp[h];
        dtv[u] = to_f32(dtp[dt_idx]) + (k.dt_bias ? bias : 0.0f);
        xv[u] = to_f32(x[c]);
        dsk[u] = k.Dskip ? dskv : 0.0f;
        zv[u] = to_f32(zp[c]);
        st[u] = *(const f32x4 *)(k.state + c * N + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bv[u][i] = to_f32(Bm[i]);
            cv[u][i] = to_f32(Cm[i]);
            av[u][i] = HEADS ? k.A[h] : k.A[(int64_t)d * N + 4 * q + i];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float dt = k.softplus ? softplus_f32(dtv[u]) : dtv[u];
        dtx[u] = dt * xv[u];
        dtv[u] = dt;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = cs[u];
        f32x4 s = st[u];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float decay = fast_exp2(dtv[u] * av[u][i] * kLog2e);
            s[i] = fmaf(decay, s[i], dtx[u] * bv[u][i]);
            part = fmaf(cv[u][i], s[i], part);
        }
        if (ok[u]) *(f32x4 *)(k.state + c * N + 4 * q) = s;
#pragma unroll
        for (int o = 1; o < G; o <<= 1) part += __shfl_xor(part, o, 64);
        if (ok[u] && q == 0) {
            float out = fmaf(dsk[u], xv[u], part);
            if (z) out *= silu_f32(zv[u]);
            store_val((T *)k.y + c, out);
        }
    }
}

template <typename T, bool HEADS>
void launch_step(const StepK &k, int N, hipStream_t s) {
    constexpr int U = 1;                     // channel groups per thread (2 and 4 measured slower)
    const int64_t cpb = 256 / (N / 4);       // channels per block
    const dim3 grid((unsigned)((k.channels + cpb * U - 1) / (cpb * U)));
    switch (N) {
        case 16: hipLaunchKernelGGL((state_update_kernel<T, 16, HEADS, U>), grid, dim3(256), 0, s, k); break;
        case 32: hipLaunchKernelGGL((state_update_kernel<T, 32, HEADS, U>), grid, dim3(256), 0, s, k); break;
        case 64: hipLaunchKernelGGL((state_update_kernel<T, 64, HEADS, U>), grid, dim3(256), 0, s, k); break;
        case 128: hipLaunchKernelGGL((state_update_kernel<T, 128, HEADS, U>), grid, dim3(256), 0, s, k); break;
        default: hipLaunchKernelGGL((state_update_kernel<T, 256, HEADS, U>), grid, dim3(256), 0, s, k); break;
    }
}

ssm_status finish(const char *who, char *err, size_t errlen) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(err, errlen, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
        return SSM_EHIP;
    }
    return SSM_OK;
}

}  // namespace

ssm_status step_launch(const ssm_scan_step_args &a, hipStream_t s, char *err, size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();
    StepK k{};
    k.x = a.x; k.dt = a.delta; k.z = a.z; k.Bm = a.Bm; k.Cm = a.Cm;
    k.A = a.A; k.dt_bias = a.delta_bias; k.Dskip = a.Dskip;
    k.state = a.state; k.y = a.y;
    k.channels = a.batch * a.dim; k.D = (int32_t)a.dim; k.P = 1;
    k.softplus = a.delta_softplus ? 1 : 0;
    k.G = a.ngroups > 1 ? (int32_t)a.ngroups : 1;
    k.ppg = (int32_t)(a.dim / k.G);
    if (a.dtype == SSM_BF16) launch_step<uint16_t, false>(k, (int)a.dstate, s);
    else launch_step<float, false>(k, (int)a.dstate, s);
    return finish("selective_state_update", err, errlen);
}

ssm_status ssd_step_launch(const ssm_ssd_step_args &a, hipStream_t s, char *err, size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();
    StepK k{};
    k.x = a.x; k.dt = a.dt; k.z = a.z; k.Bm = a.Bm; k.Cm = a.Cm;
    k.A = a.A; k.dt_bias = a.dt_bias; k.Dskip = a.Dskip;
    k.state = a.state; k.y = a.y;
    k.channels = a.batch * a.nheads * a.headdim;
    k.D = (int32_t)(a.nheads * a.headdim); k.P = (int32_t)a.headdim;
    k.softplus = a.dt_softplus ? 1 : 0;
    k.G = a.ngroups > 1 ? (int32_t)a.ngroups : 1;
    k.ppg = (int32_t)(a.nheads / k.G);
    if (a.dtype == SSM_BF16) launch_step<uint16_t, true>(k, (int)a.dstate, s);
    else launch_step<float, true>(k, (int)a.dstate, s);
    return finish("ssd_state_update", err, errlen);
}

}  // namespace ssm
