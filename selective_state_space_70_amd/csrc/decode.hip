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

template <typename T, int N, bool HEADS>
__global__ __launch_bounds__(256) void state_update_kernel(const StepK k) {
    constexpr int G = N / 4;               // lanes per channel
    constexpr int CPB = 256 / G;           // channels per block
    const int tid = threadIdx.x, q = tid % G;
    const int64_t c = (int64_t)blockIdx.x * CPB + tid / G;
    if (c >= k.channels) return;           // whole channel groups leave together
    const int64_t b = c / k.D;
    const int d = (int)(c % k.D);
    const int h = HEADS ? d / k.P : d;     // parameter index: head or channel
    const int64_t dt_idx = HEADS ? b * (k.D / k.P) + h : c;
    const T *x = (const T *)k.x, *dtp = (const T *)k.dt, *z = (const T *)k.z;
    const int64_t row = (b * k.G + h / k.ppg) * N + 4 * q;     // (b, group, 4q..)
    const T *Bm = (const T *)k.Bm + row, *Cm = (const T *)k.Cm + row;

    float v = to_f32(dtp[dt_idx]) + (k.dt_bias ? k.dt_bias[h] : 0.0f);
    const float dt = k.softplus ? softplus_f32(v) : v;
    const float xv = to_f32(x[c]);
    const float dtx = dt * xv;

    f32x4 *sp = (f32x4 *)(k.state + c * N + 4 * q);
    f32x4 s = *sp;
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = HEADS ? k.A[h] : k.A[(int64_t)d * N + 4 * q + i];
        const float decay = fast_exp2(dt * a * kLog2e);
        s[i] = fmaf(decay, s[i], dtx * to_f32(Bm[i]));
        part = fmaf(to_f32(Cm[i]), s[i], part);
    }
    *sp = s;
#pragma unroll
    for (int o = 1; o < G; o <<= 1) part += __shfl_xor(part, o, 64);
    if (q == 0) {
        float out = fmaf(k.Dskip ? k.Dskip[h] : 0.0f, xv, part);
        if (z) out *= silu_f32(to_f32(z[c]));
        store_val((T *)k.y + c, out);
    }
}

template <typename T, bool HEADS>
void launch_step(const StepK &k, int N, hipStream_t s) {
    const int64_t cpb = 256 / (N / 4);   // channels per block
    const dim3 grid((unsigned)((k.channels + cpb - 1) / cpb));
    switch (N) {
        case 16: hipLaunchKernelGGL((state_update_kernel<T, 16, HEADS>), grid, dim3(256), 0, s, k); break;
        case 32: hipLaunchKernelGGL((state_update_kernel<T, 32, HEADS>), grid, dim3(256), 0, s, k); break;
        case 64: hipLaunchKernelGGL((state_update_kernel<T, 64, HEADS>), grid, dim3(256), 0, s, k); break;
        case 128: hipLaunchKernelGGL((state_update_kernel<T, 128, HEADS>), grid, dim3(256), 0, s, k); break;
        default: hipLaunchKernelGGL((state_update_kernel<T, 256, HEADS>), grid, dim3(256), 0, s, k); break;
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
