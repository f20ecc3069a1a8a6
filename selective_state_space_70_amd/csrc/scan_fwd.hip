// Selective scan (Mamba-1 form) for gfx950.
//
// Recurrence, per channel (b, d) with an N-dim fp32 state [Mamba-2 page
// "Mamba-2：把状态空间模型和 Attention 统一到一个数学框架里", Background: discrete
// recurrence; Core idea step 1: Delta, B, C depend on the input, A is discretised
// through Delta]:
//     dt = softplus(delta + bias),  h[n] = exp(dt A[n]) h[n] + dt B_t[n] x,
//     y  = (C_t . h + D x) silu(z)
//
// Mapping to the hardware (designed for CDNA4, not taken from the A100 kernel the
// pages describe):
//   * one lane = one channel; its N states live in VGPRs for the whole sequence,
//     so the expanded (B, L, D, N) state never exists in memory [SSM page
//     "状态空间模型与 Mamba", how it works: the scan keeps the expanded state out
//     of slow GPU memory].
//   * B_t and C_t are the same for every channel of a batch row, so they are read
//     with scalar loads into SGPRs and feed the VALU as scalar operands.
//   * x, delta, z and y are read/written once per (b, t, d); with lanes on
//     consecutive d each wave touches one contiguous 128/256-byte segment per step.
//   * Time is split into G chunks so that B*ceil(D/64)*G waves fill the 1024 SIMDs.
//     Chunk j > 0 needs the state entering it. Pass 1 runs every chunk but the last
//     from a zero state and stores its end state S_j and its summed step
//     sum(dt); pass 2 composes the affine maps h -> exp(A sum dt) h + S_j in order
//     (the associative combine (a1,b1),(a2,b2) -> (a2 a1, a2 b1 + b2) applied
//     chunk by chunk); pass 3 reruns every chunk from its true entering state and
//     writes y (and h_final from the last chunk).
//   * When a row of A has the form A[d,n] = (n+1) A[d,0] (checked exactly, per
//     channel, on the device), exp(dt A[d,n]) = r^(n+1) with r = exp(dt A[d,0]):
//     one exponential per (b,t,d) and a product tree for the powers instead of N
//     exponentials. Rows of any other form take the general path.
#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "device_common.h"
#include "internal.h"

namespace ssm {
namespace {

struct ScanK {
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *bias, *Dskip, *h0;
    void *y;
    float *h_final;
    float *carry;     // [G-1][B][D][N]
    double *dsum;     // [G-1][B][D]
    int64_t L;
    int64_t chunk_len;
    int32_t D;
    int32_t batch;
    int32_t chunks;
    int32_t softplus;
};

template <int N>
__device__ __forceinline__ bool row_is_geometric(const float *Arow) {
    const double a0 = (double)Arow[0];
    bool ok = true;
#pragma unroll
    for (int n = 1; n < N; ++n) ok = ok && ((double)Arow[n] == (double)(n + 1) * a0);
    return ok;
}

// pw[n] = r^(n+1) by a product tree: depth log2(N), fewer roundings than a chain.
template <int N>
__device__ __forceinline__ void powers(float r, float (&pw)[N]) {
    pw[0] = r;
#pragma unroll
    for (int n = 1; n < N; ++n) pw[n] = pw[(n - 1) / 2] * pw[n / 2];
}

// Runs steps [t0, t1) of one channel. READOUT: write y; otherwise accumulate sum(dt).
template <typename T, int N, bool FAST, bool READOUT>
__device__ __forceinline__ double run_steps(const ScanK &p, int b, int dc, bool act,
                                            int64_t t0, int64_t t1, float (&h)[N],
                                            const float (&Al2)[N], float bias, float dsk) {
    const int64_t row = (int64_t)b * p.L;
    const T *xb = (const T *)p.x + row * p.D;
    const T *db = (const T *)p.delta + row * p.D;
    const T *zb = p.z ? (const T *)p.z + row * p.D : nullptr;
    T *yb = READOUT ? (T *)p.y + row * p.D : nullptr;
    const T *Bb = (const T *)p.Bm + row * N;
    const T *Cb = (const T *)p.Cm + row * N;
    const bool softplus = p.softplus != 0;
    double dsum = 0.0;

#pragma unroll 2
    for (int64_t t = t0; t < t1; ++t) {
        const uint32_t off = (uint32_t)(t * p.D) + (uint32_t)dc;
        const float xv = to_f32(xb[off]);
        const float v = to_f32(db[off]) + bias;
        const float dt = softplus ? softplus_f32(v) : v;
        const float dtx = dt * xv;
        float Bv[N];
        SharedRow<T, N>::load(Bb + t * N, Bv);
        float a[N];
        if constexpr (FAST) {
            powers<N>(fast_exp2(dt * Al2[0]), a);
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) a[n] = fast_exp2(dt * Al2[n]);
        }
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = fmaf(a[n], h[n], Bv[n] * dtx);
        if constexpr (READOUT) {
            float Cv[N];
            SharedRow<T, N>::load(Cb + t * N, Cv);
            float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
            for (int n = 0; n < N; n += 2) {
                acc0 = fmaf(Cv[n], h[n], acc0);
                acc1 = fmaf(Cv[n + 1], h[n + 1], acc1);
            }
            float yv = fmaf(dsk, xv, acc0 + acc1);
            if (zb) yv *= silu_f32(to_f32(zb[off]));
            if (act) store_val(yb + off, yv);
        } else {
            dsum += (double)dt;
        }
    }
    return dsum;
}

template <typename T, int N, bool READOUT>
__device__ __forceinline__ double run_chunk(const ScanK &p, int b, int dc, bool act, int64_t t0,
                                            int64_t t1, float (&h)[N]) {
    const float *Arow = p.A + (int64_t)dc * N;
    float Al2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) Al2[n] = Arow[n] * kLog2e;
    const float bias = p.bias ? p.bias[dc] : 0.0f;
    const float dsk = p.Dskip ? p.Dskip[dc] : 0.0f;
    // wave-uniform choice of the exact fast path
    if (__all(row_is_geometric<N>(Arow)))
        return run_steps<T, N, true, READOUT>(p, b, dc, act, t0, t1, h, Al2, bias, dsk);
    return run_steps<T, N, false, READOUT>(p, b, dc, act, t0, t1, h, Al2, bias, dsk);
}

// Pass 1: end state and summed step of chunk j (0 <= j < G-1) from a zero state.
template <typename T, int N>
__global__ __launch_bounds__(64) void scan_chunk_state_kernel(const ScanK p) {
    const int d = blockIdx.x * 64 + threadIdx.x;
    const int b = blockIdx.y;
    const int j = blockIdx.z;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int64_t t0 = (int64_t)j * p.chunk_len;
    const int64_t t1 = min(p.L, t0 + p.chunk_len);
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = 0.0f;
    const double ds = run_chunk<T, N, false>(p, b, dc, act, t0, t1, h);
    if (act) {
        const int64_t c = ((int64_t)j * p.batch + b) * p.D + d;
        float *out = p.carry + c * N;
#pragma unroll
        for (int n = 0; n < N; ++n) out[n] = h[n];
        p.dsum[c] = ds;
    }
}

// Pass 2: sequential composition over chunks, one thread per (b, d, n). Slot j is
// overwritten with the state entering chunk j+1.
__global__ __launch_bounds__(256) void scan_carry_kernel(const ScanK p, int N) {
    const int64_t per = (int64_t)p.batch * p.D * N;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= per) return;
    const int64_t n = i % N;
    const int64_t bd = i / N;
    const int64_t d = bd % p.D;
    const double a = (double)p.A[d * N + n];
    float h = p.h0 ? p.h0[i] : 0.0f;
    for (int j = 0; j + 1 < p.chunks; ++j) {
        float *slot = p.carry + (int64_t)j * per + i;
        const double ds = p.dsum[(int64_t)j * p.batch * p.D + bd];
        const float decay = fast_exp2((float)(a * ds * 1.4426950408889634));
        h = fmaf(decay, h, *slot);
        *slot = h;
    }
}

// Pass 3: every chunk from its entering state, with readout, gate and store.
template <typename T, int N>
__global__ __launch_bounds__(64) void scan_main_kernel(const ScanK p) {
    const int d = blockIdx.x * 64 + threadIdx.x;
    const int b = blockIdx.y;
    const int k = blockIdx.z;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int64_t t0 = (int64_t)k * p.chunk_len;
    const int64_t t1 = min(p.L, t0 + p.chunk_len);
    const int64_t c = (int64_t)b * p.D + dc;
    const float *hin = nullptr;
    if (k == 0)
        hin = p.h0 ? p.h0 + c * N : nullptr;
    else
        hin = p.carry + ((int64_t)(k - 1) * p.batch * p.D + c) * N;
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = hin ? hin[n] : 0.0f;
    run_chunk<T, N, true>(p, b, dc, act, t0, t1, h);
    if (k == p.chunks - 1 && p.h_final && act) {
        float *out = p.h_final + c * N;
#pragma unroll
        for (int n = 0; n < N; ++n) out[n] = h[n];
    }
}

// L == 0: the final state is the initial one.
__global__ __launch_bounds__(256) void copy_state_kernel(const float *h0, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

template <typename T, int N>
ssm_status launch_typed(const ScanK &k, const ScanPlan &plan, hipStream_t s) {
    const dim3 blk(64);
    const unsigned dblocks = (unsigned)((k.D + 63) / 64);
    if (plan.chunks > 1) {
        hipLaunchKernelGGL((scan_chunk_state_kernel<T, N>),
                           dim3(dblocks, k.batch, (unsigned)(plan.chunks - 1)), blk, 0, s, k);
        const int64_t per = (int64_t)k.batch * k.D * N;
        hipLaunchKernelGGL(scan_carry_kernel, dim3((unsigned)((per + 255) / 256)), dim3(256), 0,
                           s, k, N);
    }
    hipLaunchKernelGGL((scan_main_kernel<T, N>), dim3(dblocks, k.batch, (unsigned)plan.chunks),
                       blk, 0, s, k);
    return SSM_OK;
}

}  // namespace

ScanPlan scan_plan(const ssm_scan_args &a) {
    ScanPlan pl{};
    pl.chunks = 1;
    pl.chunk_len = a.seqlen;
    if (a.seqlen <= 0 || a.batch <= 0 || a.dim <= 0) return pl;
    const int64_t waves = a.batch * ((a.dim + 63) / 64);
    // Enough waves for ~2 per SIMD (1024 SIMDs), chunks of at least 64 steps.
    int64_t G = (2048 + waves - 1) / waves;
    G = std::min<int64_t>(G, std::max<int64_t>(1, a.seqlen / 64));
    if (const char *env = std::getenv("SSM_SCAN_CHUNKS")) {  // tuning override
        const long v = std::strtol(env, nullptr, 10);
        if (v > 0) G = v;
    }
    G = std::max<int64_t>(1, std::min<int64_t>(G, std::min<int64_t>(a.seqlen, 65535)));
    pl.chunk_len = (a.seqlen + G - 1) / G;
    pl.chunks = (a.seqlen + pl.chunk_len - 1) / pl.chunk_len;
    if (pl.chunks > 1) {
        const int64_t slots = (pl.chunks - 1) * a.batch * a.dim;
        pl.carry_offset = 0;
        pl.dsum_offset = ((size_t)(slots * a.dstate) * sizeof(float) + 255) & ~(size_t)255;
        pl.bytes = pl.dsum_offset + (((size_t)slots * sizeof(double) + 255) & ~(size_t)255);
    }
    return pl;
}

ssm_status scan_launch(const ssm_scan_args &a, const ScanPlan &plan, hipStream_t s, char *err,
                       size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    if (a.seqlen == 0) {
        if (a.h_final) {
            const int64_t n = a.batch * a.dim * a.dstate;
            hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               s, a.h0, a.h_final, n);
        }
    } else {
        ScanK k{};
        k.x = a.x; k.delta = a.delta; k.z = a.z; k.Bm = a.Bm; k.Cm = a.Cm;
        k.A = a.A; k.bias = a.delta_bias; k.Dskip = a.Dskip; k.h0 = a.h0;
        k.y = a.y; k.h_final = a.h_final;
        k.carry = plan.chunks > 1 ? (float *)((char *)a.workspace + plan.carry_offset) : nullptr;
        k.dsum = plan.chunks > 1 ? (double *)((char *)a.workspace + plan.dsum_offset) : nullptr;
        k.L = a.seqlen; k.chunk_len = plan.chunk_len; k.D = (int32_t)a.dim;
        k.batch = (int32_t)a.batch; k.chunks = (int32_t)plan.chunks;
        k.softplus = a.delta_softplus ? 1 : 0;
        const bool bf = a.dtype == SSM_BF16;
        switch (a.dstate) {
            case 16: bf ? launch_typed<uint16_t, 16>(k, plan, s) : launch_typed<float, 16>(k, plan, s); break;
            case 32: bf ? launch_typed<uint16_t, 32>(k, plan, s) : launch_typed<float, 32>(k, plan, s); break;
            case 64: bf ? launch_typed<uint16_t, 64>(k, plan, s) : launch_typed<float, 64>(k, plan, s); break;
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
