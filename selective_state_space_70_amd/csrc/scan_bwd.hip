// Gradients of the selective scan (training; the pages note that training runs
// the same scan [Mamba-2 page "Mamba-2：把状态空间模型和 Attention 统一到一个数学框架里",
// Core idea: Mamba-1's scan and its training throughput]).
//
// Reverse-mode through h_t = a_t o h_{t-1} + dt_t x_t B_t, a_t = exp(dt_t A): the
// adjoint g_t = dL/dh_t runs backwards in time, g_t = C_t dyc_t + a_{t+1} o g_{t+1}
// (dyc_t = dy_t silu(z_t)), and every gradient is a local product of g_t with
// forward quantities (h_{t-1}, h_t, dt_t, x_t, B_t). Both recurrences are linear
// with the same decays, so time is cut into chunks of kChunk steps and each
// chunk's entering state (from the left) and entering adjoint (from the right)
// are composed from per-chunk aggregates:
//   1. bwd_aggregate: per (64 channels, chunk), lane = channel, one pass forward
//      through the chunk: end state from zero S_c, summed step, and the adjoint
//      aggregate Q_c = sum_s (prod_{k=t0..s} a_k) C_s dyc_s;
//   2. bwd_carry: per channel, sequential over chunks: h entering chunk c is
//      h0 carried through the maps h -> exp(A sum dt) o h + S; the adjoint entering
//      chunk c from the right is dh_final carried back through u -> exp(A sum dt) o u
//      + Q. Both are stored per (batch, chunk, channel, n);
//   3. bwd_main: per (chunk, 32/16/8 channels), lane = (channel, n) so that one
//      lane holds one scalar state: the chunk is recomputed forward with every h_t
//      kept in registers, then the adjoint sweeps it backwards. Sums over n (dx,
//      dt, the readout) are DPP row reductions and permlane swaps; sums over
//      channels (dB, dC, shared by the channels of a group) are permlane swaps,
//      then LDS and global float atomics. Per-(t, channel) work (softplus, gate,
//      dz, dx, ddelta) is done once per pair through LDS, not per lane.
#include <algorithm>
#include <cstdio>

#include "device_common.h"
#include "internal.h"

namespace ssm {
namespace {

constexpr int kChunk = kScanBwdChunk;   // steps per chunk (states of a chunk live in VGPRs)
constexpr int kWaves = 8;    // waves per workgroup of the main kernel

struct BwdK {
    const void *x, *delta, *z, *Bm, *Cm, *dy;
    const float *A, *bias, *Dskip, *h0, *dh_final;
    void *dx, *ddelta, *dz;
    float *dB, *dC, *dA, *dDskip, *dbias, *dh0;
    float *aggF;     // [chain][chunk][N+1][64]: end state from zero, then summed dt
    float *aggR;     // [chain][chunk][N][64]: adjoint aggregate
    float *hin;      // [batch][chunk][D][N]: state entering each chunk
    float *uin;      // [batch][chunk][D][N]: adjoint entering each chunk from the right
    float *dApart;   // [batch][chunk][D][N]: each chunk's share of dA
    int64_t L;
    int32_t D, batch, nch, dblocks, softplus, G, dpg;
};

// ---------------------------------------------------------------- cross-lane sums
template <int CTRL>
__device__ __forceinline__ float ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
// sum over the 16 lanes of a DPP row, in every lane of the row (rotations 1, 2, 4, 8)
__device__ __forceinline__ float row_sum(float v) {
    v += ror<0x121>(v);
    v += ror<0x122>(v);
    v += ror<0x124>(v);
    v += ror<0x128>(v);
    return v;
}
// Row-swap sums: v_permlane16_swap exchanges the odd rows of its first operand
// with the even rows of its second, v_permlane32_swap the upper half of the first
// with the lower half of the second. With v as both operands the two results add
// up to v[l] + v[l ^ 16] (v[l] + v[l ^ 32]) in every lane. The two results are
// copied out as integers before use: reinterpreting the second element of the
// returned pair in place reads the first one with this compiler.
__device__ __forceinline__ float pl16_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t a = r[0], b = r[1];
    return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float pl32_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t a = r[0], b = r[1];
    return __uint_as_float(a) + __uint_as_float(b);
}
// sum over the N lanes of one channel (lane = channel * N + n), in every lane
template <int N>
__device__ __forceinline__ float sum_n(float v) {
    v = row_sum(v);
    if constexpr (N >= 32) v = pl16_sum(v);
    if constexpr (N >= 64) v = pl32_sum(v);
    return v;
}
// sum over the 64 / N channels of a wave at equal n, in every lane
template <int N>
__device__ __forceinline__ float sum_ch(float v) {
    if constexpr (N <= 16) v = pl16_sum(v);
    if constexpr (N <= 32) v = pl32_sum(v);
    return v;
}

__device__ __forceinline__ float sigmoid_f32(float v) { return fast_rcp(1.0f + fast_exp2(-v * kLog2e)); }

// ---------------------------------------------------------------- 1. aggregates
// Rows A[d, n] = (n+1) A[d, 0] (checked exactly, in fp64) give exp(dt A[d, n]) =
// r^(n+1) with r = exp(dt A[d, 0]): the decays are powers of one exponential, and
// the running product of decays from the chunk start is a power of one scalar.
template <int N>
__device__ __forceinline__ bool geometric_row(const float *Arow) {
    const double a0 = (double)Arow[0];
    bool ok = true;
#pragma unroll
    for (int n = 1; n < N; ++n) ok = ok && ((double)Arow[n] == (double)(n + 1) * a0);
    return ok;
}

// pw[n] = r^(n+1) by a product tree
template <int N>
__device__ __forceinline__ void powers_of(float r, float (&pw)[N]) {
    pw[0] = r;
#pragma unroll
    for (int n = 1; n < N; ++n) pw[n] = pw[(n - 1) / 2] * pw[n / 2];
}

template <typename T, int N, bool HAS_Z, bool FAST>
__device__ __forceinline__ void aggregate_chunk(const BwdK &p, int b, int dc, int t0, int t1, const float (&Al2)[N],
                                                float bias, float (&S)[N], float (&Q)[N], float &dsum) {
    const int g = __builtin_amdgcn_readfirstlane(dc) / p.dpg;
    const int GN = p.G * N;
    const T *Brow = (const T *)p.Bm + ((int64_t)b * p.L * p.G + g) * N;
    const T *Crow = (const T *)p.Cm + ((int64_t)b * p.L * p.G + g) * N;
    const T *X = (const T *)p.x, *Dl = (const T *)p.delta, *Z = (const T *)p.z, *DY = (const T *)p.dy;
    float R[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        S[n] = 0.0f;
        R[n] = 1.0f;
        Q[n] = 0.0f;
    }
    float rho = 1.0f;   // FAST: product of r over the chunk so far
    dsum = 0.0f;
    constexpr int U = 8;   // steps whose loads are issued together
    for (int t = t0; t < t1; t += U) {
        float xs[U], vs[U], dys[U], zs[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = ((int64_t)b * p.L + min(t + u, t1 - 1)) * p.D + dc;
            xs[u] = to_f32(X[e]);
            vs[u] = to_f32(Dl[e]);
            dys[u] = to_f32(DY[e]);
            zs[u] = HAS_Z ? to_f32(Z[e]) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t + u < t1) {
                const float v = vs[u] + bias;
                const float dt = p.softplus ? softplus_f32(v) : v;
                float dyc = dys[u];
                if constexpr (HAS_Z) dyc *= silu_f32(zs[u]);
                float Bv[N], Cv[N];
                SharedRow<T, N>::load(Brow + (t + u) * GN, Bv);
                SharedRow<T, N>::load(Crow + (t + u) * GN, Cv);
                const float dtx = dt * xs[u];
                dsum += dt;
                if constexpr (FAST) {
                    const float r = fast_exp2(dt * Al2[0]);
                    rho *= r;
                    float a[N];
                    powers_of<N>(r, a);
                    float q = rho * dyc;                      // rho^(n+1) dyc, built up over n
#pragma unroll
                    for (int n = 0; n < N; ++n) {
                        S[n] = fmaf(a[n], S[n], dtx * Bv[n]);
                        Q[n] = fmaf(Cv[n], q, Q[n]);
                        q *= rho;
                    }
                } else {
#pragma unroll
                    for (int n = 0; n < N; ++n) {
                        const float a = fast_exp2(dt * Al2[n]);
                        S[n] = fmaf(a, S[n], dtx * Bv[n]);
                        R[n] *= a;
                        Q[n] = fmaf(R[n], Cv[n] * dyc, Q[n]);
                    }
                }
            }
        }
    }
}

template <typename T, int N, bool HAS_Z>
__global__ __launch_bounds__(64) void bwd_aggregate_kernel(const BwdK p) {
    const int chain = blockIdx.x, c = blockIdx.y;   // chains on x (no 65535 limit), chunks on y
    const int b = chain / p.dblocks;
    const int d = (chain % p.dblocks) * 64 + threadIdx.x;
    const int dc = d < p.D ? d : p.D - 1;
    const int t0 = c * kChunk;
    const int t1 = (int)std::min<int64_t>(p.L, (int64_t)t0 + kChunk);
    float Al2[N];
#pragma unroll
    for (int n = 0; n < N; ++n) Al2[n] = p.A[(int64_t)dc * N + n] * kLog2e;
    const float bias = p.bias ? p.bias[dc] : 0.0f;
    float S[N], Q[N], dsum;
    if (__all(geometric_row<N>(p.A + (int64_t)dc * N)))   // wave-uniform choice
        aggregate_chunk<T, N, HAS_Z, true>(p, b, dc, t0, t1, Al2, bias, S, Q, dsum);
    else
        aggregate_chunk<T, N, HAS_Z, false>(p, b, dc, t0, t1, Al2, bias, S, Q, dsum);
    float *f = p.aggF + ((size_t)chain * p.nch + c) * (N + 1) * 64 + threadIdx.x;
    float *r = p.aggR + ((size_t)chain * p.nch + c) * N * 64 + threadIdx.x;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        f[n * 64] = S[n];
        r[n * 64] = Q[n];
    }
    f[N * 64] = dsum;
}

// ---------------------------------------------------------------- 2. carry
template <int N>
__global__ __launch_bounds__(64) void bwd_carry_kernel(const BwdK p) {
    const int chain = blockIdx.x;
    const int b = chain / p.dblocks;
    const int d = (chain % p.dblocks) * 64 + threadIdx.x;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    float Al2[N], h[N];
    const int64_t ci = (int64_t)b * p.D + dc;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        Al2[n] = p.A[(int64_t)dc * N + n] * kLog2e;
        h[n] = p.h0 ? p.h0[ci * N + n] : 0.0f;
    }
    const float *F = p.aggF + (size_t)chain * p.nch * (N + 1) * 64 + threadIdx.x;
    const float *Rg = p.aggR + (size_t)chain * p.nch * N * 64 + threadIdx.x;
    // The aggregates of the next chunk are loaded one chunk ahead, before this chunk's
    // stores: the chain is serial over chunks, and the memory counter completes in
    // order, so a load issued after a store could not be waited for without the store.
    // Chunk indices are clamped into the chain (loaded again, not used).
    const int last = p.nch - 1;
    float cur[N + 1], nxt[N + 1];   // end state from zero (n < N), summed step (N)
    auto load_f = [&](int c, float (&r)[N + 1]) {
        const float *f = F + (size_t)min(c, last) * (N + 1) * 64;
#pragma unroll
        for (int n = 0; n <= N; ++n) r[n] = f[n * 64];
    };
    load_f(0, cur);
    for (int c = 0; c < p.nch; ++c) {
        load_f(c + 1, nxt);
        float *o = p.hin + (((int64_t)b * p.nch + c) * p.D + dc) * N;
        if (act) {
#pragma unroll
            for (int n = 0; n < N; ++n) o[n] = h[n];
        }
        if (c < last) {
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = fmaf(fast_exp2(Al2[n] * cur[N]), h[n], cur[n]);
        }
#pragma unroll
        for (int n = 0; n <= N; ++n) cur[n] = nxt[n];
    }
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = p.dh_final ? p.dh_final[ci * N + n] : 0.0f;
    // backwards: chunk c needs its summed step and its adjoint aggregate (c > 0)
    auto load_r = [&](int c, float (&r)[N + 1]) {
        const int cc = max(c, 0);
        const float *q = Rg + (size_t)cc * N * 64;
#pragma unroll
        for (int n = 0; n < N; ++n) r[n] = q[n * 64];
        r[N] = F[(size_t)cc * (N + 1) * 64 + N * 64];
    };
    load_r(last, cur);
    for (int c = last; c >= 0; --c) {
        load_r(c - 1, nxt);
        float *o = p.uin + (((int64_t)b * p.nch + c) * p.D + dc) * N;
        if (act) {
#pragma unroll
            for (int n = 0; n < N; ++n) o[n] = h[n];
        }
        if (c > 0) {
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = fmaf(fast_exp2(Al2[n] * cur[N]), h[n], cur[n]);
        }
#pragma unroll
        for (int n = 0; n <= N; ++n) cur[n] = nxt[n];
    }
}

// ---------------------------------------------------------------- 3. main
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// Forward recompute and adjoint sweep of one chunk for lane (channel ch, state n).
// Steps past the end of the sequence were staged with dt = dt x = dyc = 0: they
// leave h and the adjoint unchanged and contribute nothing, so every chunk runs
// all kChunk steps without guards. A first forward pass keeps h at the start of
// each sub-block of SB steps; each sub-block, last first, is then recomputed with
// its states and decays kept in registers and swept backwards. This holds 2 SB
// values per lane instead of kChunk, which leaves room for more waves per SIMD.
constexpr int kSB = 16;   // steps per sub-block of the backward sweep

template <int N, int CPG>
__device__ __forceinline__ void sweep(const f32x4 (*pre)[CPG], const f32x2 (*BC)[N], float (*post)[kChunk][CPG],
                                      f32x2 (*bcw)[kSB][64], f32x2 (*bcacc)[N], int ch, int n, int lane, int wv,
                                      float An, float hin, float &v, float &dAacc) {
    constexpr int SB = kSB, NSB = kChunk / SB;
    const float A2 = An * kLog2e;
    float ck[NSB];
    float h = hin;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        ck[sb] = h;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int i = sb * SB + j;
            const f32x4 q = pre[i][ch];
            h = fmaf(fast_exp2(q[0] * A2), h, q[1] * BC[i][n][0]);
            if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);   // bound how far loads run ahead
        }
    }
#pragma unroll
    for (int sb = NSB - 1; sb >= 0; --sb) {
        __builtin_amdgcn_sched_barrier(0);
        float hs[SB], as[SB];
        float hh = ck[sb];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int i = sb * SB + j;
            const f32x4 q = pre[i][ch];
            as[j] = fast_exp2(q[0] * A2);
            hh = fmaf(as[j], hh, q[1] * BC[i][n][0]);
            hs[j] = hh;
            if (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = SB - 1; j >= 0; --j) {
            const int i = sb * SB + j;
            const f32x4 q = pre[i][ch];                   // dt, dt x, dyc, x
            const f32x2 bc = BC[i][n];                    // B, C
            const float gq = fmaf(bc[1], q[2], v);        // g_t
            const float hp = j > 0 ? hs[j - 1] : ck[sb];  // h_{t-1}
            const float gah = gq * as[j] * hp;
            dAacc = fmaf(gah, q[0], dAacc);
            const float yc = sum_n<N>(bc[1] * hs[j]);
            const float sB = sum_n<N>(gq * bc[0]);
            const float sA = sum_n<N>(An * gah);
            if (n == 0) {
                post[0][i][ch] = yc;
                post[1][i][ch] = sB;
                post[2][i][ch] = sA;
            }
            bcw[wv][j][lane] = f32x2{gq * q[1], q[2] * hs[j]};   // this lane's terms of dB_t, dC_t
            v = as[j] * gq;                               // the adjoint term for t-1
            if (j % 4 == 0) __builtin_amdgcn_sched_barrier(0);
        }
        // sum the waves' shares of this sub-block (no atomics)
        __syncthreads();
        for (int q = threadIdx.x; q < SB * N; q += kWaves * 64) {
            const int j = q / N, nn = q % N;
            f32x2 acc = f32x2{0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
#pragma unroll
                for (int c2 = 0; c2 < 64 / N; ++c2) acc += bcw[w][j][c2 * N + nn];
            bcacc[sb * SB + j][nn] = acc;
        }
        __syncthreads();
    }
}

template <typename T, int N, bool HAS_Z>
__global__ __launch_bounds__(kWaves * 64, 2) void bwd_main_kernel(const BwdK p) {
    constexpr int CPW = 64 / N;               // channels per wave
    constexpr int CPG = kWaves * CPW;         // channels per workgroup
    constexpr int NT = kWaves * 64;
    __shared__ f32x4 pre[kChunk][CPG];        // per (step, channel): dt, dt x, dyc, x
    __shared__ float post[3][kChunk][CPG];    // readout C.h, sum_n g B, sum_n A g a h_prev
    __shared__ f32x2 BC[kChunk][N];           // B_t[n], C_t[n]
    __shared__ f32x2 bcw[kWaves][kSB][64];    // per lane: its dB_t, dC_t terms (one sub-block)
    __shared__ f32x2 bcacc[kChunk][N];        // all channels of the workgroup

    const int c = blockIdx.y, b = blockIdx.z;
    const int d0 = blockIdx.x * CPG;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int t0 = c * kChunk;
    const int nt = (int)std::min<int64_t>(kChunk, p.L - t0);   // steps in this chunk
    const int g = d0 / p.dpg;                 // every channel of the workgroup is in one group
    const T *X = (const T *)p.x, *Dl = (const T *)p.delta, *Z = (const T *)p.z, *DY = (const T *)p.dy;

    // ---- stage per-step rows and per-(step, channel) quantities. Every load of a thread
    // is issued before any is used, with indices clamped into the chunk and D and an
    // absent bias read from A, so the latencies overlap instead of adding up per entry.
    constexpr int BCI = kChunk * N / NT;          // (step, n) entries per thread
    constexpr int PRI = kChunk * CPG / NT;        // (step, channel) pairs per thread
    static_assert(kChunk * N % NT == 0 && kChunk * CPG % NT == 0 && NT % CPG == 0, "entries tile the workgroup");
    {
        T braw[BCI], craw[BCI];
#pragma unroll
        for (int k = 0; k < BCI; ++k) {
            const int e = tid + k * NT, i = std::min(e / N, nt - 1), nn = e % N;
            const int64_t r = (((int64_t)b * p.L + t0 + i) * p.G + g) * N + nn;
            braw[k] = ((const T *)p.Bm)[r];
            craw[k] = ((const T *)p.Cm)[r];
        }
        const int cc = tid % CPG, dd = d0 + cc, ddc = std::min(dd, p.D - 1);
        const float *biasp = p.bias ? p.bias : p.A;
        const float biasv = biasp[ddc];
        const float bias = p.bias ? biasv : 0.0f;
        T xr[PRI], dr[PRI], yr[PRI], zr[PRI];
#pragma unroll
        for (int k = 0; k < PRI; ++k) {
            const int i = std::min(tid / CPG + k * (NT / CPG), nt - 1);
            const int64_t e = ((int64_t)b * p.L + t0 + i) * p.D + ddc;
            xr[k] = X[e];
            dr[k] = Dl[e];
            yr[k] = DY[e];
            if constexpr (HAS_Z) zr[k] = Z[e];
        }
#pragma unroll
        for (int k = 0; k < BCI; ++k) {
            const int e = tid + k * NT, i = e / N, nn = e % N;
            BC[i][nn] = i < nt ? f32x2{to_f32(braw[k]), to_f32(craw[k])} : f32x2{0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < PRI; ++k) {
            const int i = tid / CPG + k * (NT / CPG);
            f32x4 q = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < nt && dd < p.D) {
                const float xv = to_f32(xr[k]);
                const float vv = to_f32(dr[k]) + bias;
                const float dt = p.softplus ? softplus_f32(vv) : vv;
                float dyc = to_f32(yr[k]);
                if constexpr (HAS_Z) dyc *= silu_f32(to_f32(zr[k]));
                q = f32x4{dt, dt * xv, dyc, xv};
            }
            pre[i][cc] = q;
        }
    }
    __syncthreads();

    // ---- lane = (channel, n): recompute the chunk forward, then the adjoint backwards
    const int ch = wv * CPW + lane / N, n = lane % N;
    const int d = d0 + ch;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const float An = p.A[(int64_t)dc * N + n];
    const int64_t si = (((int64_t)b * p.nch + c) * p.D + dc) * N + n;
    const float hin = p.hin[si];
    float v = p.uin[si];
    float dAacc = 0.0f;
    sweep<N, CPG>(pre, BC, post, bcw, bcacc, ch, n, lane, wv, An, hin, v, dAacc);
    if (act) {
        if (c == 0 && p.dh0) p.dh0[((int64_t)b * p.D + d) * N + n] = v;
        // this chunk's share of dA, summed over (batch, chunk) by bwd_reduce_dA
        p.dApart[(((int64_t)b * p.nch + c) * p.D + d) * N + n] = dAacc;
    }
    __syncthreads();

    // ---- per (step, channel): dx, ddelta, dz; per-channel and per-row sums
    // Each thread takes EPI pairs of one channel. Every global value they need is loaded
    // before the first store: the memory counter completes in order, so a load placed
    // after a store could not be waited for without waiting for the store. Indices are
    // clamped into the chunk and D, and absent parameters read a valid stand-in (A), so
    // the loads are unconditional; the values of pairs outside are not used.
    constexpr int EPI = kChunk * CPG / NT;
    static_assert(kChunk * CPG % NT == 0 && NT % CPG == 0, "pairs tile the workgroup");
    {
        // The empty asm makes the epilogue's indices opaque, so their 64-bit addresses are
        // formed here rather than hoisted above the sweep, where they were spilled and each
        // load then waited on a scratch reload.
        int et = tid;
        asm volatile("" : "+v"(et));
        const int cc = et % CPG, dd = d0 + cc, ddc = std::min(dd, p.D - 1);
        const float *dskp = p.Dskip ? p.Dskip : p.A, *biasp = p.bias ? p.bias : p.A;
        const float dskv = dskp[ddc], biasv = biasp[ddc];
        const float dsk = p.Dskip ? dskv : 0.0f, bias = p.bias ? biasv : 0.0f;
        float dlv[EPI], zvv[EPI], dyv[EPI];
#pragma unroll
        for (int k = 0; k < EPI; ++k) {
            const int i = std::min(et / CPG + k * (NT / CPG), nt - 1);
            const int64_t e = ((int64_t)b * p.L + t0 + i) * p.D + ddc;
            dlv[k] = to_f32(Dl[e]);
            if constexpr (HAS_Z) {
                zvv[k] = to_f32(Z[e]);
                dyv[k] = to_f32(DY[e]);
            }
        }
#pragma unroll
        for (int k = 0; k < EPI; ++k) {
            const int i = et / CPG + k * (NT / CPG);
            if (i < nt && dd < p.D) {
                const int64_t e = ((int64_t)b * p.L + t0 + i) * p.D + dd;
                const f32x4 pr = pre[i][cc];
                const float dt = pr[0], dyc = pr[2], xv = pr[3];
                const float sB = post[1][i][cc], sA = post[2][i][cc];
                float gdl = fmaf(xv, sB, sA);                     // d dt
                if (p.softplus) gdl *= sigmoid_f32(dlv[k] + bias);
                store_val((T *)p.dx + e, fmaf(dyc, dsk, dt * sB));
                store_val((T *)p.ddelta + e, gdl);
                if constexpr (HAS_Z) {
                    const float zv = zvv[k], s = sigmoid_f32(zv);
                    const float dzf = dyv[k] * s * fmaf(zv, 1.0f - s, 1.0f);
                    store_val((T *)p.dz + e, dzf * fmaf(dsk, xv, post[0][i][cc]));
                }
                post[1][i][cc] = dyc * xv;                       // this pair's dDskip and dbias terms
                post[2][i][cc] = gdl;
            } else {
                post[1][i][cc] = 0.0f;
                post[2][i][cc] = 0.0f;
            }
        }
    }
    __syncthreads();
    for (int q = tid; q < nt * N; q += NT) {
        const int i = q / N, nn = q % N;
        const f32x2 acc = bcacc[i][nn];
        const int64_t r = (((int64_t)b * p.L + t0 + i) * p.G + g) * N + nn;
        atomicAdd(&p.dB[r], acc[0]);
        atomicAdd(&p.dC[r], acc[1]);
    }
    for (int q = tid; q < CPG; q += NT) {
        if (d0 + q < p.D) {
            float sd = 0.0f, sb = 0.0f;
            for (int i = 0; i < nt; ++i) {
                sd += post[1][i][q];
                sb += post[2][i][q];
            }
            if (p.dDskip) atomicAdd(&p.dDskip[d0 + q], sd);
            if (p.dbias) atomicAdd(&p.dbias[d0 + q], sb);
        }
    }
}

// dA[d, n] = sum over (batch, chunk) of the per-chunk shares
__global__ __launch_bounds__(256) void bwd_reduce_dA_kernel(const float *part, float *dA, int64_t dn, int64_t parts) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= dn) return;
    constexpr int U = 8;   // independent loads in flight
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.0f;
    int64_t k = 0;
    for (; k + U <= parts; k += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] += part[(k + u) * dn + i];
    }
    for (; k < parts; ++k) acc[0] += part[k * dn + i];
    float sum = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) sum += acc[u];
    dA[i] = sum;
}

__global__ __launch_bounds__(256) void fill_kernel(float *p, int64_t n, const float *src) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = src ? src[i] : 0.0f;
}

void fill(float *p, int64_t n, hipStream_t s, const float *src = nullptr) {
    if (p && n > 0) hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, src);
}

template <typename T, int N>
void launch_bwd(const BwdK &k, hipStream_t s) {
    const int chains = k.batch * k.dblocks;
    constexpr int CPG = kWaves * (64 / N);
    if (k.z) {
        hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, true>), dim3(chains, k.nch), dim3(64), 0, s, k);
    } else {
        hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, false>), dim3(chains, k.nch), dim3(64), 0, s, k);
    }
    hipLaunchKernelGGL((bwd_carry_kernel<N>), dim3(chains), dim3(64), 0, s, k);
    const dim3 grid((unsigned)((k.D + CPG - 1) / CPG), (unsigned)k.nch, (unsigned)k.batch);
    if (k.z)
        hipLaunchKernelGGL((bwd_main_kernel<T, N, true>), grid, dim3(kWaves * 64), 0, s, k);
    else
        hipLaunchKernelGGL((bwd_main_kernel<T, N, false>), grid, dim3(kWaves * 64), 0, s, k);
    const int64_t dn = (int64_t)k.D * N;
    hipLaunchKernelGGL(bwd_reduce_dA_kernel, dim3((unsigned)((dn + 255) / 256)), dim3(256), 0, s, k.dApart, k.dA,
                       dn, (int64_t)k.batch * k.nch);
}

}  // namespace

ssm_status scan_bwd_launch(const ssm_scan_bwd_args &a, const ScanBwdPlan &plan, hipStream_t s, char *err,
                           size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();
    const int64_t N = a.dstate;
    // outputs accumulated with atomics start from zero
    if (a.seqlen == 0) fill(a.dA, a.dim * N, s);
    fill(a.dDskip, a.dim, s);
    fill(a.ddelta_bias, a.dim, s);
    const int64_t G = a.ngroups > 1 ? a.ngroups : 1;
    fill(a.dB, a.batch * a.seqlen * G * N, s);
    fill(a.dC, a.batch * a.seqlen * G * N, s);
    if (a.seqlen == 0) {
        fill(a.dh0, a.batch * a.dim * N, s, a.dh_final);
    } else {
        BwdK k{};
        k.x = a.x; k.delta = a.delta; k.z = a.z; k.Bm = a.Bm; k.Cm = a.Cm; k.dy = a.dy;
        k.A = a.A; k.bias = a.delta_bias; k.Dskip = a.Dskip; k.h0 = a.h0; k.dh_final = a.dh_final;
        k.dx = a.dx; k.ddelta = a.ddelta; k.dz = a.dz;
        k.dB = a.dB; k.dC = a.dC; k.dA = a.dA; k.dDskip = a.dDskip; k.dbias = a.ddelta_bias; k.dh0 = a.dh0;
        char *ws = (char *)a.workspace;
        k.aggF = (float *)(ws + plan.aggF_offset);
        k.aggR = (float *)(ws + plan.aggR_offset);
        k.hin = (float *)(ws + plan.hin_offset);
        k.uin = (float *)(ws + plan.uin_offset);
        k.dApart = (float *)(ws + plan.dApart_offset);
        k.L = a.seqlen; k.D = (int32_t)a.dim; k.batch = (int32_t)a.batch; k.nch = (int32_t)plan.chunks;
        k.dblocks = (int32_t)((a.dim + 63) / 64);
        k.softplus = a.delta_softplus ? 1 : 0;
        k.G = (int32_t)G;
        k.dpg = (int32_t)(a.dim / G);
        const bool bf = a.dtype == SSM_BF16;
        switch (a.dstate) {
            case 16: bf ? launch_bwd<uint16_t, 16>(k, s) : launch_bwd<float, 16>(k, s); break;
            case 32: bf ? launch_bwd<uint16_t, 32>(k, s) : launch_bwd<float, 32>(k, s); break;
            default: bf ? launch_bwd<uint16_t, 64>(k, s) : launch_bwd<float, 64>(k, s); break;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(err, errlen, "selective_scan_bwd: kernel launch failed: %s", hipGetErrorString(e));
        return SSM_EHIP;
    }
    return SSM_OK;
}

}  // namespace ssm
