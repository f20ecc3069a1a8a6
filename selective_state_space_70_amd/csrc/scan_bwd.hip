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
//   2. bwd_carry: per (channel, n), sequential over chunks: h entering chunk c is
//      h0 carried through the maps h -> exp(A sum dt) o h + S; the adjoint entering
//      chunk c from the right is dh_final carried back through u -> exp(A sum dt) o u
//      + Q. Both are stored per (batch, chunk, n, channel);
//   3. bwd_main: per (chunk, 64 * 16 / N channels), one wave, lane = (channel, 16
//      states) so that the sums over n are in-lane, as in the forward scan: the
//      chunk is walked forwards from its entering state, then recomputed in
//      sub-blocks whose states stay in registers and swept backwards with the
//      adjoint. dB and dC (sums over the channels of a group) are reduced across
//      the wave by a butterfly and stored per (step, wave);
//   4. fixed-order sums of the per-wave and per-chunk partials (dB, dC, dA, dDskip,
//      ddelta_bias), so that every gradient is deterministic.
#include <algorithm>
#include <cstdio>

#include "device_common.h"
#include "internal.h"

namespace ssm {
namespace {

constexpr int kChunk = kScanBwdChunk;   // steps per chunk (states of a chunk live in VGPRs)

struct BwdK {
    const void *x, *delta, *z, *Bm, *Cm, *dy;
    const float *A, *bias, *Dskip, *h0, *dh_final;
    void *dx, *ddelta, *dz;
    float *dB, *dC, *dA, *dDskip, *dbias, *dh0;
    float *aggF;     // [chain][chunk][N+1][64]: end state from zero, then summed dt
    float *aggR;     // [chain][chunk][N][64]: adjoint aggregate
    float *hin;      // [batch][chunk][N][D]: state entering each chunk
    float *uin;      // [batch][chunk][N][D]: adjoint entering each chunk from the right
    float *dApart;   // [batch][chunk][D][N]: each chunk's share of dA
    float *dDpart;   // [batch][chunk][D]: each chunk's share of dDskip
    float *dbpart;   // [batch][chunk][D]: each chunk's share of ddelta_bias
    float *bcpart;   // [batch][L][nblk][2N]: per (step, wave) sums of dB_t (n < N), dC_t (n >= N);
                     // then one spare row that steps past the sequence store to
    int32_t *fast;   // [dblocks]: 1 where the 64 channels' rows of A are progressions
    int64_t L;
    int32_t D, batch, nch, dblocks, softplus, G, dpg;
    int32_t nblk;    // waves of the main kernel along D: ceil(D / (64 * 16 / N))
};

// Values made opaque at this point of the program (empty asm, no instruction): what
// produces them is computed before it.
template <int N>
__device__ __forceinline__ void tie16(float (&v)[N]) {
    static_assert(N % 16 == 0, "blocks of 16");
#pragma unroll
    for (int i = 0; i < N; i += 16)
        asm volatile("" : "+v"(v[i]), "+v"(v[i + 1]), "+v"(v[i + 2]), "+v"(v[i + 3]), "+v"(v[i + 4]),
                     "+v"(v[i + 5]), "+v"(v[i + 6]), "+v"(v[i + 7]), "+v"(v[i + 8]), "+v"(v[i + 9]),
                     "+v"(v[i + 10]), "+v"(v[i + 11]), "+v"(v[i + 12]), "+v"(v[i + 13]), "+v"(v[i + 14]),
                     "+v"(v[i + 15]));
}

// the same value, opaque to the optimiser (no instruction is emitted)
__device__ __forceinline__ float opaque_f32(float v) {
    asm volatile("" : "+v"(v));
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
    // softplus picked by a mask the optimiser cannot see through (no branch per step)
    uint32_t spm = p.softplus ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(spm));
    constexpr int U = 8;   // steps whose loads are issued together
    // the next block's loads are issued before the current block computes
    T xn[U], vn[U], yn[U], zn[U];
    auto load_block = [&](int tb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = ((int64_t)b * p.L + min(tb + u, t1 - 1)) * p.D + dc;
            xn[u] = X[e];
            vn[u] = Dl[e];
            yn[u] = DY[e];
            if constexpr (HAS_Z) zn[u] = Z[e];
        }
    };
    load_block(t0);
    for (int t = t0; t < t1; t += U) {
        float xs[U], vs[U], dys[U], zs[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xs[u] = to_f32(xn[u]);
            vs[u] = to_f32(vn[u]);
            dys[u] = to_f32(yn[u]);
            zs[u] = HAS_Z ? to_f32(zn[u]) : 0.0f;
        }
        if (t + U < t1) load_block(t + U);
        // per-step scalars of the block first (independent across steps, so their
        // exponentials and logarithms overlap); steps past the chunk are zeroed
        float dts[U], dtxs[U], dycs[U], rs[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float vm = t + u < t1 ? 1.0f : 0.0f;
            const float v = vs[u] + bias;
            const float sp = softplus_f32(v);
            dts[u] = __uint_as_float((__float_as_uint(sp) & spm) | (__float_as_uint(v) & ~spm)) * vm;
            float dyc = dys[u] * vm;
            if constexpr (HAS_Z) dyc *= silu_f32(zs[u]);
            dycs[u] = dyc;
            dtxs[u] = dts[u] * xs[u];
            rs[u] = FAST ? fast_exp2(dts[u] * Al2[0]) : 1.0f;
        }
        // then the state updates, one step (and its B, C rows in SGPRs) at a time
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tu = (int)opaque_u32((uint32_t)min(t + u, t1 - 1));
            float Bv[N], Cv[N];
            SharedRow<T, N>::load(Brow + (int64_t)tu * GN, Bv);
            SharedRow<T, N>::load(Crow + (int64_t)tu * GN, Cv);
            const float dt = dts[u], dtx = dtxs[u], dyc = dycs[u];
            dsum += dt;
            if constexpr (FAST) {
                const float r = rs[u];
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
            tie16(S);
            tie16(Q);
            __builtin_amdgcn_sched_barrier(0);
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
    const bool fast = __all(geometric_row<N>(p.A + (int64_t)dc * N));   // wave-uniform choice
    // which path these 64 channels take, for the main kernels
    if (b == 0 && c == 0 && threadIdx.x == 0) p.fast[chain] = fast ? 1 : 0;
    if (fast)
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
// One wave per (64 channels, state n): h0 carried forwards and dh_final backwards
// through the chunk maps, sequential over chunks. Each state is a chain of its own,
// so 64 / N times more waves are in flight than with a wave per 64 channels; the
// aggregates of kCarryK chunks are loaded together, so a wave waits for memory once
// per kCarryK chunks. The entering states are stored n-major, [batch][chunk][n][D],
// so that each store is one contiguous 256-byte row.
constexpr int kCarryK = 16;

template <int N>
__global__ __launch_bounds__(64) void bwd_carry_kernel(const BwdK p) {
    const int chain = blockIdx.x, n = blockIdx.y;
    const int b = chain / p.dblocks;
    const int d = (chain % p.dblocks) * 64 + threadIdx.x;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const float al2 = p.A[(int64_t)dc * N + n] * kLog2e;
    const int64_t ci = (int64_t)b * p.D + dc;
    const float *F = p.aggF + (size_t)chain * p.nch * (N + 1) * 64 + threadIdx.x;   // [chunk][N + 1][64]
    const float *Rg = p.aggR + (size_t)chain * p.nch * N * 64 + threadIdx.x;        // [chunk][N][64]
    const int64_t cstride = (int64_t)N * p.D;                                        // one chunk of hin / uin
    float *hin = p.hin + ((int64_t)b * p.nch * N + n) * p.D + dc;
    float *uin = p.uin + ((int64_t)b * p.nch * N + n) * p.D + dc;
    const int last = p.nch - 1;
    // Forwards, the state entering chunk c (chunk c < last maps h -> exp(A sum dt) h +
    // S_c), and backwards, the adjoint entering chunk c from the right (chunk c > 0
    // passes u -> exp(A sum dt) u + Q_c to chunk c - 1): two independent chains,
    // walked side by side so that their loads and latencies overlap.
    float h = p.h0 ? p.h0[ci * N + n] : 0.0f;
    float u = p.dh_final ? p.dh_final[ci * N + n] : 0.0f;
    for (int c0 = 0; c0 <= last; c0 += kCarryK) {
        float sv[kCarryK], df[kCarryK], qv[kCarryK], db[kCarryK];
#pragma unroll
        for (int k = 0; k < kCarryK; ++k) {
            const size_t cf = (size_t)min(c0 + k, last);       // clamped: loaded, not used
            const size_t cb = (size_t)max(last - c0 - k, 0);
            sv[k] = F[cf * (N + 1) * 64 + n * 64];
            df[k] = F[cf * (N + 1) * 64 + N * 64];
            qv[k] = Rg[cb * N * 64 + n * 64];
            db[k] = F[cb * (N + 1) * 64 + N * 64];
        }
#pragma unroll
        for (int k = 0; k < kCarryK; ++k) {
            const int cf = c0 + k, cb = last - c0 - k;
            if (cf > last) break;                              // uniform
            if (act) {
                hin[cf * cstride] = h;
                uin[cb * cstride] = u;
            }
            if (cf < last) h = fmaf(fast_exp2(al2 * df[k]), h, sv[k]);
            if (cb > 0) u = fmaf(fast_exp2(al2 * db[k]), u, qv[k]);
        }
    }
}

// ---------------------------------------------------------------- 3. main
// Lane = (channel, slice of 16 states): a lane keeps 16 states of one channel in
// VGPRs (N / 16 lanes per channel), as the forward scan does, so the sums over n
// (the readout, sum_n g B, sum_n A g a h) are in-lane. Per chunk:
//   * a forward walk from the entering state stores the state at every kSeg-th
//     step in LDS;
//   * then, last segment first, each sub-block of kSB steps is recomputed from
//     the state before it (the upper sub-block of a segment first walks the lower
//     one), its states kept in registers, and swept backwards with the adjoint.
// The recompute forms dC_t's per-lane terms dyc h_t, the readout and dz; the sweep
// forms g_t, dx, ddelta, dA and dB_t's terms g dt x. dB_t and dC_t are sums over
// the channels of a group: each is reduced across the wave's lanes by a butterfly
// (permlane swaps across rows, DPP within rows) and stored as one partial per
// (step, wave); bwd_reduce_bc_kernel adds the partials of a group in a fixed order.
// dA, dDskip and ddelta_bias are stored per chunk and summed the same way, so
// every gradient is deterministic.
constexpr int kSL = 16;                  // states per lane
constexpr int kSB = 8;                   // steps per sub-block
constexpr int kSeg = 2 * kSB;            // steps between stored states
constexpr int kNSeg = kChunk / kSeg;     // stored states per chunk (the first is the entering state)
static_assert(kChunk % kSeg == 0, "segments tile the chunk");

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
// a[l] + a[l ^ 32] in lanes l < 32, b[l] + b[l ^ 32] in lanes l >= 32
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const uint32_t u = r[0], w = r[1];
    return __uint_as_float(u) + __uint_as_float(w);
}
// a[l] + a[l ^ 16] in even rows of 16 lanes, b[l] + b[l ^ 16] in odd rows
__device__ __forceinline__ float swap16_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const uint32_t u = r[0], w = r[1];
    return __uint_as_float(u) + __uint_as_float(w);
}
// Within rows of 16: a[l] + a[l + k] where lane bit k is 0, b[l] + b[l - k] where it
// is 1 (row_shl:k reads lane l + k, row_shr:k lane l - k).
template <int K>
__device__ __forceinline__ float row_pair_sum(float a, float b, int lane) {
    const float lo = a + dpp<0x100 + K>(a);
    const float hi = b + dpp<0x110 + K>(b);
    return (lane & K) ? hi : lo;
}

// Sum of x[0..15] over the lanes of the wave that hold the same slice (the
// channels of the wave). Each halving step keeps, per lane, the half of the values
// selected by one lane bit and adds the partner lane's copy of that half: bits 5
// and 4 by permlane swaps, bits 3 and 2 within rows. Lane l returns value
// (l >> 2) & 15; lane bits 1 and 0, where they index channels, are added last.
template <int LPC>
__device__ __forceinline__ float chan_sum16(const float (&x)[kSL], int lane) {
    float y[8], z[4], w[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = swap32_sum(x[i], x[i + 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = swap16_sum(y[i], y[i + 4]);
#pragma unroll
    for (int i = 0; i < 2; ++i) w[i] = row_pair_sum<8>(z[i], z[i + 2], lane);
    float u = row_pair_sum<4>(w[0], w[1], lane);
    if constexpr (LPC <= 2) u += dpp<0x4E>(u);   // quad_perm [2,3,0,1]: lane bit 1
    if constexpr (LPC == 1) u += dpp<0xB1>(u);   // quad_perm [1,0,3,2]: lane bit 0
    return u;
}

// sum over the LPC lanes of one channel, in each of them
template <int LPC>
__device__ __forceinline__ float slice_sum(float v) {
    if constexpr (LPC >= 2) v += dpp<0xB1>(v);
    if constexpr (LPC >= 4) v += dpp<0x4E>(v);
    return v;
}

template <typename T, int N, bool HAS_Z, bool FAST>
__device__ __forceinline__ void bwd_chunk(const BwdK &p, float (*ck)[kSL][64], const int lane, const int b,
                                          const int c, const int blk) {
    constexpr int LPC = N / kSL;                 // lanes per channel
    constexpr int CPW = 64 / LPC;                // channels per wave
    const int s = lane % LPC;                    // slice: states 16 s .. 16 s + 15
    const int d = blk * CPW + lane / LPC;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int t0 = c * kChunk;
    const int tlast = (int)p.L - 1;
    const int g = __builtin_amdgcn_readfirstlane(blk * CPW) / p.dpg;   // the wave's group
    const int GN = p.G * N;
    const T *Brow = (const T *)p.Bm + ((int64_t)b * p.L * p.G + g) * N;
    const T *Crow = (const T *)p.Cm + ((int64_t)b * p.L * p.G + g) * N;
    const float *Arow = p.A + (int64_t)dc * N;
    const float A0 = Arow[0], A0l2 = A0 * kLog2e;
    float Al2[kSL];
    if constexpr (!FAST) {
#pragma unroll
        for (int i = 0; i < kSL; ++i) Al2[i] = Arow[s * kSL + i] * kLog2e;
    }
    const float bias = p.bias ? p.bias[dc] : 0.0f;
    const float dsk = p.Dskip ? p.Dskip[dc] : 0.0f;

    // (b, t, d) streams as raw buffers over batch row b: the time row is a uniform
    // byte offset, the lane adds its channel's offset. Stores from lanes that do not
    // own their channel's output (past D, or slices > 0) go to an offset past the
    // buffer, which the hardware drops.
    const int64_t base = (int64_t)b * p.L * p.D;
    const uint32_t bytes = (uint32_t)(p.L * p.D * (int64_t)sizeof(T));
    const rsrc_t xr = make_rsrc((const T *)p.x + base, bytes);
    const rsrc_t dr = make_rsrc((const T *)p.delta + base, bytes);
    const rsrc_t zr = make_rsrc(HAS_Z ? (const T *)p.z + base : (const T *)p.x + base, bytes);
    const rsrc_t yr = make_rsrc((const T *)p.dy + base, bytes);
    const rsrc_t dxr = make_rsrc((T *)p.dx + base, bytes);
    const rsrc_t ddr = make_rsrc((T *)p.ddelta + base, bytes);
    const rsrc_t dzr = make_rsrc(HAS_Z ? (T *)p.dz + base : (T *)p.dx + base, bytes);
    const uint32_t lo = (uint32_t)dc * sizeof(T);
    const uint32_t rowb = (uint32_t)p.D * sizeof(T);
    const uint32_t st_off = (act && s == 0) ? lo : 0x80000000u;
    // butterfly results: lane l holds state 16 s + ((l >> 2) & 15)
    const int wn = s * kSL + ((lane >> 2) & 15);
    float *bcp = p.bcpart + (size_t)blk * 2 * N + wn;   // + ((b L + t) nblk) 2N

    auto decays = [&](float dt, float (&a)[kSL]) {
        if constexpr (FAST) {
            powers_of<kSL>(fast_exp2(dt * A0l2), a);
            if constexpr (LPC > 1) {   // states 16 s + i decay by r^(16 s) r^(i+1)
                const float r16 = a[kSL - 1];
                float bs = (s & 1) ? r16 : 1.0f;
                if constexpr (LPC == 4) bs *= (s & 2) ? r16 * r16 : 1.0f;
#pragma unroll
                for (int i = 0; i < kSL; ++i) a[i] *= bs;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kSL; ++i) a[i] = fast_exp2(dt * Al2[i]);
        }
    };
    // The row offset passes through an empty asm statement at every use: loads from the
    // constant address space are invariant, and the recompute's and the sweep's loads
    // of one row would otherwise be merged and held in SGPRs across the sub-block.
    auto load_row16 = [&](const T *row, int t, float (&v)[kSL]) {
        const int64_t off = (int64_t)opaque_u32((uint32_t)min(t, tlast)) * GN;
        if constexpr (LPC == 1) {
            SharedRow<T, kSL>::load(row + off, v);
        } else {
            const T *q = row + off + s * kSL;
#pragma unroll
            for (int i = 0; i < kSL; ++i) v[i] = to_f32(q[i]);
        }
    };
    // No branch inside a step: a branch would split the step into blocks across which
    // the invariant row loads get hoisted (and the compiler turns a select of an
    // expensive value into one). softplus is always formed and picked by a bit mask
    // the optimiser cannot see through; steps past the sequence multiply by zero.
    uint32_t spm = p.softplus ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(spm));
    auto pick_sp = [&](float on, float off) {
        return __uint_as_float((__float_as_uint(on) & spm) | (__float_as_uint(off) & ~spm));
    };
    auto step_dt = [&](T draw, float vm) {
        const float v = to_f32(draw) + bias;
        return pick_sp(softplus_f32(v), v) * vm;
    };
    // x, delta of the 8 steps from tb (clamped into the sequence)
    auto load8 = [&](int tb, T (&xs)[kSB], T (&ds)[kSB]) {
        const uint32_t rb = opaque_u32(rowb);
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            const uint32_t so = (uint32_t)min(tb + u, tlast) * rb;
            buf_load(xr, lo, so, xs[u]);
            buf_load(dr, lo, so, ds[u]);
        }
    };
    // h <- the state after the 8 steps from tb: the steps' scalars first (independent
    // across steps, so their exponentials overlap), then the updates one step at a time
    auto adv8 = [&](int tb, const T (&xs)[kSB], const T (&ds)[kSB], float (&h)[kSL]) {
        float dts[kSB], dtxs[kSB];
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            dts[u] = step_dt(ds[u], tb + u <= tlast ? 1.0f : 0.0f);
            dtxs[u] = act ? dts[u] * to_f32(xs[u]) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            const int t = (int)opaque_u32((uint32_t)(tb + u));
            float a[kSL], Bv[kSL];
            decays(dts[u], a);
            load_row16(Brow, t, Bv);
#pragma unroll
            for (int i = 0; i < kSL; ++i) h[i] = fmaf(a[i], h[i], dtxs[u] * Bv[i]);
            tie16(h);   // the step's arithmetic stays in the step
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    float h[kSL], v[kSL], dA[kSL];
    {
        // n-major: each state's row of the wave's channels is contiguous
        const int64_t si = (((int64_t)b * p.nch + c) * N + s * kSL) * p.D + dc;
#pragma unroll
        for (int i = 0; i < kSL; ++i) {
            h[i] = p.hin[si + (int64_t)i * p.D];
            v[i] = p.uin[si + (int64_t)i * p.D];
            dA[i] = 0.0f;
        }
    }
    float dD = 0.0f, dbias = 0.0f;

    // ---- forward walk: the state at the start of every segment, into LDS
    {
        T xa[kSB], da[kSB], xb[kSB], db[kSB];
        load8(t0, xa, da);
#pragma unroll
        for (int i = 0; i < kSL; ++i) ck[0][i][lane] = h[i];
#pragma unroll
        for (int k = 1; k < kNSeg; ++k) {
            load8(t0 + kSeg * (k - 1) + kSB, xb, db);
            adv8(t0 + kSeg * (k - 1), xa, da, h);
            if (k + 1 < kNSeg) load8(t0 + kSeg * k, xa, da);
            adv8(t0 + kSeg * (k - 1) + kSB, xb, db, h);
#pragma unroll
            for (int i = 0; i < kSL; ++i) ck[k][i][lane] = h[i];
        }
    }

    // ---- one sub-block of kSB steps from tb, entered with state hs: recompute, then sweep
    auto sub_block = [&](int tb, const float (&hs)[kSL]) {
        float sdt[kSB], sx[kSB], sdyc[kSB], spd[kSB], sdz[kSB];
        {
            T xs[kSB], ds[kSB], zs[kSB], ys[kSB];
            const uint32_t rb = opaque_u32(rowb);
#pragma unroll
            for (int u = 0; u < kSB; ++u) {
                const uint32_t so = (uint32_t)min(tb + u, tlast) * rb;
                buf_load(xr, lo, so, xs[u]);
                buf_load(dr, lo, so, ds[u]);
                buf_load(yr, lo, so, ys[u]);
                if constexpr (HAS_Z) buf_load(zr, lo, so, zs[u]);
            }
#pragma unroll
            for (int u = 0; u < kSB; ++u) {
                const float vm = tb + u <= tlast ? 1.0f : 0.0f;
                const float vv = to_f32(ds[u]) + bias;
                sdt[u] = pick_sp(softplus_f32(vv), vv) * vm;
                spd[u] = pick_sp(sigmoid_f32(vv), 1.0f);
                sx[u] = to_f32(xs[u]);
                const float dyv = to_f32(ys[u]);
                float dyc = dyv;
                sdz[u] = 0.0f;
                if constexpr (HAS_Z) {
                    const float zv = to_f32(zs[u]), sg = sigmoid_f32(zv);
                    dyc = dyv * zv * sg;
                    sdz[u] = dyv * sg * fmaf(zv, 1.0f - sg, 1.0f);
                }
                sdyc[u] = dyc * (act ? vm : 0.0f);
            }
        }
        // recompute: states of the sub-block, dC terms, readout, dz
        float hb[kSB + 1][kSL];
#pragma unroll
        for (int i = 0; i < kSL; ++i) hb[0][i] = hs[i];
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            const int t = (int)opaque_u32((uint32_t)(tb + u));   // per-step offsets formed in the step
            float a[kSL], Bv[kSL], Cv[kSL];
            decays(sdt[u], a);
            load_row16(Brow, t, Bv);
            load_row16(Crow, t, Cv);
            const float dtx = act ? sdt[u] * sx[u] : 0.0f;
            float dcv[kSL], yc = 0.0f;
#pragma unroll
            for (int i = 0; i < kSL; ++i) {
                hb[u + 1][i] = fmaf(a[i], hb[u][i], dtx * Bv[i]);
                dcv[i] = sdyc[u] * hb[u + 1][i];
                yc = fmaf(Cv[i], hb[u + 1][i], yc);
            }
            const float dCt = chan_sum16<LPC>(dcv, lane);
            const bool valid = t <= tlast;
            // a step past the sequence stores to the spare row after the last batch row;
            // lanes that hold the same value store the same value
            bcp[(valid ? (int64_t)b * p.L + t : (int64_t)p.batch * p.L) * p.nblk * 2 * N + N] = dCt;
            dD = fmaf(sdyc[u], sx[u], dD);
            if constexpr (HAS_Z) {
                yc = slice_sum<LPC>(yc);
                const float dzv = sdz[u] * fmaf(dsk, sx[u], yc);
                if constexpr (sizeof(T) == 2)
                    buf_store(dzr, valid ? st_off : 0x80000000u, (uint32_t)min(t, tlast) * rowb, f32_to_bf16(dzv));
                else
                    buf_store(dzr, valid ? st_off : 0x80000000u, (uint32_t)min(t, tlast) * rowb, dzv);
            }
            tie16(hb[u + 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // sweep backwards
#pragma unroll
        for (int u = kSB - 1; u >= 0; --u) {
            const int t = (int)opaque_u32((uint32_t)(tb + u));   // per-step offsets formed in the step
            float a[kSL], Bv[kSL], Cv[kSL];
            // the decays are formed again (not kept from the recompute: 16 registers per step)
            const float dt = opaque_f32(sdt[u]), dyc = sdyc[u];
            decays(dt, a);
            load_row16(Brow, t, Bv);
            load_row16(Crow, t, Cv);
            const float dtx = act ? dt * sx[u] : 0.0f;
            float dbv[kSL], sB = 0.0f, sA = 0.0f, sM = 0.0f;
#pragma unroll
            for (int i = 0; i < kSL; ++i) {
                const float gq = fmaf(Cv[i], dyc, v[i]);   // g_t
                sB = fmaf(gq, Bv[i], sB);
                dbv[i] = gq * dtx;
                const float w = gq * a[i];
                const float m = w * hb[u][i];               // g_t a_t h_{t-1}
                dA[i] = fmaf(dt, m, dA[i]);
                if constexpr (FAST) {
                    sA = fmaf((float)(i + 1), m, sA);
                    if constexpr (LPC > 1) sM += m;
                } else {
                    sA = fmaf(Al2[i], m, sA);
                }
                v[i] = w;                                   // adjoint term carried to t - 1
            }
            if constexpr (FAST) {
                if constexpr (LPC > 1) sA = fmaf((float)(s * kSL), sM, sA);
                sA *= A0;
            } else {
                sA *= kLn2;
            }
            sB = slice_sum<LPC>(sB);
            sA = slice_sum<LPC>(sA);
            const float dBt = chan_sum16<LPC>(dbv, lane);
            const bool valid = t <= tlast;
            bcp[(valid ? (int64_t)b * p.L + t : (int64_t)p.batch * p.L) * p.nblk * 2 * N] = dBt;
            const float dxv = fmaf(dt, sB, dsk * dyc);
            const float ddl = fmaf(sx[u], sB, sA) * spd[u];
            dbias += valid ? ddl : 0.0f;
            const uint32_t so = (uint32_t)min(t, tlast) * rowb, vo = valid ? st_off : 0x80000000u;
            if constexpr (sizeof(T) == 2) {
                buf_store(dxr, vo, so, f32_to_bf16(dxv));
                buf_store(ddr, vo, so, f32_to_bf16(ddl));
            } else {
                buf_store(dxr, vo, so, dxv);
                buf_store(ddr, vo, so, ddl);
            }
            tie16(v);
            tie16(dA);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- backward over the segments, last first
#pragma unroll 1
    for (int k = kNSeg - 1; k >= 0; --k) {
        const int ts = t0 + kSeg * k;
        if (ts > tlast) continue;                       // uniform: segment past the sequence
        float hs[kSL];
#pragma unroll
        for (int i = 0; i < kSL; ++i) hs[i] = ck[k][i][lane];
        if (ts + kSB <= tlast) {                        // the upper sub-block has steps
            T xs[kSB], ds[kSB];
            load8(ts, xs, ds);
            float hm[kSL];
#pragma unroll
            for (int i = 0; i < kSL; ++i) hm[i] = hs[i];
            adv8(ts, xs, ds, hm);
            sub_block(ts + kSB, hm);
        }
        sub_block(ts, hs);
    }

    if (act && c == 0 && p.dh0) {
        float *o = p.dh0 + ((int64_t)b * p.D + d) * N + s * kSL;
#pragma unroll
        for (int i = 0; i < kSL; ++i) o[i] = v[i];
    }
    if (act) {
        float *o = p.dApart + (((int64_t)b * p.nch + c) * p.D + d) * N + s * kSL;
#pragma unroll
        for (int i = 0; i < kSL; ++i) o[i] = dA[i];
        if (s == 0) {
            const int64_t q = ((int64_t)b * p.nch + c) * p.D + d;
            p.dDpart[q] = dD;
            p.dbpart[q] = dbias;
        }
    }
}

// One launch per path: a wave whose 64 channels all have progression rows of A runs
// in the FAST launch, any other wave in the general one (each launch's waves of the
// other kind return at once), so each path gets its own register allocation.
template <typename T, int N, bool HAS_Z, bool FAST>
__global__ __launch_bounds__(64, FAST ? 2 : 1) void bwd_main_kernel(const BwdK p) {
    __shared__ float ck[kNSeg][kSL][64];          // the state at the start of each segment
    const int lane = threadIdx.x;
    const int blk = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
    constexpr int CPW = 64 * kSL / N;
    if ((p.fast[(blk * CPW) / 64] != 0) != FAST) return;   // the aggregate kernel's choice
    bwd_chunk<T, N, HAS_Z, FAST>(p, ck, lane, b, c, blk);
}

// dB, dC of (batch, step, group): the partials of the group's waves, added in order
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float *part, float *dB, float *dC, int64_t total,
                                                            int nblk, int G, int bpg, int N) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
        const int two_n = 2 * N;
        const int idx = (int)(i % two_n);
        const int64_t rest = i / two_n;
        const int g = (int)(rest % G);
        const int64_t row = rest / G;              // b L + t
        const float *q = part + (row * nblk + (int64_t)g * bpg) * two_n + idx;
        float acc = 0.0f;
        for (int k = 0; k < bpg; ++k) acc += q[(int64_t)k * two_n];
        const int n = idx < N ? idx : idx - N;
        (idx < N ? dB : dC)[(row * G + g) * N + n] = acc;
    }
}

// out_j[i] = sum over k < parts of part_j[k dn_j + i] for up to three arrays j (dA, dDskip,
// ddelta_bias from their per-(batch, chunk) shares). A block takes 32 columns; its 8 rows
// of threads each sum every 8th share, and row 0 adds the 8 results in order.
struct ColSums {
    const float *part[3];
    float *out[3];
    int64_t dn[3];
    int64_t parts;
};
constexpr int kColW = 32, kColR = 8;
__global__ __launch_bounds__(kColW * kColR) void bwd_colsum_kernel(const ColSums cs) {
    __shared__ float acc[kColR][kColW];
    const int j = blockIdx.y;
    const int cx = threadIdx.x % kColW, r = threadIdx.x / kColW;
    const int64_t dn = cs.dn[j];
    const int64_t i = (int64_t)blockIdx.x * kColW + cx;
    const float *part = cs.part[j] + (i < dn ? i : 0);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    if (i < dn) {
        int64_t k = r;
        for (; k + 3 * kColR < cs.parts; k += 4 * kColR) {
            s0 += part[k * dn];
            s1 += part[(k + kColR) * dn];
            s2 += part[(k + 2 * kColR) * dn];
            s3 += part[(k + 3 * kColR) * dn];
        }
        for (; k < cs.parts; k += kColR) s0 += part[k * dn];
    }
    acc[r][cx] = (s0 + s1) + (s2 + s3);
    __syncthreads();
    if (r == 0 && i < dn) {
        float t = 0.0f;
#pragma unroll
        for (int q = 0; q < kColR; ++q) t += acc[q][cx];
        cs.out[j][i] = t;
    }
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
    if (k.z) {
        hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, true>), dim3(chains, k.nch), dim3(64), 0, s, k);
    } else {
        hipLaunchKernelGGL((bwd_aggregate_kernel<T, N, false>), dim3(chains, k.nch), dim3(64), 0, s, k);
    }
    hipLaunchKernelGGL((bwd_carry_kernel<N>), dim3(chains, N), dim3(64), 0, s, k);
    const dim3 grid((unsigned)k.nblk, (unsigned)k.nch, (unsigned)k.batch);
    if (k.z) {
        hipLaunchKernelGGL((bwd_main_kernel<T, N, true, true>), grid, dim3(64), 0, s, k);
        hipLaunchKernelGGL((bwd_main_kernel<T, N, true, false>), grid, dim3(64), 0, s, k);
    } else {
        hipLaunchKernelGGL((bwd_main_kernel<T, N, false, true>), grid, dim3(64), 0, s, k);
        hipLaunchKernelGGL((bwd_main_kernel<T, N, false, false>), grid, dim3(64), 0, s, k);
    }
    ColSums cs{};
    int nj = 0;
    auto add = [&](const float *part, float *out, int64_t dn) {
        if (!out) return;
        cs.part[nj] = part;
        cs.out[nj] = out;
        cs.dn[nj] = dn;
        ++nj;
    };
    add(k.dApart, k.dA, (int64_t)k.D * N);
    add(k.dDpart, k.dDskip, k.D);
    add(k.dbpart, k.dbias, k.D);
    cs.parts = (int64_t)k.batch * k.nch;
    hipLaunchKernelGGL(bwd_colsum_kernel, dim3((unsigned)(((int64_t)k.D * N + kColW - 1) / kColW), nj),
                       dim3(kColW * kColR), 0, s, cs);
    constexpr int CPW = 64 * kSL / N;
    const int bpg = k.G > 1 ? k.dpg / CPW : k.nblk;
    const int64_t total = (int64_t)k.batch * k.L * k.G * 2 * N;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 1 << 20);
    hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3((unsigned)blocks), dim3(256), 0, s, k.bcpart, k.dB, k.dC, total,
                       k.nblk, k.G, bpg, N);
}

}  // namespace

ssm_status scan_bwd_launch(const ssm_scan_bwd_args &a, const ScanBwdPlan &plan, hipStream_t s, char *err,
                           size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();
    const int64_t N = a.dstate;
    const int64_t G = a.ngroups > 1 ? a.ngroups : 1;
    if (a.seqlen == 0) {
        // no step: the parameter gradients are zero and dh0 is dh_final
        fill(a.dA, a.dim * N, s);
        fill(a.dDskip, a.dim, s);
        fill(a.ddelta_bias, a.dim, s);
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
        k.dDpart = (float *)(ws + plan.dDpart_offset);
        k.dbpart = (float *)(ws + plan.dbpart_offset);
        k.bcpart = (float *)(ws + plan.bcpart_offset);
        k.fast = (int32_t *)(ws + plan.fast_offset);
        k.L = a.seqlen; k.D = (int32_t)a.dim; k.batch = (int32_t)a.batch; k.nch = (int32_t)plan.chunks;
        k.dblocks = (int32_t)((a.dim + 63) / 64);
        k.softplus = a.delta_softplus ? 1 : 0;
        k.G = (int32_t)G;
        k.dpg = (int32_t)(a.dim / G);
        k.nblk = (int32_t)((a.dim + 64 * kSL / N - 1) / (64 * kSL / N));
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
