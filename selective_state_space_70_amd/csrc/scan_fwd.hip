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

#include "chain.h"
#include "device_common.h"
#include "internal.h"

namespace ssm {
namespace {

struct ScanK {
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *bias, *Dskip, *h0;
    void *y;
    float *h_final;
    float *agg;       // [chains][G-1][N+1][64]: end state from zero, then summed step
    int64_t L;
    int64_t chunk_len;
    int32_t D;
    int32_t batch;
    int32_t chunks;     // G
    int32_t dblocks;    // ceil(D / 64)
    int32_t softplus;
    int32_t G;          // groups of B, C
    int32_t dpg;        // channels per group (a multiple of 64 when G > 1)
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

// Words per B/C row: bf16 rows pack two states per dword.
template <typename T, int N>
struct RowWords { static constexpr int value = sizeof(T) == 2 ? N / 2 : N; };

template <typename T, int N>
__device__ __forceinline__ void load_row(cu32 *row, uint32_t (&w)[RowWords<T, N>::value]) {
#pragma unroll
    for (int j = 0; j < RowWords<T, N>::value; ++j) w[j] = row[j];
}

template <typename T, int N>
__device__ __forceinline__ void unpack_row(const uint32_t (&w)[RowWords<T, N>::value], float (&v)[N]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            v[2 * j] = bf16_lo(w[j]);
            v[2 * j + 1] = bf16_hi(w[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) v[j] = __uint_as_float(w[j]);
    }
}

// Per-channel constants of one call.
template <int N>
struct Chan {
    float Al2[N];    // A[d, n] * log2(e)
    float bias, dsk;
};

// One step with readout: h <- exp(dt A) h + dt B x; y = (C.h + D x) silu(z).
template <typename T, int N, bool FAST, bool HAS_Z>
__device__ __forceinline__ void step_readout(const Chan<N> &c, bool softplus, T xraw, T draw, T zraw,
                                             const uint32_t (&bw)[RowWords<T, N>::value],
                                             const uint32_t (&cw)[RowWords<T, N>::value],
                                             float (&h)[N], rsrc_t yr, uint32_t lo, uint32_t soff,
                                             bool act) {
    const float xv = to_f32(xraw);
    const float v = to_f32(draw) + c.bias;
    const float dt = softplus ? softplus_f32(v) : v;
    const float dtx = dt * xv;
    float a[N];
    if constexpr (FAST) {
        powers<N>(fast_exp2(dt * c.Al2[0]), a);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) a[n] = fast_exp2(dt * c.Al2[n]);
    }
    float Bv[N], Cv[N];
    unpack_row<T, N>(bw, Bv);
    unpack_row<T, N>(cw, Cv);
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = fmaf(a[n], h[n], Bv[n] * dtx);
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int n = 0; n < N; n += 2) {
        acc0 = fmaf(Cv[n], h[n], acc0);
        acc1 = fmaf(Cv[n + 1], h[n + 1], acc1);
    }
    float yv = fmaf(c.dsk, xv, acc0 + acc1);
    if constexpr (HAS_Z) yv *= silu_f32(to_f32(zraw));
    // Unconditional: a lane past D stores at an offset beyond the buffer's range, which
    // the hardware drops. With no branch around the stores the compiler knows how many
    // are in flight, so waiting for the next block's loads does not wait for them.
    const uint32_t voff = act ? lo : 0x80000000u;
    if constexpr (sizeof(T) == 2)
        buf_store(yr, voff, soff, f32_to_bf16(yv));
    else
        buf_store(yr, voff, soff, yv);
}

// Forward pass over [t0, t1) with readout. x/delta/z of the next block of U steps
// are loaded while the current block computes (their latency is hidden behind
// U steps of arithmetic); B/C rows are fetched one step ahead into SGPRs.
// Addresses: the time row is a wave-uniform pointer (SGPRs), the lane adds a
// fixed element offset, so no per-step vector address arithmetic is needed.
template <typename T, int N, bool FAST, bool HAS_Z>
__device__ __forceinline__ void run_readout(const ScanK &p, int b, int dc, bool act, int t0, int t1,
                                            float (&h)[N], const Chan<N> &c) {
    constexpr int U = 8;
    constexpr int NW = RowWords<T, N>::value;
    const int64_t base = ((int64_t)b * p.L) * p.D;
    const uint32_t bytes = (uint32_t)(p.L * p.D * (int64_t)sizeof(T));
    const rsrc_t xr = make_rsrc((const T *)p.x + base, bytes);
    const rsrc_t dr = make_rsrc((const T *)p.delta + base, bytes);
    const rsrc_t zr = make_rsrc(HAS_Z ? (const T *)p.z + base : (const T *)p.x + base, bytes);
    const rsrc_t yr = make_rsrc((T *)p.y + base, bytes);
    const uint32_t lo = (uint32_t)dc * sizeof(T);         // lane byte offset
    const uint32_t rowb = (uint32_t)p.D * sizeof(T);      // bytes per time step
    // the wave's group of B, C rows (every channel of a wave is in one group)
    const int g = __builtin_amdgcn_readfirstlane(dc) / p.dpg;
    const int GN = p.G * N;                               // elements per time step (< 2^31 / L)
    const T *Brow = (const T *)p.Bm + ((int64_t)b * p.L * p.G + g) * N;
    const T *Crow = (const T *)p.Cm + ((int64_t)b * p.L * p.G + g) * N;
    const bool softplus = p.softplus != 0;

    uint32_t bw[NW], cw[NW];
    load_row<T, N>(as_const(Brow + t0 * GN), bw);
    load_row<T, N>(as_const(Crow + t0 * GN), cw);

    int t = t0;
    if (t1 - t0 >= U) {
        T xa[U], da[U], za[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t so = (uint32_t)(t + u) * rowb;
            buf_load(xr, lo, so, xa[u]);
            buf_load(dr, lo, so, da[u]);
            if constexpr (HAS_Z) buf_load(zr, lo, so, za[u]);
        }
        for (; t + U <= t1; t += U) {
            // next block, clamped to the last step so every read stays in bounds
            T xb[U], db[U], zb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t so = (uint32_t)min(t + U + u, t1 - 1) * rowb;
                buf_load(xr, lo, so, xb[u]);
                buf_load(dr, lo, so, db[u]);
                if constexpr (HAS_Z) buf_load(zr, lo, so, zb[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t bn[NW], cn[NW];
                const int rn = min(t + u + 1, t1 - 1) * GN;
                load_row<T, N>(as_const(Brow + rn), bn);
                load_row<T, N>(as_const(Crow + rn), cn);
                step_readout<T, N, FAST, HAS_Z>(c, softplus, xa[u], da[u], HAS_Z ? za[u] : xa[u],
                                                bw, cw, h, yr, lo, (uint32_t)(t + u) * rowb, act);
#pragma unroll
                for (int j = 0; j < NW; ++j) { bw[j] = bn[j]; cw[j] = cn[j]; }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xa[u] = xb[u];
                da[u] = db[u];
                if constexpr (HAS_Z) za[u] = zb[u];
            }
        }
        // tail of fewer than U steps: their rows are already in xa (the last
        // prefetch clamps to t1 - 1)
#pragma unroll
        for (int u = 0; u < U - 1; ++u) {
            if (t + u < t1) {
                uint32_t bn[NW], cn[NW];
                const int rn = min(t + u + 1, t1 - 1) * GN;
                load_row<T, N>(as_const(Brow + rn), bn);
                load_row<T, N>(as_const(Crow + rn), cn);
                step_readout<T, N, FAST, HAS_Z>(c, softplus, xa[u], da[u], HAS_Z ? za[u] : xa[u],
                                                bw, cw, h, yr, lo, (uint32_t)(t + u) * rowb, act);
#pragma unroll
                for (int j = 0; j < NW; ++j) { bw[j] = bn[j]; cw[j] = cn[j]; }
            }
        }
        t = t1;
    }
    for (; t < t1; ++t) {  // a chunk shorter than U steps
        uint32_t bn[NW], cn[NW];
        const int rn = min(t + 1, t1 - 1) * GN;
        load_row<T, N>(as_const(Brow + rn), bn);
        load_row<T, N>(as_const(Crow + rn), cn);
        const uint32_t so = (uint32_t)t * rowb;
        T xv, dv, zv;
        buf_load(xr, lo, so, xv);
        buf_load(dr, lo, so, dv);
        if constexpr (HAS_Z) buf_load(zr, lo, so, zv); else zv = xv;
        step_readout<T, N, FAST, HAS_Z>(c, softplus, xv, dv, zv, bw, cw, h, yr, lo, so, act);
#pragma unroll
        for (int j = 0; j < NW; ++j) { bw[j] = bn[j]; cw[j] = cn[j]; }
    }
}

// End state of [t0, t1) from a zero state, and the summed step, walking time
// backwards: with R = prod_{k>t} exp(dt_k A[0]) the fast path adds
// B_t[n] * dt_t x_t * R^(n+1) to S[n], i.e. one multiply and one FMA per state
// (the decay of everything after t is applied once, as a power of R). The
// general path runs the recurrence forwards.
template <typename T, int N, bool FAST>
__device__ __forceinline__ double run_aggregate(const ScanK &p, int b, int dc, int t0, int t1,
                                                float (&S)[N], const Chan<N> &c) {
    constexpr int U = 8;
    constexpr int NW = RowWords<T, N>::value;
    const int64_t base = ((int64_t)b * p.L) * p.D;
    const uint32_t bytes = (uint32_t)(p.L * p.D * (int64_t)sizeof(T));
    const rsrc_t xr = make_rsrc((const T *)p.x + base, bytes);
    const rsrc_t dr = make_rsrc((const T *)p.delta + base, bytes);
    const uint32_t lo = (uint32_t)dc * sizeof(T);
    const uint32_t rowb = (uint32_t)p.D * sizeof(T);
    const int g = __builtin_amdgcn_readfirstlane(dc) / p.dpg;
    const int GN = p.G * N;
    const T *Brow = (const T *)p.Bm + ((int64_t)b * p.L * p.G + g) * N;
    const bool softplus = p.softplus != 0;
    double dsum = 0.0;
    float R = 1.0f;

    auto one = [&](T xraw, T draw, const uint32_t (&bw)[NW]) {
        const float xv = to_f32(xraw);
        const float v = to_f32(draw) + c.bias;
        const float dt = softplus ? softplus_f32(v) : v;
        const float dtx = dt * xv;
        float Bv[N];
        unpack_row<T, N>(bw, Bv);
        dsum += (double)dt;
        if constexpr (FAST) {
            float q = R * dtx;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                S[n] = fmaf(Bv[n], q, S[n]);
                q *= R;
            }
            R *= fast_exp2(dt * c.Al2[0]);
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) S[n] = fmaf(fast_exp2(dt * c.Al2[n]), S[n], Bv[n] * dtx);
        }
    };

    if constexpr (FAST) {
        // backwards in time
        int t = t1 - 1;
        uint32_t bw[NW];
        load_row<T, N>(as_const(Brow + t * GN), bw);
        if (t - t0 + 1 >= U) {
            T xa[U], da[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t so = (uint32_t)(t - u) * rowb;
                buf_load(xr, lo, so, xa[u]);
                buf_load(dr, lo, so, da[u]);
            }
            for (; t - U + 1 >= t0; t -= U) {
                T xb[U], db[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t so = (uint32_t)max(t - U - u, t0) * rowb;
                    buf_load(xr, lo, so, xb[u]);
                    buf_load(dr, lo, so, db[u]);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    uint32_t bn[NW];
                    load_row<T, N>(as_const(Brow + max(t - u - 1, t0) * GN), bn);
                    one(xa[u], da[u], bw);
#pragma unroll
                    for (int j = 0; j < NW; ++j) bw[j] = bn[j];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) { xa[u] = xb[u]; da[u] = db[u]; }
            }
            // the first t - t0 + 1 < U steps of the chunk: already in xa (the last
            // prefetch clamps to t0)
#pragma unroll
            for (int u = 0; u < U - 1; ++u) {
                if (t - u >= t0) {
                    uint32_t bn[NW];
                    load_row<T, N>(as_const(Brow + max(t - u - 1, t0) * GN), bn);
                    one(xa[u], da[u], bw);
#pragma unroll
                    for (int j = 0; j < NW; ++j) bw[j] = bn[j];
                }
            }
            t = t0 - 1;
        }
        for (; t >= t0; --t) {
            uint32_t bn[NW];
            load_row<T, N>(as_const(Brow + max(t - 1, t0) * GN), bn);
            T xv, dv;
            buf_load(xr, lo, (uint32_t)t * rowb, xv);
            buf_load(dr, lo, (uint32_t)t * rowb, dv);
            one(xv, dv, bw);
#pragma unroll
            for (int j = 0; j < NW; ++j) bw[j] = bn[j];
        }
    } else {
        for (int t = t0; t < t1; ++t) {
            uint32_t bw[NW];
            load_row<T, N>(as_const(Brow + t * GN), bw);
            T xv, dv;
            buf_load(xr, lo, (uint32_t)t * rowb, xv);
            buf_load(dr, lo, (uint32_t)t * rowb, dv);
            one(xv, dv, bw);
        }
    }
    return dsum;
}

template <int N>
__device__ __forceinline__ Chan<N> load_chan(const ScanK &p, int dc) {
    Chan<N> c;
    const float *Arow = p.A + (int64_t)dc * N;
#pragma unroll
    for (int n = 0; n < N; ++n) c.Al2[n] = Arow[n] * kLog2e;
    c.bias = p.bias ? p.bias[dc] : 0.0f;
    c.dsk = p.Dskip ? p.Dskip[dc] : 0.0f;
    return c;
}

// exp(A[d, n] * s) for all n (the decay a chunk with summed step s applies).
template <int N, bool FAST>
__device__ __forceinline__ void chunk_decay(const Chan<N> &c, float s, float (&P)[N]) {
    if constexpr (FAST) {
        powers<N>(fast_exp2(c.Al2[0] * s), P);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) P[n] = fast_exp2(c.Al2[n] * s);
    }
}

// Pass 1: the end state of chunk k (k < G-1) from a zero state and its summed
// step, stored for the chunks after it (layout [chain][k][n][lane]: one
// contiguous 256-byte row per state index).
template <typename T, int N>
__global__ __launch_bounds__(64) void scan_chunk_state_kernel(const ScanK p) {
    const ChainSlot slot = chain_slot(p.batch * p.dblocks, p.chunks - 1);
    if (!slot.valid) return;
    const int b = slot.chain / p.dblocks;
    const int d = (slot.chain % p.dblocks) * 64 + threadIdx.x;
    const int dc = d < p.D ? d : p.D - 1;
    const int k = slot.pos;
    const int t0 = (int)((int64_t)k * p.chunk_len);
    const int t1 = (int)min(p.L, (int64_t)t0 + p.chunk_len);
    const Chan<N> c = load_chan<N>(p, dc);
    float S[N];
#pragma unroll
    for (int n = 0; n < N; ++n) S[n] = 0.0f;
    // wave-uniform choice of the exact fast path
    const double ds = __all(row_is_geometric<N>(p.A + (int64_t)dc * N))
                          ? run_aggregate<T, N, true>(p, b, dc, t0, t1, S, c)
                          : run_aggregate<T, N, false>(p, b, dc, t0, t1, S, c);
    float *a = p.agg + ((size_t)slot.chain * (p.chunks - 1) + k) * (N + 1) * 64 + threadIdx.x;
#pragma unroll
    for (int n = 0; n < N; ++n) a[n * 64] = S[n];
    a[N * 64] = (float)ds;
}

// State entering chunk k: h0 (or zero) carried through chunks 0..k-1 by their
// affine maps h -> exp(A sum dt) o h + S_j, in order. The aggregates of one chain
// were written by workgroups on the same XCD, so these reads hit its L2; the loads
// of a group of chunks are issued together.
template <int N, bool FAST>
__device__ __forceinline__ void enter_state(const ScanK &p, const Chan<N> &c, int chain, int k,
                                            float (&h)[N]) {
    constexpr int K = 4;
    const float *a0 = p.agg + (size_t)chain * (p.chunks - 1) * (N + 1) * 64 + threadIdx.x;
    for (int j0 = 0; j0 < k; j0 += K) {
        float S[K][N], ds[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const float *a = a0 + (size_t)min(j0 + u, k - 1) * (N + 1) * 64;
#pragma unroll
            for (int n = 0; n < N; ++n) S[u][n] = a[n * 64];
            ds[u] = a[N * 64];
        }
#pragma unroll
        for (int u = 0; u < K; ++u) {
            if (j0 + u < k) {
                float P[N];
                chunk_decay<N, FAST>(c, ds[u], P);
#pragma unroll
                for (int n = 0; n < N; ++n) h[n] = fmaf(P[n], h[n], S[u][n]);
            }
        }
    }
}

// Pass 2: every chunk from its entering state, with readout, gate and store; the
// last chunk writes h_final.
template <typename T, int N, bool HAS_Z, bool FAST>
__device__ __forceinline__ void scan_chunk(const ScanK &p, const Chan<N> &c, int chain, int k, int b,
                                           int dc, bool act) {
    const int t0 = (int)((int64_t)k * p.chunk_len);
    const int t1 = (int)min(p.L, (int64_t)t0 + p.chunk_len);
    const int64_t ci = (int64_t)b * p.D + dc;
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = p.h0 ? p.h0[ci * N + n] : 0.0f;
    if (k > 0) enter_state<N, FAST>(p, c, chain, k, h);
    run_readout<T, N, FAST, HAS_Z>(p, b, dc, act, t0, t1, h, c);
    if (k == p.chunks - 1 && p.h_final && act) {
        float *out = p.h_final + ci * N;
#pragma unroll
        for (int n = 0; n < N; ++n) out[n] = h[n];
    }
}

template <typename T, int N, bool HAS_Z>
__global__ __launch_bounds__(64) void scan_main_kernel(const ScanK p) {
    const ChainSlot slot = chain_slot(p.batch * p.dblocks, p.chunks);
    if (!slot.valid) return;
    const int b = slot.chain / p.dblocks;
    const int d = (slot.chain % p.dblocks) * 64 + threadIdx.x;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const Chan<N> c = load_chan<N>(p, dc);
    // wave-uniform choice of the exact fast path
    if (__all(row_is_geometric<N>(p.A + (int64_t)dc * N)))
        scan_chunk<T, N, HAS_Z, true>(p, c, slot.chain, slot.pos, b, dc, act);
    else
        scan_chunk<T, N, HAS_Z, false>(p, c, slot.chain, slot.pos, b, dc, act);
}

// L == 0: the final state is the initial one.
__global__ __launch_bounds__(256) void copy_state_kernel(const float *h0, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

template <typename T, int N>
ssm_status launch_typed(const ScanK &k, hipStream_t s, int passes) {
    const int chains = k.batch * k.dblocks;
    if (k.chunks > 1 && (passes & 1))
        hipLaunchKernelGGL((scan_chunk_state_kernel<T, N>), dim3(chain_grid(chains, k.chunks - 1)),
                           dim3(64), 0, s, k);
    if (!(passes & 2)) return SSM_OK;
    const int grid = chain_grid(chains, k.chunks);
    if (k.z)
        hipLaunchKernelGGL((scan_main_kernel<T, N, true>), dim3(grid), dim3(64), 0, s, k);
    else
        hipLaunchKernelGGL((scan_main_kernel<T, N, false>), dim3(grid), dim3(64), 0, s, k);
    return SSM_OK;
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
        k.L = a.seqlen; k.chunk_len = plan.chunk_len; k.D = (int32_t)a.dim;
        k.batch = (int32_t)a.batch; k.chunks = (int32_t)plan.chunks;
        k.dblocks = (int32_t)((a.dim + 63) / 64);
        k.softplus = a.delta_softplus ? 1 : 0;
        k.G = a.ngroups > 1 ? (int32_t)a.ngroups : 1;
        k.dpg = (int32_t)(a.dim / k.G);
        const bool bf = a.dtype == SSM_BF16;
        switch (a.dstate) {
            case 16: bf ? launch_typed<uint16_t, 16>(k, s, passes) : launch_typed<float, 16>(k, s, passes); break;
            case 32: bf ? launch_typed<uint16_t, 32>(k, s, passes) : launch_typed<float, 32>(k, s, passes); break;
            case 64: bf ? launch_typed<uint16_t, 64>(k, s, passes) : launch_typed<float, 64>(k, s, passes); break;
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
