// Selective scan (Mamba-1 form) for gfx950: the kernels, as templates over the
// storage type T and the state size N. Each scan_fwd_n*.hip instantiates one N;
// scan_fwd.hip holds the dispatcher.
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
//     Chunk j > 0 needs the state entering it. Pass 1a runs every chunk but the last
//     from a zero state and stores the chunk's affine map h -> P_j o h + S_j (its end
//     state S_j and its decay, P_j[n] = exp(A[n] sum dt)); pass 1b composes those
//     maps in order, once per chain (the associative combine (a1,b1),(a2,b2) ->
//     (a2 a1, a2 b1 + b2) applied chunk by chunk), into the map from the sequence
//     start to each chunk; pass 2 applies that map to h0, reruns every chunk from its
//     true entering state and writes y (and h_final from the last chunk).
//   * When a row of A has the form A[d,n] = (n+1) A[d,0] (checked exactly, per
//     channel, on the device), exp(dt A[d,n]) = r^(n+1) with r = exp(dt A[d,0]):
//     one exponential per (b,t,d) and a product tree for the powers instead of N
//     exponentials. Rows of any other form take the general path.
#pragma once

#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "chain.h"
#include "device_common.h"
#include "internal.h"

namespace ssm {

struct ScanK {
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *bias, *Dskip, *h0;
    void *y;
    float *h_final;
    float *agg;       // [chains][G-1][N+1][64]: each chunk's end state from zero, then its decay
    float *pre;       // [chains][G-1][N+1][64]: the composed map entering chunks 1..G-1
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

// Launch the passes of one call for one state size (bit 0 of passes: chunk
// aggregates and their prefix; bit 1: apply); bf16: storage type.
ssm_status scan_launch_n16(const ScanK &k, hipStream_t s, int passes, bool bf16);
ssm_status scan_launch_n32(const ScanK &k, hipStream_t s, int passes, bool bf16);
ssm_status scan_launch_n64(const ScanK &k, hipStream_t s, int passes, bool bf16);

namespace {

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
template <typename T, int N, bool FAST, bool HAS_Z, bool SP>
__device__ __forceinline__ void step_readout(const Chan<N> &c, T xraw, T draw, T zraw,
                                             const uint32_t (&bw)[RowWords<T, N>::value],
                                             const uint32_t (&cw)[RowWords<T, N>::value],
                                             float (&h)[N], rsrc_t yr, uint32_t lo, uint32_t soff,
                                             bool act) {
    const float xv = to_f32(xraw);
    const float v = to_f32(draw) + c.bias;
    const float dt = SP ? softplus_f32(v) : v;
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
    float yv = c.dsk * xv;     // the readout accumulates onto the skip term
#pragma unroll
    for (int n = 0; n < N; ++n) yv = fmaf(Cv[n], h[n], yv);
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
template <typename T, int N, bool FAST, bool HAS_Z, bool SP>
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

    uint32_t bw[NW], cw[NW];
    load_row<T, N>(as_const(Brow + t0 * GN), bw);
    load_row<T, N>(as_const(Crow + t0 * GN), cw);

    // x, delta, z of the U steps from tb on, clamped to the last step so every read
    // stays in bounds
    auto load_block = [&](T (&xx)[U], T (&dd)[U], T (&zz)[U], int tb) {
        const uint32_t rb = opaque_u32(rowb);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t so = (uint32_t)min(tb + u, t1 - 1) * rb;
            buf_load(xr, lo, so, xx[u]);
            buf_load(dr, lo, so, dd[u]);
            if constexpr (HAS_Z) buf_load(zr, lo, so, zz[u]);
        }
    };
    // the first cnt (<= U, uniform) steps from tb, inputs already in registers
    auto run_block = [&](const T (&xx)[U], const T (&dd)[U], const T (&zz)[U], int tb, int cnt) {
        // per-block copies the compiler cannot see through: the step offsets are then
        // formed in the block (scalar ALU) instead of being precomputed for every step
        // of the loop and kept in spilled SGPRs
        const uint32_t rb = opaque_u32(rowb);
        const int gn = (int)opaque_u32((uint32_t)GN);
        const int tbo = (int)opaque_u32((uint32_t)tb), tlast = (int)opaque_u32((uint32_t)(t1 - 1));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u < cnt) {
                uint32_t bn[NW], cn[NW];
                const int rn = min(tbo + u + 1, tlast) * gn;
                load_row<T, N>(as_const(Brow + rn), bn);
                load_row<T, N>(as_const(Crow + rn), cn);
                step_readout<T, N, FAST, HAS_Z, SP>(c, xx[u], dd[u], HAS_Z ? zz[u] : xx[u], bw, cw, h, yr,
                                                    lo, (uint32_t)(tbo + u) * rb, act);
#pragma unroll
                for (int j = 0; j < NW; ++j) { bw[j] = bn[j]; cw[j] = cn[j]; }
                // keep the steps apart in the schedule: interleaving several steps'
                // unpacked B/C rows runs out of SGPRs (spilled through VGPR lanes)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Two register blocks used in turn (no copies between them): the next block's
    // loads are in flight while the current one computes.
    T xa[U], da[U], za[U], xb[U], db[U], zb[U];
    load_block(xa, da, za, t0);
    for (int t = t0;;) {
        if (t1 - t <= U) { run_block(xa, da, za, t, t1 - t); break; }
        load_block(xb, db, zb, t + U);
        run_block(xa, da, za, t, U);
        t += U;
        if (t1 - t <= U) { run_block(xb, db, zb, t, t1 - t); break; }
        load_block(xa, da, za, t + U);
        run_block(xb, db, zb, t, U);
        t += U;
    }
}

// End state of [t0, t1) from a zero state, and the chunk's decay, walking time
// backwards: with R = prod_{k>t} exp(dt_k A[0]) the fast path adds
// B_t[n] * dt_t x_t * R^(n+1) to S[n], i.e. one multiply and one FMA per state
// (the decay of everything after t is applied once, as a power of R). At the end
// R is the product of every step's decay r = exp(dt A[0]), and the chunk decays
// state n by R^(n+1); that product is returned. The general path runs the
// recurrence forwards and returns the summed step (state n decays by
// exp(A[n] sum dt)).
template <typename T, int N, bool FAST, bool SP>
__device__ __forceinline__ float run_aggregate(const ScanK &p, int b, int dc, int t0, int t1,
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
    double dsum = 0.0;   // general path only
    float R = 1.0f;      // fast path only

    auto one = [&](T xraw, T draw, const uint32_t (&bw)[NW]) {
        const float xv = to_f32(xraw);
        const float v = to_f32(draw) + c.bias;
        const float dt = SP ? softplus_f32(v) : v;
        const float dtx = dt * xv;
        float Bv[N];
        unpack_row<T, N>(bw, Bv);
        if constexpr (!FAST) dsum += (double)dt;
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
        // backwards in time, U steps per register block, two blocks used in turn
        uint32_t bw[NW];
        load_row<T, N>(as_const(Brow + (t1 - 1) * GN), bw);
        // x, delta of steps tb, tb-1, ..., tb-U+1 (clamped to t0)
        auto load_block = [&](T (&xx)[U], T (&dd)[U], int tb) {
            const uint32_t rb = opaque_u32(rowb);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t so = (uint32_t)max(tb - u, t0) * rb;
                buf_load(xr, lo, so, xx[u]);
                buf_load(dr, lo, so, dd[u]);
            }
        };
        auto run_block = [&](const T (&xx)[U], const T (&dd)[U], int tb, int cnt) {
            const int gn = (int)opaque_u32((uint32_t)GN);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u < cnt) {
                    uint32_t bn[NW];
                    load_row<T, N>(as_const(Brow + max(tb - u - 1, t0) * gn), bn);
                    one(xx[u], dd[u], bw);
#pragma unroll
                    for (int j = 0; j < NW; ++j) bw[j] = bn[j];
                    __builtin_amdgcn_sched_barrier(0);   // one step's B row in SGPRs at a time
                }
            }
        };
        T xa[U], da[U], xb[U], db[U];
        load_block(xa, da, t1 - 1);
        for (int t = t1 - 1;;) {              // t: latest step not yet added
            if (t - t0 + 1 <= U) { run_block(xa, da, t, t - t0 + 1); break; }
            load_block(xb, db, t - U);
            run_block(xa, da, t, U);
            t -= U;
            if (t - t0 + 1 <= U) { run_block(xb, db, t, t - t0 + 1); break; }
            load_block(xa, da, t - U);
            run_block(xb, db, t, U);
            t -= U;
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
    if constexpr (FAST) return R;
    return (float)dsum;
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

// Pass 1a: the end state of chunk k (k < G-1) from a zero state and its decay
// (the product of its steps' exp(dt A[0]) in the fast path, its summed step
// otherwise), stored for the prefix pass (layout [chain][k][n][lane]: one
// contiguous 256-byte row per state index, the decay in row N).
template <typename T, int N, bool SP>
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
    const float dec = __all(row_is_geometric<N>(p.A + (int64_t)dc * N))
                          ? run_aggregate<T, N, true, SP>(p, b, dc, t0, t1, S, c)
                          : run_aggregate<T, N, false, SP>(p, b, dc, t0, t1, S, c);
    float *a = p.agg + ((size_t)slot.chain * (p.chunks - 1) + k) * (N + 1) * 64 + threadIdx.x;
#pragma unroll
    for (int n = 0; n < N; ++n) a[n * 64] = S[n];
    a[N * 64] = dec;
}

// r^m for a wave-uniform m in [1, 64]: squares of r multiplied in by the binary
// digits of m (uniform branches, at most 12 products).
__device__ __forceinline__ float pow_uniform(float r, int m) {
    float acc = 1.0f, sq = r;
#pragma unroll
    for (int bit = 0; bit < 7; ++bit) {
        if ((m >> bit) & 1) acc *= sq;
        if ((m >> (bit + 1)) == 0) break;
        sq *= sq;
    }
    return acc;
}

// Pass 1b: prefix of the chunk maps. Chunk k >= 1 enters with h = Pp_k o h0 + Sp_k,
// where (Pp_k, Sp_k) composes, in order, the maps h -> P_j o h + S_j of chunks
// j < k: Sp_{k+1} = P_k o Sp_k + S_k, and Pp accumulates the decays (their
// product in the fast path, where P_j[n] = R_j^(n+1); their summed step
// otherwise). One workgroup per (chain, row): rows n < N carry Sp[n], row N
// carries Pp. The chain's chunks are cut into segments of about 16, one per wave
// (at most kPrefixSeg; blockDim.x / 64 of them): each wave composes its segment,
// the waves exchange the segment maps through LDS, and each wave walks its segment
// again from the composed map of the segments before it, writing the prefix for
// chunk k to pre[k-1]. Nothing in
// it depends on h0, so a caller that learns h0 later (another device's share of
// the sequence) can still run the apply pass with it.
constexpr int kPrefixSeg = 8;
// Up to this many chunks the apply pass composes the chunk maps itself (at most
// kWalkChunks - 1 per wave) and no prefix pass runs.
constexpr int kWalkChunks = 24;

template <int N>
__global__ __launch_bounds__(64 * kPrefixSeg) void scan_prefix_kernel(const ScanK p) {
    const ChainSlot slot = chain_slot(p.batch * p.dblocks, N + 1);
    if (!slot.valid) return;                              // uniform over the workgroup
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int d = (slot.chain % p.dblocks) * 64 + lane;
    const int dc = d < p.D ? d : p.D - 1;
    const int n = slot.pos;                                // uniform
    const size_t blk = (size_t)(N + 1) * 64;
    const int K = p.chunks - 1;                            // aggregates of chunks 0..K-1
    const float *src = p.agg + (size_t)slot.chain * K * blk + lane;
    float *dst = p.pre + (size_t)slot.chain * K * blk + lane;
    const size_t row = (size_t)min(n, N) * 64, drow = (size_t)N * 64;
    const int nseg = blockDim.x >> 6;
    const int per = (K + nseg - 1) / nseg;
    const int j0 = min(K, w * per), j1 = min(K, j0 + per);
    constexpr int U = 16;
    float sv[U], rv[U];
    auto load_block = [&](int jb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t kk = (size_t)min(jb + u, K - 1) * blk;
            sv[u] = src[kk + row];
            rv[u] = src[kk + drow];
        }
    };
    // the segment's first block goes out before the A row is read and tested
    load_block(j0);
    const bool fast = __all(row_is_geometric<N>(p.A + (int64_t)dc * N));
    const float al2 = p.A[(int64_t)dc * N + min(n, N - 1)] * kLog2e;
    const float unit = fast ? 1.0f : 0.0f;                // identity of the decay combine
    auto decay = [&](float rr) { return fast ? pow_uniform(rr, n + 1) : fast_exp2(al2 * rr); };
    auto comb = [&](float a, float rr) { return fast ? a * rr : a + rr; };

    // 1. this segment's map: decay combine Rs, state part Ss (rows < N)
    float Rs = unit, Ss = 0.0f;
    for (int jb = j0; jb < j1; jb += U) {
        if (jb != j0) load_block(jb);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (jb + u < j1) {                             // uniform
                if (n < N) Ss = fmaf(decay(rv[u]), Ss, sv[u]);
                Rs = comb(Rs, rv[u]);
            }
        }
    }
    // 2. the maps of the segments before this one, composed in order
    __shared__ float segR[kPrefixSeg][64], segS[kPrefixSeg][64];
    segR[w][lane] = Rs;
    segS[w][lane] = Ss;
    __syncthreads();
    float Rp = unit, Sp = 0.0f;
    for (int v = 0; v < w; ++v) {
        if (n < N) Sp = fmaf(decay(segR[v][lane]), Sp, segS[v][lane]);
        Rp = comb(Rp, segR[v][lane]);
    }
    // 3. walk the segment again from that map, writing each chunk's successor prefix
    // (a segment of one block is still in the registers)
    for (int jb = j0; jb < j1; jb += U) {
        if (j1 - j0 > U) load_block(jb);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (jb + u < j1) {
                if (n < N) Sp = fmaf(decay(rv[u]), Sp, sv[u]);
                Rp = comb(Rp, rv[u]);
                dst[(size_t)(jb + u) * blk + row] = n < N ? Sp : Rp;
            }
        }
    }
}

// Pass 2: every chunk from its entering state, with readout, gate and store; the
// last chunk writes h_final.
template <typename T, int N, bool HAS_Z, bool FAST, bool SP, bool WALK>
__device__ __forceinline__ void scan_chunk(const ScanK &p, const Chan<N> &c, int chain, int k, int b,
                                           int dc, bool act) {
    const int t0 = (int)((int64_t)k * p.chunk_len);
    const int t1 = (int)min(p.L, (int64_t)t0 + p.chunk_len);
    const int64_t ci = (int64_t)b * p.D + dc;
    float h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = p.h0 ? p.h0[ci * N + n] : 0.0f;
    if (WALK && k > 0) {
        // few chunks, no prefix pass: the maps of chunks 0..k-1 applied in order,
        // h <- P_j o h + S_j, from the aggregates (k - 1 < kWalkChunks)
        const float *ag = p.agg + (size_t)chain * (p.chunks - 1) * (N + 1) * 64 + threadIdx.x;
        for (int j = 0; j < k; ++j) {
            const float *a = ag + (size_t)j * (N + 1) * 64;
            float sj[N];
#pragma unroll
            for (int n = 0; n < N; ++n) sj[n] = a[n * 64];
            const float dj = a[N * 64];
            float P[N];
            if constexpr (FAST) {
                powers<N>(dj, P);
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n) P[n] = fast_exp2(c.Al2[n] * dj);
            }
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = fmaf(P[n], h[n], sj[n]);
        }
    } else if (!WALK && k > 0) {
        // the composed map of chunks 0..k-1 applied to h0: h = Pp o h0 + Sp
        const float *pr = p.pre + ((size_t)chain * (p.chunks - 1) + (k - 1)) * (N + 1) * 64 + threadIdx.x;
        float sp[N];
#pragma unroll
        for (int n = 0; n < N; ++n) sp[n] = pr[n * 64];
        const float pp = pr[N * 64];
        if (p.h0) {                                        // uniform
            float P[N];
            if constexpr (FAST) {
                powers<N>(pp, P);
            } else {
#pragma unroll
                for (int n = 0; n < N; ++n) P[n] = fast_exp2(c.Al2[n] * pp);
            }
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = fmaf(P[n], h[n], sp[n]);
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = sp[n];
        }
    }
    run_readout<T, N, FAST, HAS_Z, SP>(p, b, dc, act, t0, t1, h, c);
    if (k == p.chunks - 1 && p.h_final && act) {
        float *out = p.h_final + ci * N;
#pragma unroll
        for (int n = 0; n < N; ++n) out[n] = h[n];
    }
}

// WALK: the call has too few chunks for a prefix pass (p.pre is null), and each
// wave composes the maps of the chunks before its own.
template <typename T, int N, bool HAS_Z, bool SP, bool WALK>
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
        scan_chunk<T, N, HAS_Z, true, SP, WALK>(p, c, slot.chain, slot.pos, b, dc, act);
    else
        scan_chunk<T, N, HAS_Z, false, SP, WALK>(p, c, slot.chain, slot.pos, b, dc, act);
}

template <typename T, int N, bool SP>
ssm_status launch_typed(const ScanK &k, hipStream_t s, int passes) {
    const int chains = k.batch * k.dblocks;
    if (k.chunks > 1 && (passes & 1)) {
        hipLaunchKernelGGL((scan_chunk_state_kernel<T, N, SP>), dim3(chain_grid(chains, k.chunks - 1)),
                           dim3(64), 0, s, k);
        if (k.pre) {
            const int nseg = std::min(kPrefixSeg, std::max(1, (k.chunks - 1 + 15) / 16));
            hipLaunchKernelGGL((scan_prefix_kernel<N>), dim3(chain_grid(chains, N + 1)), dim3(64 * nseg), 0, s, k);
        }
    }
    if (!(passes & 2)) return SSM_OK;
    const int grid = chain_grid(chains, k.chunks);
    const bool walk = k.pre == nullptr;                   // also a single chunk: nothing to compose
    if (k.z) {
        if (walk) hipLaunchKernelGGL((scan_main_kernel<T, N, true, SP, true>), dim3(grid), dim3(64), 0, s, k);
        else hipLaunchKernelGGL((scan_main_kernel<T, N, true, SP, false>), dim3(grid), dim3(64), 0, s, k);
    } else {
        if (walk) hipLaunchKernelGGL((scan_main_kernel<T, N, false, SP, true>), dim3(grid), dim3(64), 0, s, k);
        else hipLaunchKernelGGL((scan_main_kernel<T, N, false, SP, false>), dim3(grid), dim3(64), 0, s, k);
    }
    return SSM_OK;
}

// softplus on or off as a template parameter: no per-step branch in the loops
template <typename T, int N>
ssm_status launch_sp(const ScanK &k, hipStream_t s, int passes) {
    return k.softplus ? launch_typed<T, N, true>(k, s, passes) : launch_typed<T, N, false>(k, s, passes);
}

}  // namespace
}  // namespace ssm
