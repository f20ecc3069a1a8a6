// Gradients of the scalar-A (SSD) form on the matrix cores (training runs the
// scan [Mamba-2 page "Mamba-2：把状态空间模型和 Attention 统一到一个数学框架里", Core
// idea: Mamba-1's scan and its training throughput; key point 1: the
// semiseparable matrix, whose off-diagonal blocks pass through one state per
// chunk]).
//
// Per head (channels p, states n) the forward is S_t = a_t S_{t-1} + dt_t x_t B_t^T,
// y_t = S_t C_t + D x_t (then the gate), a_t = exp(A dt_t). With dyc = dy silu(z)
// the adjoint state g_t = dL/dS_t runs backwards: g_t = dyc_t C_t^T + a_{t+1} g_{t+1}.
// Inside a chunk with Lm[t,s] = exp(cs_t - cs_s) [s <= t] (cs the in-chunk
// cumulative A dt), the entering state Sin and the adjoint Gout of the chunk's end
// state (the state entering the next chunk):
//   dx_s  = dt_s (sum_t Lm[t,s] (C_t.B_s) dyc_t + e_s Gout B_s) + D dyc_s,  e_s = exp(cs_end - cs_s)
//   dB_s += dt_s (sum_t Lm[t,s] (dyc_t.x_s) C_t + e_s x_s Gout)            (over heads)
//   dC_t += sum_{s<=t} Lm[t,s] dt_s (dyc_t.x_s) B_s + exp(cs_t) dyc_t Sin   (over heads)
// and for the decays, with W[t,s] = Lm[t,s] (C_t.B_s) dt_s (dyc_t.x_s):
//   q_t    = sum_s W[t,s] + exp(cs_t) dyc_t Sin C_t        (= dyc_t.(y_t - D x_t))
//   dd_s   = sum_t W[t,s] / dt_s + e_s x_s Gout B_s        (= sum g_s x_s B_s), dtdd = dt dd
//   da_t   = sum_{t'>=t in chunk} (q_t' - dtdd_t') + <Gout, S_end>   (dL/d(A dt_t))
//   d dt_t = dd_t + A da_t,  dA += dt_t da_t
// (the last identity: dL/d log a_t = <g_t, S_t> - dt_t <g_t, x_t B_t^T>, and
// <g_t, S_t> telescopes along the chunk to the sums above).
//
// Kernels, in order:
//   recompute (ssd_fwd.hip): chunk states with the weighted x split into bf16
//     hi + lo, the entering states in fp32 (and bf16), and with z the fp32
//     pre-gate output for dz;
//   gate (with z): dD, dz and dyc as bf16 hi + lo (without z the column kernel
//     sums dD);
//   adjoint aggregates (ssd_fwd.hip): R_c = sum_t exp(cs_t) dyc_t^T C_t (split);
//   reverse state pass: Gout_c, <Gout_c, S_end,c>, dh0;
//   row kernel: dC (partial sums over a slice of heads) and q;
//   column kernel: dx, dd, dtdd and dB (partial sums);
//   finish: d dt, dA, d bias; reduce: dB, dC over the head slices.
// Precision: the fp32 sums q and dtdd and the chunk-end terms cancel to a small
// da, so every matrix-core operand that feeds them is split into bf16 hi + lo
// parts (chunk states, adjoint aggregates, Sin, Gout, and dyc when the gate makes
// it inexact); the
// products that only feed dx, dB, dC use single bf16 operands.
#include <algorithm>
#include <cstdio>

#include "device_common.h"
#include "internal.h"
#include "ssd_common.h"

namespace ssm {
namespace {

constexpr int kHsCol = kSsdBwdHeadsCol;
constexpr int kHsRow = kSsdBwdHeadsRow;

struct BwdK {
    SSDK f;
    const uint16_t *dy;
    uint16_t *dych, *dycl;         // dy silu(z) as bf16 hi + lo (with z); dych = dy without
    const float *dh_final;
    uint16_t *dx, *ddt, *dz;
    float *dA, *dD, *dbias, *dh0;
    float *sin32, *gout, *hfin, *kc;   // kc: [B][H][nc][kcw] per-wave shares of <Gout, S_end>
    float *q, *dtdd, *dd;
    float *dBp, *dCp, *dB, *dC;
    int32_t nsl_col, nsl_row, batch;
    int32_t kcw;                       // waves per (b, h) in the reverse state pass: N / 4
};

typedef __attribute__((ext_vector_type(2))) float f32x2;

__device__ __forceinline__ float sigmoid_f32(float v) { return 1.0f / (1.0f + fast_exp2(-v * kLog2e)); }

template <int CTRL>
__device__ __forceinline__ float dpp_ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
// sum over the 16 lanes of a DPP row (lanes with the same l >> 4), in every lane of it
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_ror<0x121>(v);
    v += dpp_ror<0x122>(v);
    v += dpp_ror<0x124>(v);
    v += dpp_ror<0x128>(v);
    return v;
}
// sum over the 4 lanes l, l^16, l^32, l^48 (the same r16), in each of them
__device__ __forceinline__ float kb_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return kb_sum(v);
}

// hi + lo bf16 parts of 8 fp32 values (hi = RNE(v), lo = RNE(v - hi))
__device__ __forceinline__ void split8(const f32x4 &a, const f32x4 &b, u32x4 &hi, u32x4 &lo) {
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
        lo[e] = pack_bf16(v[2 * e] - bf16_lo(hi[e]), v[2 * e + 1] - bf16_hi(hi[e]));
    }
}

// ---------------------------------------------------------------- LDS staging
// Natural-layout tiles written by block_both / block_split_both (B, C, dyc and Gout
// rows) hold element (row R, column j) at column j ^ nsw(R). The 16 lanes that write
// rows 4 rg + i of one column group at once then cover 8 bank groups instead of 2
// (rows 4 apart of a 16-byte-aligned padded row fall on two). Every read of these
// tiles applies the same XOR; it keeps 8-column groups whole, so 16-byte fragment
// reads stay contiguous.
__device__ __forceinline__ int nsw(int row) { return ((row >> 3) & 7) << 3; }

// One 4 x 8 block of a bf16 tile (rows 4 rg .. +3 at row stride rs, columns gcol ..
// +7) through a buffer resource (rows past its range read as 0), written to LDS in
// natural layout nat[row][lcol ..] and/or transposed tr[lcol + c][perm_s(row)].
__device__ __forceinline__ void block_both(rsrc_t r, int64_t rs, int rg, int gcol, uint16_t *nat, int ld,
                                           uint16_t *tr, int ldt, int lcol) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = load16(r, (uint32_t)(((rg * 4 + i) * rs + gcol) * 2));
    if (nat) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)&nat[(rg * 4 + i) * ld + (lcol ^ nsw(rg * 4 + i))] = v[i];
    }
    if (tr) store_transposed(v, tr, ldt, lcol, perm_s(rg * 4));
}
// One 4 x 8 block of an fp32 [64][rs] tile (rows 4 rg .., columns 8 cg ..) as bf16
// hi and lo parts, natural [row][col] and/or transposed [col][row] (rows in order).
__device__ __forceinline__ void block_split_both(const float *src, int64_t rs, int rg, int cg, uint16_t *nat_hi,
                                                 uint16_t *nat_lo, int ld, uint16_t *tr_hi, uint16_t *tr_lo,
                                                 int ldt) {
    u32x4 hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float *q = src + (rg * 4 + i) * rs + cg * 8;
        split8(*(const f32x4 *)q, *(const f32x4 *)(q + 4), hi[i], lo[i]);
    }
    if (nat_hi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *(u32x4 *)&nat_hi[(rg * 4 + i) * ld + ((cg * 8) ^ nsw(rg * 4 + i))] = hi[i];
            *(u32x4 *)&nat_lo[(rg * 4 + i) * ld + ((cg * 8) ^ nsw(rg * 4 + i))] = lo[i];
        }
    }
    if (tr_hi) {
        store_transposed(hi, tr_hi, ldt, cg * 8, rg * 4);
        store_transposed(lo, tr_lo, ldt, cg * 8, rg * 4);
    }
}

// 16-byte fragment of a bf16 row through a buffer resource (0 past its range)
__device__ __forceinline__ bf16x8 frag(rsrc_t r, uint32_t byte_off) { return as_bf16x8(load16(r, byte_off)); }

// A fragment from two D tiles (k = 8 kb + e <-> the tiles' 4 kb + i, see perm_s)
__device__ __forceinline__ bf16x8 afrag(const f32x4 &lo_tile, const f32x4 &hi_tile) {
    return as_bf16x8(u32x4{pack_bf16(lo_tile[0], lo_tile[1]), pack_bf16(lo_tile[2], lo_tile[3]),
                           pack_bf16(hi_tile[0], hi_tile[1]), pack_bf16(hi_tile[2], hi_tile[3])});
}

// workgroup -> (b, c, g, slice, 64-row block); the blocks of one (b, c, g, slice)
// are consecutive
struct Tile { int b, c, g, sl, blk; };
__device__ __forceinline__ Tile decode_tile(int id, int TBS, int nsl, int G, int nc) {
    Tile t;
    t.blk = id % TBS; id /= TBS;
    t.sl = id % nsl; id /= nsl;
    t.g = id % G; id /= G;
    t.c = id % nc;
    t.b = id / nc;
    return t;
}

// per-head dt and cs * log2(e) of a chunk into LDS (wave w does heads w, w+4, ...)
template <int Q, int HS>
__device__ __forceinline__ void head_tables(const SSDK &p, int b, int c, int hfirst, int hend,
                                            float (*cs2)[Q], float (*dts)[Q]) {
    constexpr int SPL = Q / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int j = wv; j < HS; j += 4) {
        float dtv[SPL], cs[SPL];
        head_dt_cs<Q>(p, b, std::min(hfirst + j, hend - 1), c, dtv, cs);
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            cs2[j][lane * SPL + i] = cs[i] * kLog2e;
            dts[j][lane * SPL + i] = dtv[i];
        }
    }
}

// ---------------------------------------------------------------- gate
// With z: one workgroup per (head, 256 rows of (b, t)); a lane owns 8 consecutive
// p. dyc = dy silu(z) as bf16 hi + lo, dz = dy (y_pre) silu'(z), dDskip.
__global__ __launch_bounds__(256) void ssd_bwd_gate_kernel(const BwdK k, int64_t rows) {
    const int h = blockIdx.y, H = k.f.H;   // rows of (b, t) on x (no 65535 limit), heads on y
    const int v = threadIdx.x & 7, rsub = threadIdx.x >> 3;
    float dsum = 0.0f;
    for (int it = 0; it < 8; ++it) {
        const int64_t row = (int64_t)blockIdx.x * 256 + it * 32 + rsub;
        if (row >= rows) break;
        const int64_t e = (row * H + h) * kP + v * 8;
        const u32x4 xv = *(const u32x4 *)(k.f.x + e);
        const u32x4 dv = *(const u32x4 *)(k.dy + e);
        const u32x4 zv = *(const u32x4 *)(k.f.z + e);
        const f32x4 y0 = *(const f32x4 *)(k.f.y32 + e), y1 = *(const f32x4 *)(k.f.y32 + e + 4);
        const float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        u32x4 hi, lo, dzv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float g2[2], dz2[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float zz = r ? bf16_hi(zv[q]) : bf16_lo(zv[q]);
                const float dyv = r ? bf16_hi(dv[q]) : bf16_lo(dv[q]);
                const float xx = r ? bf16_hi(xv[q]) : bf16_lo(xv[q]);
                const float sg = sigmoid_f32(zz);
                g2[r] = dyv * zz * sg;
                dz2[r] = dyv * yv[2 * q + r] * sg * (1.0f + zz * (1.0f - sg));
                dsum = fmaf(g2[r], xx, dsum);
            }
            hi[q] = pack_bf16(g2[0], g2[1]);
            lo[q] = pack_bf16(g2[0] - bf16_lo(hi[q]), g2[1] - bf16_hi(hi[q]));
            dzv[q] = pack_bf16(dz2[0], dz2[1]);
        }
        *(u32x4 *)(k.dych + e) = hi;
        *(u32x4 *)(k.dycl + e) = lo;
        *(u32x4 *)(k.dz + e) = dzv;
    }
    if (!k.dD) return;
    __shared__ float red[4];
    dsum = wave_sum(dsum);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dsum;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(k.dD + h, red[0] + red[1] + red[2] + red[3]);
}

// ---------------------------------------------------------------- reverse state pass
// One thread per (b, h, p, 4 n): the adjoint of the state entering chunk c is
// Lam_c = R_c + decay_c Lam_{c+1} (Lam_nc = dh_final); Gout_c = Lam_{c+1} replaces
// R_c in place, and <Gout_c, S_end,c> (S_end,c = Sin_{c+1}, or the final state)
// is summed per wave and stored as that wave's share (no atomics: the finish
// kernel adds the kcw shares of a (b, h, c) in a fixed order, so d dt does not
// depend on the order in which waves run).
__global__ __launch_bounds__(256) void ssd_bwd_state_pass_kernel(const BwdK k, int N, int64_t total) {
    constexpr int K = 4;
    const SSDK &p = k.f;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;                     // total is a multiple of 256: whole waves
    const int64_t per_bh = (int64_t)kP * N / 4;
    const int64_t bh = i / per_bh;
    const int64_t pn = (i % per_bh) * 4;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t hidx = bh * kP * N + pn;
    const int64_t wslot = (i % per_bh) >> 6;   // this wave's share index within (b, h)
    f32x4 lam = f32x4{0.f, 0.f, 0.f, 0.f};
    if (k.dh_final) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lam[e] = k.dh_final[hidx + e];
    }
    const float *dec = p.decay + bh * p.nc;
    const int64_t cstride = (int64_t)p.H * kP * N;
    const int64_t base = (b * p.nc * p.H + h) * kP * N + pn;
    for (int c0 = p.nc - 1; c0 >= 0; c0 -= K) {
        f32x4 rc[K], se[K];
        float dc[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const int c = std::max(c0 - u, 0);
            rc[u] = *(const f32x4 *)(k.gout + base + c * cstride);
            se[u] = c + 1 < p.nc ? *(const f32x4 *)(k.sin32 + base + (c + 1) * cstride)
                                 : *(const f32x4 *)(k.hfin + hidx);
            dc[u] = dec[c];
        }
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const int c = c0 - u;
            if (c >= 0) {                       // uniform
                *(f32x4 *)(k.gout + base + c * cstride) = lam;
                float part = lam[0] * se[u][0] + lam[1] * se[u][1] + lam[2] * se[u][2] + lam[3] * se[u][3];
                part = wave_sum(part);
                if ((threadIdx.x & 63) == 0) k.kc[(bh * p.nc + c) * k.kcw + wslot] = part;
#pragma unroll
                for (int e = 0; e < 4; ++e) lam[e] = fmaf(dc[u], lam[e], rc[u][e]);
            }
        }
    }
    if (k.dh0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) k.dh0[hidx + e] = lam[e];
    }
}

// ---------------------------------------------------------------- row kernel
// One workgroup per (b, chunk, group, slice of kHsRow heads, 64-row block tb of t);
// wave w owns rows t = 64 tb + 16 w .. +15. Each block of s <= tb is staged once
// (B natural and transposed from one load, x of every head of the slice); the
// score tile (B_s.C_t) is formed once and reused by the heads; per head the tile
// (x_s.dyc_t) gives W (summed over s into q) and, weighted, the A operand of
// dC += M3 B. Then per head the entering-state term exp(cs_t) dyc_t Sin (split
// operands) adds to dC and, dotted with C_t, to q.
// (At N = 256 one workgroup per CU: its LDS blocks take 113 KB.)
template <int N, int Q, bool SPLIT>
__global__ __launch_bounds__(kThreads, N > 128 ? 1 : 2) void ssd_bwd_row_kernel(const BwdK k) {
    constexpr int HS = kHsRow;
    constexpr int TBS = Q / 64, KN = N / 32, NT = N / 16;
    constexpr int LDB = N + 8, LDT = 64 + 8, LDX = kP + 8;
    constexpr int MAIN_BYTES = (64 * LDB + N * LDT + HS * 64 * LDX) * 2;
    constexpr int END_BYTES = (2 * N * LDT + 64 * LDB) * 2;
    __shared__ float cs2[HS][Q], dts[HS][Q];
    __shared__ float qsh[4][16];
    __shared__ __attribute__((aligned(16))) uint8_t ubuf[std::max(MAIN_BYTES, END_BYTES)];
    uint16_t *Bn = reinterpret_cast<uint16_t *>(ubuf);          // [64][LDB] B rows of the s block
    uint16_t *BT = Bn + 64 * LDB;                                  // [N][LDT] B^T, s permuted
    uint16_t *Xn = BT + N * LDT;                                   // [HS][64][LDX] x rows per head
    uint16_t *ST = reinterpret_cast<uint16_t *>(ubuf);           // [2][N][LDT] Sin^T hi, lo
    uint16_t *Cn = ST + 2 * N * LDT;                               // [64][LDB] C rows of the t block

    const SSDK &p = k.f;
    const Tile tl = decode_tile(blockIdx.x, TBS, k.nsl_row, p.G, p.nc);
    const int b = tl.b, c = tl.c, g = tl.g, tb = tl.blk;
    const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, kb = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: addresses built from it stay scalar
    const int64_t t_base = (int64_t)c * Q;
    const int T = (int)std::min<int64_t>(Q, p.L - t_base);
    if (tb * 64 >= T) return;                                       // uniform
    const int hfirst = g * p.hpg + tl.sl * HS, hend = std::min((g + 1) * p.hpg, hfirst + HS);
    const int nh = hend - hfirst;
    const int GN = p.G * N;
    const int64_t xs = (int64_t)p.H * kP;                            // row stride of (B, L, H, P)
    const int t0 = tb * 64 + wv * 16;                                // this wave's first row
    const uint16_t *Bbase = p.Bm + (((int64_t)b * p.L + t_base) * p.G + g) * N;
    const uint16_t *Cbase = p.Cm + (((int64_t)b * p.L + t_base) * p.G + g) * N;
    const uint16_t *Xbase = p.x + ((int64_t)b * p.L + t_base) * xs;
    const int64_t dbase = ((int64_t)b * p.L + t_base) * xs;

    head_tables<Q, HS>(p, b, c, hfirst, hend, cs2, dts);
    // C_t of this lane's column t = t0 + r16 (B operand of B_s . C_t, k = n)
    bf16x8 cfr[KN];
    {
        const rsrc_t rc = make_rsrc_u(Cbase + (int64_t)t0 * GN, (uint32_t)(std::max(0, T - t0) * GN * 2));
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) cfr[kk] = frag(rc, (uint32_t)((r16 * GN + 32 * kk + 8 * kb) * 2));
    }
    // dyc of row t0 + r16 for head h (k = p): the B operand of x_s . dyc_t and the
    // A operand of dyc_t Sin
    const rsrc_t rdh = make_rsrc_u(k.dych + dbase + (int64_t)t0 * xs, (uint32_t)(std::max(0, T - t0) * xs * 2));
    const rsrc_t rdl = make_rsrc_u(SPLIT ? k.dycl + dbase + (int64_t)t0 * xs : k.dych, SPLIT ? (uint32_t)(std::max(0, T - t0) * xs * 2) : 0u);
    auto load_dyc = [&](int h, bf16x8 (&fh)[2], bf16x8 (&fl)[2]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const uint32_t off = (uint32_t)((r16 * xs + h * kP + 32 * kk + 8 * kb) * 2);
            fh[kk] = frag(rdh, off);
            if constexpr (SPLIT) fl[kk] = frag(rdl, off);
        }
    };

    const int tl_row = t0 + r16;                                      // chunk-local t of this lane
    const int r = std::max(tb * 64 - 1, 0);                           // last step before the t block (tb > 0)
    float wrow[HS];
#pragma unroll
    for (int j = 0; j < HS; ++j) wrow[j] = 0.0f;
    f32x4 dc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) dc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int sb = 0; sb <= tb; ++sb) {
        const int s0 = sb * 64;
        const bool diag = sb == tb;
        __syncthreads();
        {   // B block (natural + transposed from one load) and x of every head
            const rsrc_t rb = make_rsrc_u(Bbase + (int64_t)s0 * GN, (uint32_t)(std::max(0, T - s0) * GN * 2));
            for (int blk = tid; blk < 16 * (N / 8); blk += kThreads)
                block_both(rb, GN, blk & 15, (blk >> 4) * 8, Bn, LDB, BT, LDT, (blk >> 4) * 8);
            const rsrc_t rx = make_rsrc_u(Xbase + (int64_t)s0 * xs + hfirst * kP,
                                        (uint32_t)(std::max(0, T - s0) * xs * 2));
            // loads in batches of XB, each batch issued before any of its stores (a load
            // under the head test would be waited for at the test's end, one at a time);
            // a head past the group reads other x or zeros and is not stored
            constexpr int XI = HS * 64 * 8 / kThreads, XB = XI < 4 ? XI : 4;
#pragma unroll
            for (int i0 = 0; i0 < XI; i0 += XB) {
                u32x4 xr[XB];
#pragma unroll
                for (int i = 0; i < XB; ++i) {
                    const int v = tid + kThreads * (i0 + i), j = v >> 9, row = (v >> 3) & 63, cv = v & 7;
                    xr[i] = load16(rx, (uint32_t)((row * xs + j * kP + cv * 8) * 2));
                }
#pragma unroll
                for (int i = 0; i < XB; ++i) {
                    const int v = tid + kThreads * (i0 + i), j = v >> 9, row = (v >> 3) & 63, cv = v & 7;
                    if (j < nh) *(u32x4 *)&Xn[(j * 64 + row) * LDX + cv * 8] = xr[i];
                }
            }
        }
        __syncthreads();
        // (B_s . C_t): lane holds s = s0 + 16u + 4kb + i, t = t0 + r16
        f32x4 cb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            cb[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!diag || u <= wv) {
#pragma unroll
                for (int kk = 0; kk < KN; ++kk)
                    cb[u] = mfma16x16x32(
                        as_bf16x8(*(const u32x4 *)&Bn[(16 * u + r16) * LDB + ((32 * kk + 8 * kb) ^ nsw(16 * u + r16))]),
                        cfr[kk], cb[u]);
            }
        }
#pragma unroll
        for (int j = 0; j < HS; ++j) {
            if (j >= nh) break;                                       // uniform
            const int h = hfirst + j;
            bf16x8 fh[2], fl[2];
            load_dyc(h, fh, fl);
            const uint16_t *X = Xn + j * 64 * LDX;
            // (x_s . dyc_t), same layout as cb
            f32x4 xd[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                xd[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (!diag || u <= wv) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const bf16x8 xa = as_bf16x8(*(const u32x4 *)&X[(16 * u + r16) * LDX + 32 * kk + 8 * kb]);
                        xd[u] = mfma16x16x32(xa, fh[kk], xd[u]);
                        if constexpr (SPLIT) xd[u] = mfma16x16x32(xa, fl[kk], xd[u]);
                    }
                }
            }
            // M3[t,s] = Lm dt_s (x_s.dyc_t); W = M3 (B_s.C_t)
            const float ct = cs2[j][tl_row];
            const float cr = cs2[j][r];
            const float at = diag ? 1.0f : fast_exp2(ct - cr);
            float wacc = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int sl = s0 + 16 * u + 4 * kb;
                const f32x4 cs4 = *(const f32x4 *)&cs2[j][sl];
                const f32x4 dt4 = *(const f32x4 *)&dts[j][sl];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float lw;
                    if (diag) lw = sl + i <= tl_row ? fast_exp2(ct - cs4[i]) : 0.0f;
                    else lw = at * fast_exp2(cr - cs4[i]);
                    const float m = lw * dt4[i] * xd[u][i];
                    wacc = fmaf(m, cb[u][i], wacc);
                    xd[u][i] = m;
                }
            }
            wrow[j] += wacc;
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                if (diag && 32 * a > 16 * wv + 15) continue;          // every s of this half is after every row
                const bf16x8 mf = afrag(xd[2 * a], xd[2 * a + 1]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    dc[nt] = mfma16x16x32(mf, as_bf16x8(*(const u32x4 *)&BT[(16 * nt + r16) * LDT + 32 * a + 8 * kb]), dc[nt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // entering-state term, per head
    __syncthreads();
    {
        const rsrc_t rc = make_rsrc_u(Cbase + (int64_t)(tb * 64) * GN, (uint32_t)(std::max(0, T - tb * 64) * GN * 2));
        for (int blk = tid; blk < 16 * (N / 8); blk += kThreads)
            block_both(rc, GN, blk & 15, (blk >> 4) * 8, Cn, LDB, nullptr, 0, (blk >> 4) * 8);
    }
    float qv[HS][4];
#pragma unroll
    for (int j = 0; j < HS; ++j) {
        if (j >= nh) break;                                           // uniform
        const int h = hfirst + j;
        const float *sinh = k.sin32 + ((((int64_t)b * p.nc + c) * p.H + h) * kP) * N;
        if (j) __syncthreads();
        for (int blk = tid; blk < 16 * (N / 8); blk += kThreads)
            block_split_both(sinh, N, blk & 15, blk >> 4, nullptr, nullptr, 0, ST, ST + N * LDT, LDT);
        __syncthreads();
        bf16x8 fh[2], fl[2];
        load_dyc(h, fh, fl);
        f32x4 tmp[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            tmp[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 sh = as_bf16x8(*(const u32x4 *)&ST[(16 * nt + r16) * LDT + 32 * kk + 8 * kb]);
                const bf16x8 sl = as_bf16x8(*(const u32x4 *)&ST[N * LDT + (16 * nt + r16) * LDT + 32 * kk + 8 * kb]);
                tmp[nt] = mfma16x16x32(fh[kk], sh, tmp[nt]);
                tmp[nt] = mfma16x16x32(fh[kk], sl, tmp[nt]);
                if constexpr (SPLIT) tmp[nt] = mfma16x16x32(fl[kk], sh, tmp[nt]);
            }
        }
        // rows t = t0 + 4kb + i: scale by exp(cs_t), V_t = C_t . tmp_t
        const f32x4 c4 = *(const f32x4 *)&cs2[j][t0 + 4 * kb];
        float vp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2(c4[i]);
            float s = 0.0f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                tmp[nt][i] *= e;
                const int R = wv * 16 + 4 * kb + i;
                s = fmaf(to_f32(Cn[R * LDB + ((16 * nt + r16) ^ nsw(R))]), tmp[nt][i], s);
            }
            vp[i] = row16_sum(s);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) dc[nt] += tmp[nt];
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[j][i] = vp[i];
    }
    // q_t = sum_s W[t,s] (lane t = r16 after the sum over kb) + V_t (lane rows 4kb + i)
#pragma unroll
    for (int j = 0; j < HS; ++j) {
        if (j >= nh) break;                                           // uniform
        const float w = kb_sum(wrow[j]);
        if (kb == 0) qsh[wv][r16] = w;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (r16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) qsh[wv][4 * kb + i] += qv[j][i];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (lane < 16 && t0 + lane < T)
            k.q[((int64_t)b * p.L + t_base + t0 + lane) * p.H + hfirst + j] = qsh[wv][lane];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    // dC share of this slice: rows t0 + 4kb + i, n = 16 nt + r16
    float *out = k.dCp + ((((int64_t)tl.sl * k.batch + b) * p.L + t_base) * p.G + g) * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * kb + i;
        if (t < T) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) out[(int64_t)t * GN + 16 * nt + r16] = dc[nt][i];
        }
    }
}

// ---------------------------------------------------------------- column kernel
// One workgroup per (b, chunk, group, slice of kHsCol heads, 64-row block sb of s);
// wave w owns rows s = 64 sb + 16 w .. +15. Each block of t >= sb is staged once
// (C natural and transposed, dyc of every head of the slice natural and
// transposed, each from one load); the score tile (C_t.B_s) is formed once for
// the slice; per head the tile (dyc_t.x_s) gives W (summed over t into dd) and,
// weighted, the A operands of dx += M1 dyc and dB += M2 C. Then per head the
// chunk-end terms e_s B_s Gout and e_s x_s Gout (split Gout) complete dx, dd, dtdd
// and dB.
// (At N = 256 one workgroup per CU: its LDS blocks take 146 KB.)
template <int N, int Q, bool SPLIT>
__global__ __launch_bounds__(kThreads, N > 128 ? 1 : 2) void ssd_bwd_col_kernel(const BwdK k) {
    constexpr int HS = kHsCol;
    constexpr int TBS = Q / 64, KN = N / 32, NT = N / 16;
    constexpr int LDB = N + 8, LDT = 64 + 8, LDX = kP + 8, LDO = kP + 4;
    constexpr int MAIN_BYTES = (64 * LDB + N * LDT + HS * 64 * LDX * (SPLIT ? 2 : 1) + HS * kP * LDT) * 2;
    constexpr int END_BYTES = (2 * kP * LDB + 2 * N * LDT) * 2;
    static_assert(4 * 16 * LDO * 4 <= 2 * kP * LDB * 2, "output tiles alias Gout rows");
    __shared__ float cs2[HS][Q], dts[HS][Q];
    __shared__ float qsh[4][16];
    __shared__ __attribute__((aligned(16))) uint8_t ubuf[std::max(MAIN_BYTES, END_BYTES)];
    uint16_t *Cn = reinterpret_cast<uint16_t *>(ubuf);           // [64][LDB] C rows of the t block
    uint16_t *CT = Cn + 64 * LDB;                                  // [N][LDT] C^T, t permuted
    uint16_t *Dh = CT + N * LDT;                                   // [HS][64][LDX] dyc rows (hi)
    uint16_t *DT = Dh + HS * 64 * LDX;                             // [HS][P][LDT] dyc^T (hi), t permuted
    uint16_t *Dl = DT + HS * kP * LDT;                             // [HS][64][LDX] dyc rows (lo)
    uint16_t *Gn = reinterpret_cast<uint16_t *>(ubuf);           // [2][P][LDB] Gout rows hi, lo
    uint16_t *GT = Gn + 2 * kP * LDB;                              // [2][N][LDT] Gout^T hi, lo
    float *Ot = reinterpret_cast<float *>(ubuf);                   // [4][16][LDO] output tiles (after G)

    const SSDK &p = k.f;
    const Tile tl = decode_tile(blockIdx.x, TBS, k.nsl_col, p.G, p.nc);
    const int b = tl.b, c = tl.c, g = tl.g, sb = tl.blk;
    const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, kb = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: addresses built from it stay scalar
    const int64_t t_base = (int64_t)c * Q;
    const int T = (int)std::min<int64_t>(Q, p.L - t_base);
    if (sb * 64 >= T) return;                                       // uniform
    const int hfirst = g * p.hpg + tl.sl * HS, hend = std::min((g + 1) * p.hpg, hfirst + HS);
    const int nh = hend - hfirst;
    const int GN = p.G * N;
    const int64_t xs = (int64_t)p.H * kP;
    const int s0w = sb * 64 + wv * 16;                               // this wave's first row
    const uint16_t *Bbase = p.Bm + (((int64_t)b * p.L + t_base) * p.G + g) * N;
    const uint16_t *Cbase = p.Cm + (((int64_t)b * p.L + t_base) * p.G + g) * N;
    const int64_t dbase = ((int64_t)b * p.L + t_base) * xs;

    head_tables<Q, HS>(p, b, c, hfirst, hend, cs2, dts);
    // B_s of this lane's column s = s0w + r16 (k = n): B operand of (C_t.B_s), A
    // operand of B_s Gout^T
    bf16x8 bfr[KN];
    {
        const rsrc_t rb = make_rsrc_u(Bbase + (int64_t)s0w * GN, (uint32_t)(std::max(0, T - s0w) * GN * 2));
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) bfr[kk] = frag(rb, (uint32_t)((r16 * GN + 32 * kk + 8 * kb) * 2));
    }
    const rsrc_t rx = make_rsrc_u(p.x + dbase + (int64_t)s0w * xs, (uint32_t)(std::max(0, T - s0w) * xs * 2));
    auto load_x = [&](int h, bf16x8 (&xf)[2]) {     // x_s rows (k = p)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) xf[kk] = frag(rx, (uint32_t)((r16 * xs + h * kP + 32 * kk + 8 * kb) * 2));
    };

    const int sl_col = s0w + r16;                                     // chunk-local s of this lane
    const int rr = sb * 64 + 63;                                      // last step of the s block
    f32x4 dxa[HS][4];
#pragma unroll
    for (int j = 0; j < HS; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) dxa[j][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 db[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) db[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float wcol[HS];
#pragma unroll
    for (int j = 0; j < HS; ++j) wcol[j] = 0.0f;

    for (int tb = sb; tb < TBS; ++tb) {
        const int tb0 = tb * 64;
        if (tb0 >= T) break;                                          // uniform
        const bool diag = tb == sb;
        __syncthreads();
        {   // C block, and dyc of every head (natural and transposed; lo natural)
            const rsrc_t rc = make_rsrc_u(Cbase + (int64_t)tb0 * GN, (uint32_t)(std::max(0, T - tb0) * GN * 2));
            for (int blk = tid; blk < 16 * (N / 8); blk += kThreads)
                block_both(rc, GN, blk & 15, (blk >> 4) * 8, Cn, LDB, CT, LDT, (blk >> 4) * 8);
            const rsrc_t rd = make_rsrc_u(k.dych + dbase + (int64_t)tb0 * xs + hfirst * kP,
                                        (uint32_t)(std::max(0, T - tb0) * xs * 2));
            for (int blk = tid; blk < HS * 128; blk += kThreads) {
                const int j = blk >> 7, rg = blk & 15, cg = (blk >> 4) & 7;
                if (j < nh)
                    block_both(rd, xs, rg, j * kP + cg * 8, Dh + j * 64 * LDX, LDX, DT + j * kP * LDT, LDT, cg * 8);
            }
            if constexpr (SPLIT) {
                const rsrc_t rl = make_rsrc_u(k.dycl + dbase + (int64_t)tb0 * xs + hfirst * kP,
                                            (uint32_t)(std::max(0, T - tb0) * xs * 2));
#pragma unroll
                for (int i = 0; i < HS * 64 * 8 / kThreads; ++i) {
                    const int v = tid + kThreads * i, j = v >> 9, row = (v >> 3) & 63, cv = v & 7;
                    if (j < nh)
                        *(u32x4 *)&Dl[(j * 64 + row) * LDX + cv * 8] = load16(rl, (uint32_t)((row * xs + j * kP + cv * 8) * 2));
                }
            }
        }
        __syncthreads();
        // (C_t.B_s): lane holds t = tb0 + 16u + 4kb + i, s = s0w + r16
        f32x4 cb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            cb[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (!diag || u >= wv) {
#pragma unroll
                for (int kk = 0; kk < KN; ++kk)
                    cb[u] = mfma16x16x32(
                        as_bf16x8(*(const u32x4 *)&Cn[(16 * u + r16) * LDB + ((32 * kk + 8 * kb) ^ nsw(16 * u + r16))]),
                        bfr[kk], cb[u]);
            }
        }
#pragma unroll
        for (int j = 0; j < HS; ++j) {
            if (j >= nh) break;                                       // uniform
            const int h = hfirst + j;
            const uint16_t *Dhj = Dh + j * 64 * LDX, *Dlj = Dl + j * 64 * LDX, *DTj = DT + j * kP * LDT;
            bf16x8 xf[2];
            load_x(h, xf);
            // (dyc_t.x_s), same layout as cb
            f32x4 dx4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dx4[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (!diag || u >= wv) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        dx4[u] = mfma16x16x32(
                            as_bf16x8(*(const u32x4 *)&Dhj[(16 * u + r16) * LDX + ((32 * kk + 8 * kb) ^ nsw(16 * u + r16))]),
                            xf[kk], dx4[u]);
                        if constexpr (SPLIT)
                            dx4[u] = mfma16x16x32(as_bf16x8(*(const u32x4 *)&Dlj[(16 * u + r16) * LDX + 32 * kk + 8 * kb]), xf[kk], dx4[u]);
                    }
                }
            }
            // M1[s,t] = Lm (C_t.B_s), M2[s,t] = Lm dt_s (dyc_t.x_s); W / dt_s = Lm (dyc_t.x_s) (C_t.B_s)
            const float cs_s = cs2[j][sl_col];
            const float dts_s = dts[j][sl_col];
            const float crr = cs2[j][rr];
            const float ws = diag ? 1.0f : fast_exp2(crr - cs_s);
            float wacc = 0.0f;
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                if (diag && 32 * a + 31 < 16 * wv) continue;          // every t of this half is before every row
                f32x4 m1[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int u = 2 * a + hh;
                    const int tlc = tb0 + 16 * u + 4 * kb;
                    const f32x4 ct4 = *(const f32x4 *)&cs2[j][tlc];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float lw;
                        if (diag) lw = tlc + i >= sl_col ? fast_exp2(ct4[i] - cs_s) : 0.0f;
                        else lw = ws * fast_exp2(ct4[i] - crr);
                        m1[hh][i] = lw * cb[u][i];
                        const float m = lw * dx4[u][i];
                        wacc = fmaf(m, cb[u][i], wacc);                // W / dt_s
                        dx4[u][i] = m * dts_s;
                    }
                }
                const bf16x8 f1 = afrag(m1[0], m1[1]);
                const bf16x8 f2 = afrag(dx4[2 * a], dx4[2 * a + 1]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dxa[j][q] = mfma16x16x32(f1, as_bf16x8(*(const u32x4 *)&DTj[(16 * q + r16) * LDT + 32 * a + 8 * kb]), dxa[j][q]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    db[nt] = mfma16x16x32(f2, as_bf16x8(*(const u32x4 *)&CT[(16 * nt + r16) * LDT + 32 * a + 8 * kb]), db[nt]);
            }
            wcol[j] += wacc;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // chunk-end terms, per head
#pragma unroll
    for (int j = 0; j < HS; ++j) {
        if (j >= nh) break;                                           // uniform
        const int h = hfirst + j;
        const float *gh = k.gout + ((((int64_t)b * p.nc + c) * p.H + h) * kP) * N;
        // x_s in the accumulator layout (rows s0w + 4kb + i, p = 16q + r16) and as the
        // A operand, loaded before the staging barrier so their latency overlaps it
        // (rows clamped into the chunk so the loads are unconditional and overlap; a
        // load under a branch is waited for at the branch's end, one at a time)
        float xv[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sl = s0w + 4 * kb + i, slc = std::min(sl, T - 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float xr = to_f32(p.x[(dbase + (int64_t)slc * xs) + h * kP + 16 * q + r16]);
                xv[i][q] = sl < T ? xr : 0.0f;
            }
        }
        bf16x8 xf[2];
        load_x(h, xf);
        __syncthreads();
        for (int blk = tid; blk < 16 * (N / 8); blk += kThreads)
            block_split_both(gh, N, blk & 15, blk >> 4, Gn, Gn + kP * LDB, LDB, GT, GT + N * LDT, LDT);
        __syncthreads();
        f32x4 xi[4], bi[NT];
#pragma unroll
        for (int q = 0; q < 4; ++q) xi[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bi[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            const uint16_t *G1 = Gn + part * kP * LDB, *G2 = GT + part * N * LDT;
            // B_s Gout^T: rows s = s0w + 4kb + i, p = 16q + r16
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int kk = 0; kk < KN; ++kk)
                    xi[q] = mfma16x16x32(
                        bfr[kk], as_bf16x8(*(const u32x4 *)&G1[(16 * q + r16) * LDB + ((32 * kk + 8 * kb) ^ nsw(16 * q + r16))]),
                        xi[q]);
            // x_s Gout: rows s, n = 16nt + r16
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    bi[nt] = mfma16x16x32(xf[kk], as_bf16x8(*(const u32x4 *)&G2[(16 * nt + r16) * LDT + 32 * kk + 8 * kb]), bi[nt]);
        }
        // rows s = s0w + 4kb + i
        const float cend = cs2[j][Q - 1];
        const f32x4 c4 = *(const f32x4 *)&cs2[j][s0w + 4 * kb];
        const f32x4 d4 = *(const f32x4 *)&dts[j][s0w + 4 * kb];
        const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;
        float xi_s[4], e_s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e_s[i] = fast_exp2(cend - c4[i]);
            float si = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                si = fmaf(xv[i][q], xi[q][i], si);
                dxa[j][q][i] = fmaf(e_s[i], xi[q][i], dxa[j][q][i]);    // dx / dt before D dyc
            }
            xi_s[i] = row16_sum(si);
            const float sc = d4[i] * e_s[i];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) db[nt][i] = fmaf(sc, bi[nt][i], db[nt][i]);
        }
        // dd_s = sum_{p,n} g_s x_s B_s = colsum(W / dt)_s + e_s x_s Gout B_s, from the
        // fp32 sums (not from the bf16-rounded dx product); dtdd = dt_s dd_s
        const float wsum = kb_sum(wcol[j]);
        if (kb == 0) qsh[wv][r16] = wsum;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (r16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) qsh[wv][4 * kb + i] += e_s[i] * xi_s[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (lane < 16 && s0w + lane < T) {
            const int64_t o = ((int64_t)b * p.L + t_base + s0w + lane) * p.H + h;
            const float ddv = qsh[wv][lane];
            k.dd[o] = ddv;
            k.dtdd[o] = dts[j][s0w + lane] * ddv;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // dx = dt_s (the tile) + D dyc_s, through the wave's LDS rows for 16-byte
        // stores (the rows alias Gout: every wave is done with it first)
        __syncthreads();
        float *ot = Ot + wv * 16 * LDO;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) ot[(4 * kb + i) * LDO + 16 * q + r16] = dxa[j][q][i] * d4[i];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        float dsum = 0.0f;                             // dDskip share (no gate: dyc = dy)
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
            const int row = rh * 8 + (lane >> 3), c8 = (lane & 7) * 8;
            const int sl = s0w + row;
            if (sl < T) {
                const int64_t e = dbase + (int64_t)sl * xs + h * kP + c8;
                const u32x4 gh8 = *(const u32x4 *)(k.dych + e);
                u32x4 gl8 = u32x4{0u, 0u, 0u, 0u};
                if constexpr (SPLIT) gl8 = *(const u32x4 *)(k.dycl + e);
                u32x4 xv8 = u32x4{0u, 0u, 0u, 0u};
                if (!SPLIT && k.dD) xv8 = *(const u32x4 *)(p.x + e);
                const f32x4 o0 = *(const f32x4 *)&ot[row * LDO + c8];
                const f32x4 o1 = *(const f32x4 *)&ot[row * LDO + c8 + 4];
                const float o[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
                u32x4 outv;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float g0 = bf16_lo(gh8[e2]) + bf16_lo(gl8[e2]);
                    const float g1 = bf16_hi(gh8[e2]) + bf16_hi(gl8[e2]);
                    outv[e2] = pack_bf16(fmaf(dsk, g0, o[2 * e2]), fmaf(dsk, g1, o[2 * e2 + 1]));
                    dsum = fmaf(g0, bf16_lo(xv8[e2]), dsum);
                    dsum = fmaf(g1, bf16_hi(xv8[e2]), dsum);
                }
                *(u32x4 *)(k.dx + e) = outv;
            }
        }
        if (!SPLIT && k.dD) {
            dsum = wave_sum(dsum);
            if (lane == 0) atomicAdd(k.dD + h, dsum);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    // dB share of this slice: rows s0w + 4kb + i, n = 16 nt + r16
    float *out = k.dBp + ((((int64_t)tl.sl * k.batch + b) * p.L + t_base) * p.G + g) * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = s0w + 4 * kb + i;
        if (sl < T) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) out[(int64_t)sl * GN + 16 * nt + r16] = db[nt][i];
        }
    }
}

// ---------------------------------------------------------------- finish
// One workgroup per (chunk, 64 heads, b); wave w takes the kFinSeg steps from
// kFinSeg w of the chunk and lane = head, so every (step, head) array is read and
// written as contiguous rows. da_t = sum over t' >= t in the chunk of (q - dtdd) plus
// <Gout, S_end>: each wave sums its steps, the totals of the later waves come through
// LDS, and each wave then walks its steps backwards. d dt = dd + A da; dA, d bias.
constexpr int kFinSeg = 16;

template <int Q>
__global__ __launch_bounds__(Q / kFinSeg * 64) void ssd_bwd_finish_kernel(const BwdK k) {
    constexpr int NW = Q / kFinSeg;
    const SSDK &p = k.f;
    const int c = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hh = hg * 64 + lane;
    const bool hok = hh < p.H;
    const int h = hok ? hh : p.H - 1;
    const int64_t t0 = (int64_t)c * Q + kFinSeg * wv;      // this wave's first step
    const int nt = (int)std::max<int64_t>(0, std::min<int64_t>(kFinSeg, p.L - t0));   // uniform
    // element of step t0 + j, the step clamped into the sequence (loaded, not used past it)
    auto at = [&](int j) { return ((int64_t)b * p.L + std::min<int64_t>(t0 + j, p.L - 1)) * p.H + h; };
    // <Gout, S_end> has kcw shares: wave w adds shares w, w + NW, ... (issued first, so
    // they overlap the loads below); the waves' parts are added through LDS in order
    const float *kcp = k.kc + (((int64_t)b * p.H + h) * p.nc + c) * k.kcw;
    float kpart = 0.0f;
    for (int w2 = wv; w2 < k.kcw; w2 += NW) kpart += kcp[w2];
    float r[kFinSeg], ddv[kFinSeg];
    uint16_t dtr[kFinSeg];
#pragma unroll
    for (int j = 0; j < kFinSeg; ++j) {                    // every load of the wave goes out at once
        const int64_t o = at(j);
        r[j] = k.q[o];
        ddv[j] = k.dtdd[o];
    }
#pragma unroll
    for (int j = 0; j < kFinSeg; ++j) {
        const int64_t o = at(j);
        dtr[j] = p.dt[o];
        r[j] = j < nt ? r[j] - ddv[j] : 0.0f;
        ddv[j] = k.dd[o];
    }
    float seg = 0.0f;
#pragma unroll
    for (int j = 0; j < kFinSeg; ++j) seg += r[j];
    __shared__ float segs[NW][64];
    __shared__ float kps[NW][64];
    __shared__ float red[2][NW][64];
    segs[wv][lane] = seg;
    kps[wv][lane] = kpart;
    __syncthreads();
    float v = 0.0f;
    for (int w2 = 0; w2 < NW; ++w2) v += kps[w2][lane];
    for (int w2 = NW - 1; w2 > wv; --w2) v += segs[w2][lane];
    const float Ah = p.A[h], bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int j = kFinSeg - 1; j >= 0; --j) {
        if (j >= nt) continue;                              // uniform
        v += r[j];                                          // da of step t0 + j
        const float raw = to_f32(dtr[j]) + bias;
        const float dtv = p.softplus ? softplus_f32(raw) : raw;
        const float ddt = ddv[j] + Ah * v;
        const float dr = p.softplus ? ddt * sigmoid_f32(raw) : ddt;
        if (hok) k.ddt[at(j)] = f32_to_bf16(dr);
        sa = fmaf(dtv, v, sa);
        sb += dr;
    }
    red[0][wv][lane] = sa;
    red[1][wv][lane] = sb;
    __syncthreads();
    if (wv == 0 && hok) {
        float a = 0.0f, bsum = 0.0f;
        for (int w2 = 0; w2 < NW; ++w2) {
            a += red[0][w2][lane];
            bsum += red[1][w2][lane];
        }
        atomicAdd(k.dA + h, a);
        if (k.dbias) atomicAdd(k.dbias + h, bsum);
    }
}

// dB, dC: the sum of the slices' shares
__global__ __launch_bounds__(256) void ssd_bwd_reduce_kernel(const float *part, int nsl, int64_t total, float *out) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= total) return;
    f32x4 s = *(const f32x4 *)(part + i);
    for (int q = 1; q < nsl; ++q) s += *(const f32x4 *)(part + (int64_t)q * total + i);
    *(f32x4 *)(out + i) = s;
}

__global__ __launch_bounds__(256) void ssd_bwd_zero_kernel(float *a, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) a[i] = 0.0f;
}

template <int N, int Q>
void launch_main(const BwdK &k, bool split, int nrow, int ncol, hipStream_t s) {
    if (split) {
        hipLaunchKernelGGL((ssd_bwd_row_kernel<N, Q, true>), dim3((unsigned)nrow), dim3(kThreads), 0, s, k);
        hipLaunchKernelGGL((ssd_bwd_col_kernel<N, Q, true>), dim3((unsigned)ncol), dim3(kThreads), 0, s, k);
    } else {
        hipLaunchKernelGGL((ssd_bwd_row_kernel<N, Q, false>), dim3((unsigned)nrow), dim3(kThreads), 0, s, k);
        hipLaunchKernelGGL((ssd_bwd_col_kernel<N, Q, false>), dim3((unsigned)ncol), dim3(kThreads), 0, s, k);
    }
    hipLaunchKernelGGL((ssd_bwd_finish_kernel<Q>), dim3((unsigned)k.f.nc, (unsigned)((k.f.H + 63) / 64),
                                                         (unsigned)k.batch),
                       dim3(Q / kFinSeg * 64), 0, s, k);
}

template <int N>
void launch_main_n(const BwdK &k, int Q, bool split, int nrow, int ncol, hipStream_t s) {
    switch (Q) {
        case 64: launch_main<N, 64>(k, split, nrow, ncol, s); break;
        case 128: launch_main<N, 128>(k, split, nrow, ncol, s); break;
        default: launch_main<N, 256>(k, split, nrow, ncol, s); break;
    }
}

void zero(float *a, int64_t n, hipStream_t s) {
    if (a && n > 0) hipLaunchKernelGGL(ssd_bwd_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, n);
}

}  // namespace

ssm_status ssd_bwd_launch(const ssm_ssd_bwd_args &a, const SSDBwdPlan &plan, hipStream_t s, char *err,
                          size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();
    const int64_t G = a.ngroups > 1 ? a.ngroups : 1;
    const int N = (int)a.dstate, Q = (int)a.chunk;
    if (a.seqlen == 0) {
        // no steps: every gradient is zero except dh0 = dh_final
        zero(a.dA, a.nheads, s);
        zero(a.dDskip, a.nheads, s);
        zero(a.ddt_bias, a.nheads, s);
        if (a.dh0) {
            const int64_t n = a.batch * a.nheads * a.headdim * a.dstate;
            if (a.dh_final)
                (void)hipMemcpyAsync(a.dh0, a.dh_final, n * 4, hipMemcpyDeviceToDevice, s);
            else
                zero(a.dh0, n, s);
        }
    } else {
        char *ws = (char *)a.workspace;
        BwdK k{};
        SSDK &f = k.f;
        f.x = (const uint16_t *)a.x; f.dt = (const uint16_t *)a.dt;
        f.Bm = (const uint16_t *)a.Bm; f.Cm = (const uint16_t *)a.Cm; f.z = (const uint16_t *)a.z;
        f.dt_bias = a.dt_bias; f.A = a.A; f.Dskip = a.Dskip; f.h0 = a.h0;
        f.y = nullptr;
        f.h_final = (float *)(ws + plan.hfin_offset);
        f.states = (float *)(ws + plan.sin32_offset);
        f.sin = (uint16_t *)(ws + plan.sin_offset);
        f.decay = (float *)(ws + plan.decay_offset);
        f.sin32 = f.states;                              // entering states replace the chunk states
        f.y32 = a.z ? (float *)(ws + plan.y32_offset) : nullptr;
        f.L = a.seqlen; f.H = (int32_t)a.nheads; f.nc = (int32_t)plan.nchunks;
        f.softplus = a.dt_softplus ? 1 : 0;
        f.G = (int32_t)G;
        f.hpg = (int32_t)(a.nheads / G);
        k.dy = (const uint16_t *)a.dy;
        k.dych = a.z ? (uint16_t *)(ws + plan.dych_offset) : (uint16_t *)a.dy;
        k.dycl = a.z ? (uint16_t *)(ws + plan.dycl_offset) : nullptr;
        k.dh_final = a.dh_final;
        k.dx = (uint16_t *)a.dx; k.ddt = (uint16_t *)a.ddt; k.dz = (uint16_t *)a.dz;
        k.dA = a.dA; k.dD = a.dDskip; k.dbias = a.ddt_bias; k.dh0 = a.dh0;
        k.sin32 = f.states;
        k.gout = (float *)(ws + plan.gout_offset);
        k.hfin = f.h_final;
        k.kc = (float *)(ws + plan.kc_offset);
        k.q = (float *)(ws + plan.q_offset);
        k.dtdd = (float *)(ws + plan.dtdd_offset);
        k.dd = (float *)(ws + plan.dd_offset);
        k.dBp = (float *)(ws + plan.dBp_offset);
        k.dCp = (float *)(ws + plan.dCp_offset);
        k.dB = a.dB; k.dC = a.dC;
        k.nsl_col = (int32_t)plan.slices_col;
        k.nsl_row = (int32_t)plan.slices_row;
        k.batch = (int32_t)a.batch;
        k.kcw = (int32_t)(a.headdim * a.dstate / 256);   // (P N / 4) threads per (b, h) / 64

        zero(a.dA, a.nheads, s);
        zero(a.dDskip, a.nheads, s);
        zero(a.ddt_bias, a.nheads, s);
        // forward recompute: chunk states (split), entering states, final state
        ssd_recompute_launch(f, (int)a.batch, Q, N, 0, s);
        if (a.z) ssd_recompute_launch(f, (int)a.batch, Q, N, 1, s);   // fp32 pre-gate output
        // gate: dD (and dz, dyc with z)
        const int64_t rows = a.batch * a.seqlen;
        const dim3 ggrid((unsigned)((rows + 255) / 256), (unsigned)a.nheads);
        if (a.z) hipLaunchKernelGGL(ssd_bwd_gate_kernel, ggrid, dim3(256), 0, s, k, rows);
        // without z, dDskip is summed by the column kernel (dyc = dy)
        // adjoint aggregates: the chunk-state kernel with x := dyc, B := C, exp(cs_t)
        // weights, output into the Gout buffer
        {
            SSDK fa = f;
            fa.x = k.dych;
            fa.xlo = k.dycl;
            fa.Bm = f.Cm;
            fa.states = k.gout;
            ssd_recompute_launch(fa, (int)a.batch, Q, N, 2, s);
        }
        const int64_t total = a.batch * a.nheads * a.headdim * a.dstate / 4;
        hipLaunchKernelGGL(ssd_bwd_state_pass_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                           k, N, total);
        const int tbs = Q / 64;
        const int nrow = (int)(a.batch * plan.nchunks * G * plan.slices_row * tbs);
        const int ncol = (int)(a.batch * plan.nchunks * G * plan.slices_col * tbs);
        if (N == 64) launch_main_n<64>(k, Q, a.z != nullptr, nrow, ncol, s);
        else if (N == 128) launch_main_n<128>(k, Q, a.z != nullptr, nrow, ncol, s);
        else launch_main_n<256>(k, Q, a.z != nullptr, nrow, ncol, s);
        const int64_t bln = a.batch * a.seqlen * G * a.dstate;
        hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3((unsigned)((bln / 4 + 255) / 256)), dim3(256), 0, s,
                           (const float *)k.dBp, (int)plan.slices_col, bln, a.dB);
        hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3((unsigned)((bln / 4 + 255) / 256)), dim3(256), 0, s,
                           (const float *)k.dCp, (int)plan.slices_row, bln, a.dC);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(err, errlen, "ssd_chunked_bwd: kernel launch failed: %s", hipGetErrorString(e));
        return SSM_EHIP;
    }
    return SSM_OK;
}

}  // namespace ssm
