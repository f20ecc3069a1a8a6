// Scalar-A state-space form (Mamba-2 "SSD") for gfx950, on the matrix cores.
//
// With one scalar decay per head the mixing matrix of a chunk is semiseparable:
// inside a chunk of Q steps, y = (L o C B^T o exp(cs_t - cs_s) o dt_s) x, and the
// influence of everything before the chunk passes through one N x P state per
// head [Mamba-2 page "Mamba-2：把状态空间模型和 Attention 统一到一个数学框架里", Core
// idea step 2 (the SSM as a structured attention-like matrix y = (L o M) x) and key
// point 1 (semiseparable: every off-diagonal block is low rank, O(L) storage)].
// With cs_t = sum_{k<=t in chunk} A dt_k:
//   state of chunk c  : S_c = sum_s exp(cs_end - cs_s) dt_s B_s (x) x_s   (N x P)
//   entering state    : Sin_0 = h0, Sin_{c+1} = exp(cs_end,c) Sin_c + S_c
//   output            : y_t = sum_{s<=t} (C_t.B_s) exp(cs_t - cs_s) dt_s x_s
//                            + exp(cs_t) C_t . Sin_c + D x_t,   then * silu(z_t)
//
// Three launches per call (matrix cores, fp32 accumulation):
//   1. ssd_chunk_state: per (batch, chunk, 4 heads), v_mfma_f32_16x16x32_bf16. B
//      of the chunk is transposed into LDS once and shared by the 4 heads (one wave
//      each); x is transposed and scaled by exp(cs_end - cs_s) dt_s while staging.
//      S_c is written in bf16, layout [p][n] (fp32 in the gradient pass's
//      recompute). In the forward, extra workgroups of the same launch form the score
//      blocks G^T = B C^T of every (batch, chunk, group) once, in fp32, on
//      v_mfma_f32_32x32x16_bf16: every head of the group reads them.
//   2. ssd_state_pass: sequential over chunks per (batch, head, p, 4 n); writes the
//      entering state of every chunk already rounded to bf16 in the [p][n] layout
//      the output kernels read as MFMA B fragments, and h_final in fp32.
//   3. ssd_out_head (the forward): per (batch, chunk, head), Q/64 waves on 32 x 32
//      tiles, each wave owning the tiles w and Q/32 - 1 - w (equal causal work).
//      x is staged transposed in LDS once; each score block is read from L2, scaled
//      by the decays in registers and rounded to bf16 straight into the A operand
//      of Y += M X (x stored with the matching order of s, which the contraction
//      over s does not care about). The carried state enters as exp(cs_t) (C Sin)
//      on the same units; D x and the gate are applied in fp32 on the way out.
//      ssd_chunk_out (the fp32 pre-gate recompute of the gradient pass): per
//      (batch, chunk, pair of heads), one 16-row tile per wave (at chunk 256 split
//      over two workgroups); B and x stream through LDS in 64-row blocks of s, and
//      the score tile is formed on the MFMA units for each block.
// Transposes into LDS move 4 x 8 register blocks with byte permutes and 8-byte
// LDS writes.
#include <algorithm>
#include <cstdio>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

#include "ssd_common.h"

namespace ssm {
namespace {

// ---------------------------------------------------------------- score blocks
// G^T = B C^T of a chunk in 32 x 32 blocks (rows s of block sb, columns t of tile
// tau, sb <= tau), on v_mfma_f32_32x32x16_bf16, kept in fp32 as the matrix cores
// accumulate it. G depends on the group's B and C only, so it is formed once per
// (batch, chunk, group), by extra workgroups of the chunk-state kernel, and read by
// every head of the group.
//
// In the 32 x 32 accumulator layout (register v of lane l: row 8 (v >> 2) + 4 (l >> 5)
// + (v & 3), column l & 31) a block is stored as 4 runs
// of 256 floats, run i holding registers 4i .. 4i + 3 of lanes 0 .. 63 in order,
// so that each of the 4 loads (and stores) of a lane's 16 values moves 1 KiB of
// contiguous memory per wave. Block (tau, sb) of (batch, chunk, group) qg sits at
// (qg NB + tau (tau + 1) / 2 + sb) 1024 floats, NB = Q/32 (Q/32 + 1) / 2. Tiles
// with no step of the sequence are left out (and never read).
template <int Q>
constexpr int score_blocks() { return (Q / 32) * (Q / 32 + 1) / 2; }

// Score blocks (tau, 0 .. tau) of (batch, chunk) q and group gg, by one wave.
template <int N, int Q>
__device__ __forceinline__ void score_tile(const SSDK &p, int64_t q, int gg, int tau) {
    constexpr int NB = score_blocks<Q>(), KN = N / 16;
    const int c = (int)(q % p.nc), b = (int)(q / p.nc);
    const int lane = threadIdx.x & 63, c32 = lane & 31, hf = lane >> 5;
    const int64_t t_base = (int64_t)c * Q;
    const int T = (int)std::min<int64_t>(Q, p.L - t_base);
    if (32 * tau >= T) return;                                 // no step in this tile (uniform)
    const int GN = p.G * N;
    const rsrc_t rC = make_rsrc_u(p.Cm + (((int64_t)b * p.L + t_base) * p.G + gg) * N, (uint32_t)(T * GN * 2));
    const rsrc_t rB = make_rsrc_u(p.Bm + (((int64_t)b * p.L + t_base) * p.G + gg) * N, (uint32_t)(T * GN * 2));
    bf16x8 cfr[KN], bfa[KN], bfb[KN];
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
        cfr[kk] = as_bf16x8(load16(rC, (uint32_t)(((32 * tau + c32) * GN + 16 * kk + 8 * hf) * 2)));
    auto load_b = [&](int sb, bf16x8 (&dst)[KN]) {
#pragma unroll
        for (int kk = 0; kk < KN; ++kk)
            dst[kk] = as_bf16x8(load16(rB, (uint32_t)(((32 * sb + c32) * GN + 16 * kk + 8 * hf) * 2)));
    };
    float *out = p.gsc + ((q * p.G + gg) * NB + tau * (tau + 1) / 2) * 1024 + lane * 4;
    auto block = [&](int sb, const bf16x8 (&bf)[KN]) {
        f32x16 g = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) g = mfma32x32x16(bf[kk], cfr[kk], g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(f32x4 *)(out + sb * 1024 + i * 256) = f32x4{g[4 * i], g[4 * i + 1], g[4 * i + 2], g[4 * i + 3]};
    };
    load_b(0, bfa);
    for (int sb = 0;;) {
        if (sb < tau) load_b(sb + 1, bfb);
        block(sb, bfa);
        if (++sb > tau) break;
        if (sb < tau) load_b(sb + 1, bfa);
        block(sb, bfb);
        if (++sb > tau) break;
    }
}

// ---------------------------------------------------------------- chunk states
// MODE 0: S_c = sum_s exp(cs_end - cs_s) dt_s B_s (x) x_s, the weighted x rounded to
//         bf16, S_c stored in bf16 (the forward: the entering states it feeds are
//         rounded to bf16 anyway); the last chunk's, which only enters h_final, in
//         fp32;
// MODE 1: the same with the weighted x split into bf16 hi + lo parts, two products
//         (fp32-grade chunk states, for the gradient pass);
// MODE 2: R_c = sum_t exp(cs_t) B_t (x) (x_t + xlo_t), split like MODE 1, no decay
//         output (with x + xlo = dy silu(z) and B = C this is the adjoint aggregate
//         of the gradient pass).
template <int N, int Q, int MODE>
__global__ __launch_bounds__(kThreads, (N > 128 || MODE != 0) ? 1 : 2) void ssd_chunk_state_kernel(const SSDK p,
                                                                                                int64_t nq, int nscore) {
    constexpr bool SPLIT = MODE != 0;
    constexpr int SB = 64;                    // time rows staged per step
    constexpr int LDT = SB + 8;               // padded LDS row (bf16)
    constexpr int NPASS = N > 128 ? N / 128 : 1;
    constexpr int NP = N / NPASS;             // states handled per pass (<= 128)
    constexpr int NT = NP / 16;               // n tiles per pass
    constexpr int SPL = Q / 64;
    __shared__ float wsh[4][Q];
    __shared__ __attribute__((aligned(16))) uint16_t BT[NP][LDT];
    __shared__ __attribute__((aligned(16))) uint16_t XT[4][kP][LDT];
    __shared__ __attribute__((aligned(16))) uint16_t XL[SPLIT ? 4 : 1][SPLIT ? kP : 1][SPLIT ? LDT : 8];

    // block -> ((batch, chunk) q, head block). Workgroup i runs on XCD i % 8, and
    // q % 8 = i % 8 here, so every head block of a chunk runs on one XCD: the chunk's
    // B rows come into one L2 instead of all eight. Neighbouring ids are neighbouring
    // chunks, so the workgroups of a chunk still run close together in time.
    if constexpr (MODE == 0) {
        // the first nscore workgroups (a multiple of 8; dispatched first, so they run
        // beside the chunk states) form the score blocks: one per (batch, chunk,
        // group), on the XCD of the chunk; wave w takes tiles w and Q/32 - 1 - w
        // (equal causal work)
        if ((int)blockIdx.x < nscore) {
            const int64_t sid = blockIdx.x;
            const int64_t k8 = sid >> 3;
            const int64_t q = (k8 / p.G) * 8 + (sid & 7);
            const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
            if (q >= nq || 2 * w >= Q / 32) return;
            score_tile<N, Q>(p, q, (int)(k8 % p.G), w);
            score_tile<N, Q>(p, q, (int)(k8 % p.G), Q / 32 - 1 - w);
            return;
        }
    }
    const int hb = (p.hpg + 3) / 4;                   // workgroups per group of heads
    const int upc = p.G * hb;                         // workgroups per (batch, chunk)
    const int bid = (int)blockIdx.x - nscore;
    const int k8 = bid >> 3;
    const int64_t q = (int64_t)(k8 / upc) * 8 + (bid & 7);
    if (q >= nq) return;                              // whole workgroup (uniform)
    const int unit = k8 % upc;
    const int c = (int)(q % p.nc), b = (int)(q / p.nc);
    // the wave index is uniform: readfirstlane keeps it (and every address built
    // from it) in SGPRs, so buffer resources need no per-lane loop
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, kb = lane >> 4;
    const int g = unit / hb, hl = (unit % hb) * 4 + wv;
    const bool head_ok = hl < p.hpg;
    const int h = g * p.hpg + (head_ok ? hl : p.hpg - 1);   // clamped into the group
    const int hc = h;
    const int64_t t_base = (int64_t)c * Q;

    {   // per-head weights w_s = exp(cs_end - cs_s) dt_s and the chunk decay
        float dtv[SPL], cs[SPL];
        const float cs_end = head_dt_cs<Q>(p, b, hc, c, dtv, cs);
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            wsh[wv][lane * SPL + i] = MODE == 2 ? fast_exp2(cs[i] * kLog2e)
                                                : fast_exp2((cs_end - cs[i]) * kLog2e) * dtv[i];
        if (MODE != 2 && lane == 0 && head_ok)
            p.decay[((int64_t)b * p.H + h) * p.nc + c] = fast_exp2(cs_end * kLog2e);
    }

    // One 64-row block of B (this pass's states) and of x (this wave's head) is
    // loaded into registers while the previous one is multiplied. Consecutive lanes
    // read consecutive 16-byte pieces of a row (16 lanes per B row, 8 per x row).
    // In the transposed LDS copies, row r (a state n or a head-dim p) holds time
    // position j at column j ^ sw(r), sw(r) = 8 ((r >> 3) & 7), so that the lanes
    // writing 8 rows r, r + 8, .. at once start in different banks.
    const int GN = p.G * N;
    const int sg = tid >> 4, co = tid & 15;           // B block of this thread: 4 rows x 8 states
    u32x4 breg[4], xreg[2][4], xlreg[MODE == 2 ? 2 : 1][4];
    const bool has_lo = MODE == 2 && p.xlo != nullptr;
    auto fetch = [&](int pass, int s0) {
        const int rows = (int)std::max<int64_t>(0, std::min<int64_t>(SB, p.L - t_base - s0));
        const rsrc_t rb = make_rsrc_u(p.Bm + (((int64_t)b * p.L + t_base + s0) * p.G + g) * N + pass * NP,
                                    (uint32_t)(rows * GN * 2));
        const rsrc_t rx = make_rsrc_u(p.x + (((int64_t)b * p.L + t_base + s0) * p.H + hc) * kP,
                                    (uint32_t)(rows * p.H * kP * 2));
#pragma unroll
        for (int i = 0; i < 4; ++i) breg[i] = load16(rb, (uint32_t)(((sg * 4 + i) * GN + co * 8) * 2));
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int blk = lane + 64 * k, xg = blk >> 3, po = blk & 7;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xreg[k][i] = load16(rx, (uint32_t)(((xg * 4 + i) * p.H * kP + po * 8) * 2));
        }
        if constexpr (MODE == 2) {
            if (has_lo) {
                const rsrc_t rl = make_rsrc_u(p.xlo + (((int64_t)b * p.L + t_base + s0) * p.H + hc) * kP,
                                            (uint32_t)(rows * p.H * kP * 2));
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int blk = lane + 64 * k, xg = blk >> 3, po = blk & 7;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xlreg[k][i] = load16(rl, (uint32_t)(((xg * 4 + i) * p.H * kP + po * 8) * 2));
                }
            }
        }
    };
    auto stash = [&](int s0) {
        if (co < NP / 8) store_transposed(breg, &BT[0][0], LDT, co * 8, (sg * 4) ^ ((co & 7) << 3));
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int blk = lane + 64 * k, xg = blk >> 3, po = blk & 7;
            u32x4 r[4], rl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float w = wsh[wv][s0 + xg * 4 + i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x0 = bf16_lo(xreg[k][i][e]), x1 = bf16_hi(xreg[k][i][e]);
                    if constexpr (MODE == 2) {
                        if (has_lo) {
                            x0 += bf16_lo(xlreg[k][i][e]);
                            x1 += bf16_hi(xlreg[k][i][e]);
                        }
                    }
                    const float v0 = x0 * w, v1 = x1 * w;
                    r[i][e] = pack_bf16(v0, v1);
                    if constexpr (SPLIT)
                        rl[i][e] = pack_bf16(v0 - bf16_lo(r[i][e]), v1 - bf16_hi(r[i][e]));
                }
            }
            store_transposed(r, &XT[wv][0][0], LDT, po * 8, (xg * 4) ^ (po << 3));
            if constexpr (SPLIT) store_transposed(rl, &XL[wv][0][0], LDT, po * 8, (xg * 4) ^ (po << 3));
        }
    };

    auto sw = [](int r) { return ((r >> 3) & 7) << 3; };
    constexpr int NBLK = Q / SB;
    fetch(0, 0);
    for (int pass = 0; pass < NPASS; ++pass) {
        f32x4 acc[NT][4];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int blk = 0; blk < NBLK; ++blk) {
            const int s0 = blk * SB;
            __syncthreads();                              // previous block's MFMA reads are done
            stash(s0);
            // the next block (or the first of the next pass)
            if (blk + 1 < NBLK) fetch(pass, s0 + SB);
            else if (pass + 1 < NPASS) fetch(pass + 1, 0);
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < SB / 32; ++kk) {
                const int sk = kk * 32 + kb * 8;
                bf16x8 bfr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) bfr[j] = as_bf16x8(*(const u32x4 *)&XT[wv][j * 16 + r16][sk ^ sw(j * 16 + r16)]);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const bf16x8 afr = as_bf16x8(*(const u32x4 *)&BT[i * 16 + r16][sk ^ sw(i * 16 + r16)]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(afr, bfr[j], acc[i][j]);
                }
                if constexpr (SPLIT) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) bfr[j] = as_bf16x8(*(const u32x4 *)&XL[wv][j * 16 + r16][sk ^ sw(j * 16 + r16)]);
#pragma unroll
                    for (int i = 0; i < NT; ++i) {
                        const bf16x8 afr = as_bf16x8(*(const u32x4 *)&BT[i * 16 + r16][sk ^ sw(i * 16 + r16)]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(afr, bfr[j], acc[i][j]);
                    }
                }
            }
        }
        // S_c[p][n]: lane holds n = pass*NP + 16i + 4kb + e, p = 16j + r16 -> 16-byte
        // stores, 4 lanes covering 64 contiguous bytes of a row. In bf16 (the forward)
        // lanes kb and kb ^ 1 trade halves of tiles i and i + 1 first, so that a lane
        // holds 8 consecutive n: n = 16i + 8(kb / 2) .. for even kb, n = 16i + 16 +
        // 8(kb / 2) .. for odd kb.
        if (head_ok) {
            // Opaque copies of the lane's indices keep the store addresses formed here:
            // formed before the products, they were spilled and reloaded from scratch.
            int hq = h, r16 = lane & 15, kb = lane >> 4;
            asm volatile("" : "+v"(hq), "+v"(r16), "+v"(kb));
            const int64_t o = (((int64_t)b * p.nc + c) * p.H + hq) * (int64_t)kP * N;
            if (MODE == 0 && c == p.nc - 1) {
                // the last chunk's state only enters h_final: kept in fp32
                float *out = p.states_last + ((int64_t)b * p.H + hq) * (int64_t)kP * N;
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *(f32x4 *)(out + (j * 16 + r16) * N + pass * NP + i * 16 + kb * 4) = acc[i][j];
            } else if constexpr (MODE == 0) {
                static_assert(NT % 2 == 0, "tiles are paired");
                const bool odd = kb & 1;
#pragma unroll
                for (int i = 0; i < NT; i += 2)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u32x2 lo = u32x2{pack_bf16(acc[i][j][0], acc[i][j][1]),
                                               pack_bf16(acc[i][j][2], acc[i][j][3])};
                        const u32x2 hi = u32x2{pack_bf16(acc[i + 1][j][0], acc[i + 1][j][1]),
                                               pack_bf16(acc[i + 1][j][2], acc[i + 1][j][3])};
                        const u32x2 give = odd ? lo : hi;
                        const u32x2 got = u32x2{(uint32_t)__shfl_xor((int)give[0], 16, 64),
                                                (uint32_t)__shfl_xor((int)give[1], 16, 64)};
                        const u32x4 out = odd ? u32x4{got[0], got[1], hi[0], hi[1]}
                                              : u32x4{lo[0], lo[1], got[0], got[1]};
                        const int n0 = pass * NP + i * 16 + (odd ? 16 : 0) + (kb >> 1) * 8;
                        *(u32x4 *)(p.states16 + o + (j * 16 + r16) * N + n0) = out;
                    }
            } else {
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *(f32x4 *)(p.states + o + (j * 16 + r16) * N + pass * NP + i * 16 + kb * 4) = acc[i][j];
            }
        }
    }
}

// ---------------------------------------------------------------- state passing
// One thread per (b, h, p, 4 consecutive n), sequential over chunks. The chunk states
// of a group of K chunks are loaded together so their latencies overlap, and the
// next group's loads go out before this group's stores: the memory counter completes
// in order, so waiting for a load issued after a store would also wait for the store.
// S16: the forward (bf16 chunk states, the last chunk's in fp32, bf16 entering states
// only); otherwise the gradient pass (fp32 chunk states, and the fp32 entering states
// written over them: chunk c's slot is rewritten only after chunk c has been loaded).
template <bool S16>
__global__ __launch_bounds__(256) void ssd_state_pass_kernel(const SSDK p, int N, int64_t total) {
    constexpr int K = 8;
    typedef typename std::conditional<S16, u32x2, f32x4>::type Raw;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t per_bh = (int64_t)kP * N / 4;
    const int64_t bh = i / per_bh;            // b*H + h
    const int64_t pn = (i % per_bh) * 4;      // p*N + n
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t hidx = bh * kP * N + pn;    // (b, h, p, n) of h0 / h_final
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.h0) {   // h0 and h_final are only 4-byte aligned
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = p.h0[hidx + e];
    }
    const float *dec = p.decay + bh * p.nc;
    const int64_t cstride = (int64_t)p.H * kP * N;
    const int64_t base = (b * p.nc * p.H + h) * kP * N + pn;
    f32x4 last = f32x4{0.f, 0.f, 0.f, 0.f};   // the forward's last chunk state, fp32
    if constexpr (S16) last = *(const f32x4 *)(p.states_last + bh * kP * N + pn);
    // chunks past the end are clamped to the last one (loaded again, not used)
    auto load_group = [&](int c0, Raw (&r)[K], float (&d)[K]) {
#pragma unroll
        for (int u = 0; u < K; ++u) {
            const int cc = min(c0 + u, p.nc - 1);
            if constexpr (S16) r[u] = *(const u32x2 *)(p.states16 + base + cc * cstride);
            else r[u] = *(const f32x4 *)(p.states + base + cc * cstride);
            d[u] = dec[cc];
        }
    };
    Raw cur[K], nxt[K];
    float dcur[K], dnxt[K];
    load_group(0, cur, dcur);
    for (int c0 = 0; c0 < p.nc; c0 += K) {
        load_group(c0 + K, nxt, dnxt);
        // In the forward the entering states overwrite the chunk states in place
        // (sin == states16): each thread writes only the elements it read, and
        // every chunk state of the group is unpacked (its load has returned) before
        // the first store of the group is issued.
        f32x4 scv[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            if constexpr (S16) {
                const u32x2 v = cur[u];
                scv[u] = c0 + u == p.nc - 1 ? last
                                            : f32x4{bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])};
            } else {
                scv[u] = cur[u];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < K; ++u) {
            if (c0 + u < p.nc) {
                const f32x4 sc = scv[u];
                *(u32x2 *)(p.sin + base + (c0 + u) * cstride) = u32x2{pack_bf16(s[0], s[1]), pack_bf16(s[2], s[3])};
                if constexpr (!S16) *(f32x4 *)(p.sin32 + base + (c0 + u) * cstride) = s;
#pragma unroll
                for (int e = 0; e < 4; ++e) s[e] = fmaf(dcur[u], s[e], sc[e]);
            }
        }
#pragma unroll
        for (int u = 0; u < K; ++u) {
            cur[u] = nxt[u];
            dcur[u] = dnxt[u];
        }
    }
    if (p.h_final) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p.h_final[hidx + e] = s[e];
    }
}

// ---------------------------------------------------------------- chunk output
// Per (batch, chunk, pair of heads of one B/C group); each wave owns 16 rows of the
// chunk for both heads. The prologue of a chunk (dt and cumulative decays, the
// entering states, C rows) is done once per workgroup for all of its rows, and each
// 64-row block of B and x is loaded once and used by every wave whose rows come at
// or after it. The score tile G^T = B C^T is computed once per wave and reused by
// both heads: only the decay weights differ per head.
//
// With r = 64 tb - 1 (the last step before the time block; cs_r = 0 for tb = 0)
// the decay of s <= r < t factors as exp(cs_t - cs_s) = a_t w_s, a_t = exp(cs_t -
// cs_r), w_s = exp(cs_r - cs_s), both <= 1. So for every block of s before the
// time block, M = G o (w_s dt_s) needs no exponential per element; those blocks and
// the entering state (exp(cs_t) C Sin = a_t exp(cs_r) C Sin) accumulate into one
// tile that is scaled by a_t once, after which the diagonal block adds its terms
// with the exact per-element weight exp(cs_t - cs_s) dt_s [s <= t]. w_s dt_s is
// tabulated per time block.
//
// Layouts in LDS: B rows natural ([s][n], the A operand of G^T); x transposed per
// head ([p][s], the B operand of Y += M X) with s permuted inside each 32-block so
// that a lane's 8 k-values (s = 32a + 16h + 4kb + i, h, i in 0..1, 0..3 from the
// accumulator layout of G^T) sit in 16 contiguous bytes. The next block of B and x
// is loaded into registers while the current one is computed.
template <int N>
struct OutCfg {
    static constexpr int HG = 2;   // heads per workgroup
};

// Workgroups per (chunk, head pair). At chunk 256 two 8-wave workgroups share the
// chunk's time blocks (0 and 3, 1 and 2: equal causal work), so two of them fit a CU
// and one's loads overlap the other's arithmetic. With N = 256 the C fragments do
// not fit the 128 registers that takes.
template <int N, int Q>
constexpr int out_split() { return Q == 256 && N <= 128 ? 2 : 1; }

// It writes the pre-gate output (C S + D x) in fp32 to y32: the recompute the
// gradient pass needs for dz (the forward's gated bf16 y comes from ssd_out_head).
template <int N, int Q>
__global__ __launch_bounds__((Q * 4 / out_split<N, Q>()), (out_split<N, Q>() == 2 ? 4 : 2))
void ssd_chunk_out_kernel(const SSDK p, int nhg, int64_t nq) {
    constexpr int HG = OutCfg<N>::HG;
    constexpr int SPLIT = out_split<N, Q>();  // workgroups per (chunk, head pair)
    constexpr int NW = Q / (16 * SPLIT);      // waves, 16 rows each
    constexpr int NTH = NW * 64;              // threads
    constexpr int TBS = Q / 64;               // 64-row time blocks per chunk
    constexpr int KN = N / 32;                // k steps over the state dimension
    constexpr int SPL = Q / 64;
    constexpr int LDB = N + 8;                // padded bf16 rows of B and Sin
    constexpr int LDX = 64 + 8;               // padded bf16 rows of transposed x
    constexpr int LDO = kP + 4;               // padded fp32 rows of the output tile
    constexpr int SIN_HEADS = 2;              // heads of Sin staged together
    constexpr int BB_BYTES = 64 * LDB * 2;
    constexpr int XT_BYTES = HG * kP * LDX * 2;
    constexpr int SIN_BYTES = SIN_HEADS * kP * LDB * 2;
    constexpr int OT_BYTES = NW * 16 * LDO * 4;
    constexpr int R0_BYTES = std::max(BB_BYTES, OT_BYTES);   // B block, later the output tiles
    constexpr int U_BYTES = std::max(R0_BYTES + XT_BYTES, SIN_BYTES);
    constexpr int NBV = 64 * N / 8;           // 16-byte B vectors per block
    constexpr int BV = (NBV + NTH - 1) / NTH;
    constexpr int NXV = HG * 64 * 8;          // 16-byte x vectors (8 p of one row) per block
    constexpr int XV = (NXV + NTH - 1) / NTH;
    constexpr int NSV = SIN_HEADS * kP * N / 8;   // 16-byte Sin vectors per staging
    constexpr int SV = (NSV + NTH - 1) / NTH;
    static_assert(NTH % 64 == 0 && NXV % 64 == 0, "staging split is per wave");
    __shared__ float cs2[HG][Q];              // cs * log2(e) per head
    __shared__ float dts[HG][Q];              // dt (0 past the end of the sequence)
    __shared__ float wts[TBS][HG][Q];         // w_s dt_s of time block tb (s < 64 tb)
    __shared__ __attribute__((aligned(16))) uint8_t ubuf[U_BYTES];
    uint16_t (*Bb)[LDB] = reinterpret_cast<uint16_t (*)[LDB]>(ubuf);
    uint16_t (*XT)[kP][LDX] = reinterpret_cast<uint16_t (*)[kP][LDX]>(ubuf + R0_BYTES);
    uint16_t (*SinL)[kP][LDB] = reinterpret_cast<uint16_t (*)[kP][LDB]>(ubuf);
    float (*Ot)[16][LDO] = reinterpret_cast<float (*)[16][LDO]>(ubuf);

    // block -> (chunk, head pair, part); the workgroups of one chunk share an XCD, so
    // the chunk's B and C rows (and a head pair's entering states) are shared in its L2
    const int upc = p.G * nhg * SPLIT;                 // workgroups per chunk
    const int id = blockIdx.x, k8 = id >> 3;
    const int64_t q = (int64_t)(k8 / upc) * 8 + (id & 7);
    if (q >= nq) return;                               // whole workgroup (uniform)
    const int unit = k8 % upc;
    const int part = unit % SPLIT, hp = unit / SPLIT;
    const int hl = hp % nhg, gg = hp / nhg;
    const int c = (int)(q % p.nc), b = (int)(q / p.nc);
    // the wave index is uniform: readfirstlane keeps it (and every address built
    // from it) in SGPRs, so buffer resources need no per-lane loop
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, kb = lane >> 4;
    const int64_t t_base = (int64_t)c * Q;
    const int T = (int)std::min<int64_t>(Q, p.L - t_base);
    const int nsb = (T + 63) / 64;                     // 64-row blocks holding steps
    if (SPLIT == 2 && part == 1 && nsb <= 1) return;   // its blocks 1 and 2 are empty (uniform)
    // this wave's 16 rows. Split chunk: waves 0-3 own the first time block of the part
    // (0 or 1), waves 4-7 the second (3 or 2).
    const int t0 = SPLIT == 2 ? (wv < 4 ? part : 3 - part) * 64 + (wv & 3) * 16 : wv * 16;
    const int tb = t0 >> 6;                            // the time block of its rows
    // blocks of s this workgroup stages: up to its last time block
    const int nsw = std::min(nsb, SPLIT == 2 ? 4 - part : TBS);
    const int tl0 = (t0 >> 4) & 3;                     // index of its 16 rows within it
    const bool live = tb < nsb;                        // the block has steps (uniform)
    const int h0 = gg * p.hpg + hl * HG;               // first head of this workgroup
    const int hend = (gg + 1) * p.hpg;                 // heads of the group end here
    const int GN = p.G * N;                            // B, C elements per time step

    const uint16_t *Brow = p.Bm + (((int64_t)b * p.L + t_base) * p.G + gg) * N;
    const uint16_t *Crow = p.Cm + (((int64_t)b * p.L + t_base) * p.G + gg) * N;
    const int64_t xstride = (int64_t)p.H * kP;
    const uint16_t *Xrow = p.x + ((int64_t)b * p.L + t_base) * xstride;

    // next block of B and x into registers. Buffer resources cover the rows of the
    // block that exist (s < T), so rows past the sequence read as 0; a head past H
    // gets an offset outside every resource. Threads past the vectors of a block
    // load nothing (whole waves, so the tests are uniform). A lane holds one row of
    // 8 p of x (8 lanes read a 128-byte row) and writes its 8 values into the
    // transposed rows one by one, starting at element pc so that the 8 lanes of a
    // row write to 8 different p rows (different banks) at every step.
    u32x4 breg[BV], xreg[XV];
    uint32_t boff[BV], xoff[XV];
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int v = tid + i * NTH;
        boff[i] = (uint32_t)(v / (N / 8) * GN + (v % (N / 8)) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        const int v = tid + i * NTH;
        const int pc = v & 7, sr = (v >> 3) & 63, j = v >> 9;
        xoff[i] = (v < NXV && h0 + j < hend) ? (uint32_t)((sr * xstride + (h0 + j) * kP + pc * 8) * 2)
                                             : 0x80000000u;
    }
    auto fetch = [&](int sb) {
        const int s0 = sb * 64;
        const int rows = std::max(0, T - s0);
        const rsrc_t rb = make_rsrc_u(Brow + (int64_t)s0 * GN, (uint32_t)(rows * GN * 2));
        const rsrc_t rx = make_rsrc_u(Xrow + (int64_t)s0 * xstride, (uint32_t)(rows * xstride * 2));
#pragma unroll
        for (int i = 0; i < BV; ++i)
            if (wv * 64 + i * NTH < NBV) breg[i] = load16(rb, boff[i]);
#pragma unroll
        for (int i = 0; i < XV; ++i)
            if (wv * 64 + i * NTH < NXV) xreg[i] = load16(rx, xoff[i]);
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int v = tid + i * NTH;
            if (wv * 64 + i * NTH < NBV) *(u32x4 *)&Bb[v / (N / 8)][(v % (N / 8)) * 8] = breg[i];
        }
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int v = tid + i * NTH;
            if (wv * 64 + i * NTH < NXV) {
                const int pc = v & 7, sr = (v >> 3) & 63, j = v >> 9;
                // rotate the 8 values so that element e is the row's element (e + pc) & 7
                u32x4 w = xreg[i];
                if (pc & 4) w = u32x4{w[2], w[3], w[0], w[1]};
                if (pc & 2) w = u32x4{w[1], w[2], w[3], w[0]};
                if (pc & 1)
                    w = u32x4{__builtin_amdgcn_alignbit(w[1], w[0], 16), __builtin_amdgcn_alignbit(w[2], w[1], 16),
                              __builtin_amdgcn_alignbit(w[3], w[2], 16), __builtin_amdgcn_alignbit(w[0], w[3], 16)};
                uint16_t *col = &XT[j][pc * 8][perm_s(sr)];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    col[((e + pc) & 7) * LDX] = (uint16_t)(e & 1 ? w[e >> 1] >> 16 : w[e >> 1]);
            }
        }
    };
    // Sin of SIN_HEADS heads at a time through registers into LDS
    const uint16_t *sin_c = p.sin + ((int64_t)b * p.nc + c) * p.H * (int64_t)kP * N;
    u32x4 sreg[SV];
    auto sin_fetch = [&](int j0) {
        const int nh = std::max(0, std::min(SIN_HEADS, hend - (h0 + j0)));
        const rsrc_t rs = make_rsrc_u(sin_c + (int64_t)(h0 + j0) * kP * N, (uint32_t)(nh * kP * N * 2));
#pragma unroll
        for (int i = 0; i < SV; ++i)
            if (wv * 64 + i * NTH < NSV) sreg[i] = load16(rs, (uint32_t)(tid + i * NTH) * 16u);
    };
    auto sin_stash = [&]() {
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int v = tid + i * NTH;
            if (wv * 64 + i * NTH < NSV) {
                const int jj = v / (kP * N / 8), rem = v % (kP * N / 8);
                *(u32x4 *)&SinL[jj][rem / (N / 8)][(rem % (N / 8)) * 8] = sreg[i];
            }
        }
    };
    fetch(0);
    sin_fetch(0);

    // per-head steps and cumulative log-decays (one wave per head)
    if (wv < HG) {
        float dtv[SPL], cs[SPL];
        head_dt_cs<Q>(p, b, std::min(h0 + wv, hend - 1), c, dtv, cs);
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            cs2[wv][lane * SPL + i] = cs[i] * kLog2e;
            dts[wv][lane * SPL + i] = dtv[i];
        }
    }
    bf16x8 cfr[KN];
    if (live) {
        const int trow = std::min(t0 + r16, T - 1);
#pragma unroll
        for (int k = 0; k < KN; ++k)
            cfr[k] = as_bf16x8(*(const u32x4 *)(Crow + (int64_t)trow * GN + 32 * k + 8 * kb));
    }
    sin_stash();
    if (HG > SIN_HEADS) sin_fetch(SIN_HEADS);
    __syncthreads();
    // w_s dt_s of every time block after the first: r = 64 tb - 1, s <= r
    for (int v = tid; v < (TBS - 1) * HG * Q; v += NTH) {
        const int s = v % Q, j = (v / Q) % HG, tbi = v / (Q * HG) + 1;
        if (s < 64 * tbi) wts[tbi][j][s] = fast_exp2(cs2[j][64 * tbi - 1] - cs2[j][s]) * dts[j][s];
    }

    // entering state: Y = exp(cs_r) C Sin (scaled by a_t further down)
    f32x4 yo[HG][4];
#pragma unroll
    for (int j = 0; j < HG; ++j)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) yo[j][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j0 = 0; j0 < HG; j0 += SIN_HEADS) {
        if (j0) {
            __syncthreads();
            sin_stash();
            __syncthreads();
            if (j0 + SIN_HEADS < HG) sin_fetch(j0 + SIN_HEADS);
        }
        if (live) {
#pragma unroll
            for (int jj = 0; jj < SIN_HEADS; ++jj) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                    for (int k = 0; k < KN; ++k)
                        yo[j0 + jj][qq] = mfma16x16x32(
                            cfr[k], as_bf16x8(*(const u32x4 *)&SinL[jj][qq * 16 + r16][32 * k + 8 * kb]), yo[j0 + jj][qq]);
                }
            }
        }
    }
    const int r = tb * 64 - 1;
    __syncthreads();                                   // the wts table is complete, Sin is read
    if (live && tb) {
#pragma unroll
        for (int j = 0; j < HG; ++j) {
            const float er = fast_exp2(cs2[j][r]);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) yo[j][qq] *= er;
        }
    }
    stash();
    __syncthreads();

    for (int sb = 0; sb < nsw; ++sb) {
        if (sb + 1 < nsw) fetch(sb + 1);
        if (live && sb <= tb) {
            const int s0 = sb * 64;
            const bool diag = sb == tb;
            const int tcol = t0 + r16;                // the A-operand row of this lane
            if (diag) {
                // scale what came before the time block by a_t (rows t0 + 4kb + i) and
                // add D x of these rows from the staged (diagonal) block of x
#pragma unroll
                for (int j = 0; j < HG; ++j) {
                    const float cr = tb ? cs2[j][r] : 0.0f;
                    const f32x4 crow = *(const f32x4 *)&cs2[j][t0 + 4 * kb];
                    const float dsk = (p.Dskip && h0 + j < hend) ? p.Dskip[h0 + j] : 0.0f;
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const u32x2 xv = *(const u32x2 *)&XT[j][qq * 16 + r16][perm_s(16 * tl0 + 4 * kb)];
                        const float xs[4] = {bf16_lo(xv[0]), bf16_hi(xv[0]), bf16_lo(xv[1]), bf16_hi(xv[1])};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            yo[j][qq][i] = fmaf(dsk, xs[i], yo[j][qq][i] * fast_exp2(crow[i] - cr));
                    }
                }
            }
            // one 32-column half of s at a time: G^T[s][t] tiles u = 2a, 2a + 1, lane
            // holds s = s0 + 16u + 4kb + i, t = tcol. On the diagonal block the wave
            // needs u <= tl0, and a half after all of its rows is skipped.
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                if (diag && 32 * a > 16 * tl0 + 15) continue;   // every s after every row
                f32x4 g[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int u = 2 * a + hh;
                    g[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (!diag || u <= tl0) {
#pragma unroll
                        for (int k = 0; k < KN; ++k)
                            g[hh] = mfma16x16x32(as_bf16x8(*(const u32x4 *)&Bb[16 * u + r16][32 * k + 8 * kb]), cfr[k],
                                                 g[hh]);
                    }
                }
#pragma unroll
                for (int j = 0; j < HG; ++j) {
                    float v[8];
                    if (!diag) {
                        const f32x4 w0 = *(const f32x4 *)&wts[tb][j][s0 + 32 * a + 4 * kb];
                        const f32x4 w1 = *(const f32x4 *)&wts[tb][j][s0 + 32 * a + 16 + 4 * kb];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            v[i] = g[0][i] * w0[i];
                            v[4 + i] = g[1][i] * w1[i];
                        }
                    } else {
                        const float ct = cs2[j][tcol];
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int sb0 = s0 + 32 * a + 16 * hh + 4 * kb;
                            const f32x4 cd = *(const f32x4 *)&cs2[j][sb0];
                            const f32x4 dd = *(const f32x4 *)&dts[j][sb0];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float m = g[hh][i] * fast_exp2(ct - cd[i]) * dd[i];
                                v[4 * hh + i] = sb0 + i <= tcol ? m : 0.0f;
                            }
                        }
                    }
                    const bf16x8 mfr = as_bf16x8(u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                                                       pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])});
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq)
                        yo[j][qq] = mfma16x16x32(mfr, as_bf16x8(*(const u32x4 *)&XT[j][qq * 16 + r16][32 * a + 8 * kb]),
                                                 yo[j][qq]);
                    __builtin_amdgcn_sched_barrier(0);   // one head's operands live at a time
                }
            }
        }
        if (sb + 1 < nsw) {
            __syncthreads();
            stash();
            __syncthreads();
        }
    }

    // y32 = Y + D x. Each head's tile goes through the wave's own LDS rows so that a
    // lane writes rows of 8 fp32.
    __syncthreads();                                   // every wave is done with the B block
    if (!live) return;                                 // uniform; no barrier follows
#pragma unroll
    for (int j = 0; j < HG; ++j) {
        const int h = h0 + j;
        if (h >= hend) break;                          // uniform
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int i = 0; i < 4; ++i) Ot[wv][4 * kb + i][qq * 16 + r16] = yo[j][qq][i];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the wave's own rows only
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int row = rr * 8 + (lane >> 3), c8 = (lane & 7) * 8;
            const int t = t0 + row;
            const f32x4 o0 = *(const f32x4 *)&Ot[wv][row][c8];
            const f32x4 o1 = *(const f32x4 *)&Ot[wv][row][c8 + 4];
            if (t < T) {
                float *dst = p.y32 + (((int64_t)b * p.L + t_base + t) * p.H + h) * kP + c8;
                *(f32x4 *)dst = o0;
                *(f32x4 *)(dst + 4) = o1;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
}

// ---------------------------------------------------------------- chunk output, one head
// Per (batch, chunk, head): Q/64 waves; wave w owns the 32-row tiles w and
// Q/32 - 1 - w of the chunk, whose causal work adds up to the same for every wave.
// The head's x (transposed: the B operand of Y += M X) and entering state are
// staged in LDS once (the state's buffer then holds the decay table); the score
// blocks come from L2 (formed by the chunk-state launch). At chunk 256 three
// workgroups fit a CU up to N = 128 (52 KiB of LDS, <= 168 VGPRs) and two at
// N = 256 (68 KiB), so loads of some overlap the arithmetic of others.
//
// Decays as in the 16-row kernel, with r = 32 tau - 1 the step before a tile:
// blocks of s before the tile take M = G o (w_s dt_s), w_s = exp(cs_r - cs_s)
// from a table; their sum with the entering state (exp(cs_r) C Sin) is scaled by
// a_t = exp(cs_t - cs_r) once; the tile's own block takes the exact
// exp(cs_t - cs_s) dt_s [s <= t]. A D tile over (s, t) gives a lane the 16 values
// s = 8g + 4hf + i of its t = c32, and registers 8kk .. 8kk + 7 are the A operand
// (rows t, k = s) of a K-step over s = 16 kk .. 16 kk + 15 if position k = 8 hf + e
// stands for s = 16 kk + 8 (e >> 2) + 4 hf + (e & 3): x is stored with bits 2 and
// 3 of s swapped (pos_s32).
__device__ __forceinline__ int pos_s32(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }

template <int N, int Q>
__global__ __launch_bounds__(Q, Q == 256 ? (N > 128 ? 2 : 3) : 1) void ssd_out_head_kernel(const SSDK p, int64_t nq) {
    constexpr int NT = Q / 32;                // 32-row tiles
    constexpr int NB = score_blocks<Q>();
    constexpr int NTH = Q;                    // Q / 64 waves
    constexpr int KN = N / 16;                // K-steps over the state dimension
    constexpr int SPL = Q / 64;
    constexpr int LDX = Q + 8;                // x^T rows (bf16), 16 bytes past a multiple of 128
    constexpr int LDN = N + 8;                // Sin rows (bf16)
    constexpr int RG = Q / 4;                 // 4-row groups of x
    constexpr int XB = 8 * RG / NTH;          // 4-row x 8-p blocks of x per thread
    constexpr int SV = kP * N / 8 / NTH;      // 16-byte vectors of Sin per thread
    constexpr int SIN_BYTES = kP * LDN * 2;
    constexpr int WTS_BYTES = NT * Q * 4;
    static_assert(NT % 2 == 0 && (kP * N / 8) % NTH == 0 && (8 * RG) % NTH == 0, "staging split");
    __shared__ __attribute__((aligned(16))) float cs2[Q];        // cs * log2(e)
    __shared__ __attribute__((aligned(16))) float dts[Q];        // dt (0 past the end of the sequence)
    __shared__ __attribute__((aligned(16))) uint16_t XT[kP][LDX];
    // the entering state, then (once it is used) the decay table
    __shared__ __attribute__((aligned(16))) uint8_t ubuf[SIN_BYTES > WTS_BYTES ? SIN_BYTES : WTS_BYTES];
    uint16_t (*SinL)[LDN] = reinterpret_cast<uint16_t (*)[LDN]>(ubuf);
    float (*wts)[Q] = reinterpret_cast<float (*)[Q]>(ubuf);      // tile tau: exp(cs_r - cs_s) dt_s, s < 32 tau

    // block -> (chunk, head): q = 8 (k8 / H) + (id & 7), h = k8 % H, k8 = id >> 3; the
    // heads of a chunk share an XCD (its B, C rows and score blocks in one L2)
    const int id = blockIdx.x, k8 = id >> 3;
    const int64_t q = (int64_t)(k8 / p.H) * 8 + (id & 7);
    if (q >= nq) return;                                  // whole workgroup (uniform)
    const int h = k8 % p.H, gg = h / p.hpg;
    const int c = (int)(q % p.nc), b = (int)(q / p.nc);
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, hf = lane >> 5;
    const int64_t t_base = (int64_t)c * Q;
    const int T = (int)std::min<int64_t>(Q, p.L - t_base);
    const int ta = wv, tb = NT - 1 - wv;                  // this wave's tiles (ta < tb)
    const bool live_a = 32 * ta < T, live_b = 32 * tb < T;   // uniform
    const int GN = p.G * N;
    const int64_t xstride = (int64_t)p.H * kP;
    // x^T row p holds position j at column j ^ (8 ((p >> 3) & 7)): the 8 rows that the
    // 8 lanes of one x row write at once then start in different banks. For this lane's
    // rows 32 pt + c32 that is j ^ xsw(pt).
    auto xsw = [&](int pt) { return 32 * pt + (c32 & 24); };

    // -- loads: x (4-row x 8-p blocks), the entering state, the C rows of both tiles
    // (A operand of C Sin), dt. Rows past the sequence read as 0.
    const rsrc_t rX = make_rsrc_u(p.x + ((int64_t)b * p.L + t_base) * xstride + h * kP, (uint32_t)(T * xstride * 2));
    u32x4 xr[XB][4];
#pragma unroll
    for (int m = 0; m < XB; ++m) {
        const int bi = tid + NTH * m;
        const int rg = bi / 8, pg = bi % 8;              // 8 lanes read a row's 128 bytes
        const uint32_t voff = (uint32_t)((4 * rg * xstride + pg * 8) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)   // x's last use in the call: a non-temporal load (cache policy 2)
            xr[m][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, (int)voff,
                                                                                       (int)(i * xstride * 2), 2));
    }
    const uint16_t *sin_h = p.sin + (((int64_t)b * p.nc + c) * p.H + h) * (int64_t)kP * N;
    u32x4 sr[SV];
#pragma unroll
    for (int i = 0; i < SV; ++i)   // read once: non-temporal, so the score blocks and C rows keep L2
        sr[i] = __builtin_nontemporal_load((const u32x4 *)(sin_h + (tid + i * NTH) * 8));
    const rsrc_t rC = make_rsrc_u(p.Cm + (((int64_t)b * p.L + t_base) * p.G + gg) * N, (uint32_t)(T * GN * 2));
    bf16x8 cfa[KN], cfb[KN];
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) {
        cfa[kk] = as_bf16x8(load16(rC, (uint32_t)(((32 * ta + c32) * GN + 16 * kk + 8 * hf) * 2)));
        cfb[kk] = as_bf16x8(load16(rC, (uint32_t)(((32 * tb + c32) * GN + 16 * kk + 8 * hf) * 2)));
    }
    if (wv == 0) {
        float dtv[SPL], cs[SPL];
        head_dt_cs<Q>(p, b, h, c, dtv, cs);
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            cs2[lane * SPL + i] = cs[i] * kLog2e;
            dts[lane * SPL + i] = dtv[i];
        }
    }
#pragma unroll
    for (int m = 0; m < XB; ++m) {
        const int bi = tid + NTH * m;
        const int rg = bi / 8, pg = bi % 8;
        store_transposed(xr[m], &XT[0][0], LDX, pg * 8, pos_s32(4 * rg) ^ (pg << 3));
    }
#pragma unroll
    for (int i = 0; i < SV; ++i) {
        const int v = tid + i * NTH;
        *(u32x4 *)&SinL[v / (N / 8)][(v % (N / 8)) * 8] = sr[i];
    }
    __syncthreads();
    // entering state: Y = exp(cs_r) C Sin for both tiles
    f32x16 ya[2], yb[2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
        ya[pt] = f32x16{};
        yb[pt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) {
            const bf16x8 sf = as_bf16x8(*(const u32x4 *)&SinL[32 * pt + c32][16 * kk + 8 * hf]);
            ya[pt] = mfma32x32x16(cfa[kk], sf, ya[pt]);
            yb[pt] = mfma32x32x16(cfb[kk], sf, yb[pt]);
        }
    }
    __syncthreads();                                      // Sin is read
    // w_s dt_s of every tile after the first (over Sin)
    for (int v = tid; v < (NT - 1) * Q; v += NTH) {
        const int s = v % Q, ti = v / Q + 1;
        if (s < 32 * ti) wts[ti][s] = fast_exp2(cs2[32 * ti - 1] - cs2[s]) * dts[s];
    }
    __syncthreads();                                      // the table is complete
    if (live_a) {                                         // uniform
        if (ta > 0) {
            const float er = fast_exp2(cs2[32 * ta - 1]);
            ya[0] *= er;
            ya[1] *= er;
        }
        {
            const float er = fast_exp2(cs2[32 * tb - 1]);
            yb[0] *= er;
            yb[1] *= er;
        }

        const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;
        const float *gbase = p.gsc + ((q * p.G + gg) * NB) * 1024 + lane * 4;
        auto gload = [&](int tau, int sb, f32x16 &dst) {
            const float *src = gbase + (tau * (tau + 1) / 2 + sb) * 1024;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = *(const f32x4 *)(src + i * 256);
                dst[4 * i] = v[0]; dst[4 * i + 1] = v[1]; dst[4 * i + 2] = v[2]; dst[4 * i + 3] = v[3];
            }
        };
        auto block = [&](f32x16 (&y)[2], int tau, int sb, const f32x16 &g) {
            float mv[16];
            if (sb == tau) {
                // what came before the tile times a_t, then D x of its rows
                const float cr = tau ? cs2[32 * tau - 1] : 0.0f;
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
                    for (int hv = 0; hv < 2; ++hv) {
                        const u32x4 xv = *(const u32x4 *)&XT[32 * pt + c32][(32 * tau + 16 * hv + 8 * hf) ^ xsw(pt)];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int v = 8 * hv + e;
                            const int tl = 8 * (v >> 2) + 4 * hf + (v & 3);
                            const float xs = e & 1 ? bf16_hi(xv[e >> 1]) : bf16_lo(xv[e >> 1]);
                            y[pt][v] = fmaf(dsk, xs, y[pt][v] * fast_exp2(cs2[32 * tau + tl] - cr));
                        }
                    }
                }
                const float ct = cs2[32 * tau + c32];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int sl = 8 * gq + 4 * hf;           // within the 32 rows
                    const f32x4 c4 = *(const f32x4 *)&cs2[32 * sb + sl];
                    const f32x4 d4 = *(const f32x4 *)&dts[32 * sb + sl];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float m = g[4 * gq + i] * fast_exp2(ct - c4[i]) * d4[i];
                        mv[4 * gq + i] = sl + i <= c32 ? m : 0.0f;
                    }
                }
            } else {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4 w4 = *(const f32x4 *)&wts[tau][32 * sb + 8 * gq + 4 * hf];
#pragma unroll
                    for (int i = 0; i < 4; ++i) mv[4 * gq + i] = g[4 * gq + i] * w4[i];
                }
            }
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x8 ma = as_bf16x8(u32x4{pack_bf16(mv[8 * kh], mv[8 * kh + 1]), pack_bf16(mv[8 * kh + 2], mv[8 * kh + 3]),
                                                  pack_bf16(mv[8 * kh + 4], mv[8 * kh + 5]), pack_bf16(mv[8 * kh + 6], mv[8 * kh + 7])});
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
                    y[pt] = mfma32x32x16(ma, as_bf16x8(*(const u32x4 *)&XT[32 * pt + c32][(32 * sb + 16 * kh + 8 * hf) ^ xsw(pt)]),
                                         y[pt]);
            }
        };
        // blocks (ta, j) and (tb, j) side by side for j <= ta (independent accumulators),
        // then (tb, ta + 1 .. tb); each step's score blocks are loaded at the end of the
        // previous step (three workgroups per CU hide the latency)
        f32x16 ga, gb;
        gload(ta, 0, ga);
        if (live_b) gload(tb, 0, gb);
        for (int j = 0; j <= ta; ++j) {
            block(ya, ta, j, ga);
            if (live_b) block(yb, tb, j, gb);
            if (j < ta) gload(ta, j + 1, ga);
            if (live_b) gload(tb, j + 1, gb);                 // j + 1 <= ta + 1 <= tb
        }
        if (live_b) {
            for (int j = ta + 1; j <= tb; ++j) {
                block(yb, tb, j, gb);
                if (j < tb) gload(tb, j + 1, gb);
            }
        }

    }
    __syncthreads();                                      // every wave is done with x^T
    if (!live_a) return;                                  // uniform; no barrier follows

    // -- y = (Y + D x) silu(z) through the wave's own 8 KiB of LDS (over x^T): written as
    // fp32 rows of 64 p from the accumulator layout (row 8 (v >> 2) + 4 hf + (v & 3) of
    // the tile, p = 32 pt + c32), read back as 4 consecutive p per lane (16 lanes per
    // row), gated and stored as 8 contiguous bytes per lane. Rows past the sequence fall
    // outside the buffer ranges (not written, z reads 0). The lane part of each offset
    // sits in a VGPR, the row step in the instruction's scalar offset.
    float (*Yw)[kP] = reinterpret_cast<float (*)[kP]>(&XT[0][0]) + wv * 32;
    const int64_t row0 = ((int64_t)b * p.L + t_base) * xstride + h * kP;
    const rsrc_t rY = make_rsrc_u(p.y + row0, (uint32_t)(T * xstride * 2));
    const rsrc_t rZ = make_rsrc_u(p.z ? p.z + row0 : p.x, p.z ? (uint32_t)(T * xstride * 2) : 0u);
    const int rl = lane >> 4, c4 = (lane & 15) * 4;
    auto out_tile = [&](const f32x16 (&y)[2], int tau) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int v = 0; v < 16; ++v) Yw[8 * (v >> 2) + 4 * hf + (v & 3)][32 * pt + c32] = y[pt][v];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the wave's own rows only
        const int voff = (int)(((32 * tau + rl) * xstride + c4) * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x4 o = *(const f32x4 *)&Yw[rl + 4 * i][c4];
            const int soff = (int)(4 * i * xstride * 2);
            float g0 = o[0], g1 = o[1], g2 = o[2], g3 = o[3];
            if (p.z) {
                const u32x2 zz = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rZ, voff, soff, 0));
                g0 *= silu_f32(bf16_lo(zz[0]));
                g1 *= silu_f32(bf16_hi(zz[0]));
                g2 *= silu_f32(bf16_lo(zz[1]));
                g3 *= silu_f32(bf16_hi(zz[1]));
            }
            // y is not read again by this call: a non-temporal store (cache policy
            // bit 2, `nt`) leaves the caches to x and the entering states that later
            // workgroups still read (S5 call ~206 -> ~199 us)
            constexpr int kYPolicy = 2;
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16(g0, g1), pack_bf16(g2, g3)}, rY, voff, soff,
                                                  kYPolicy);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // read back before the next tile's writes
    };
    out_tile(ya, ta);
    if (live_b) out_tile(yb, tb);
}

__global__ __launch_bounds__(256) void ssd_copy_state_kernel(const float *h0, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

// Workgroups of the chunk-state kernel: the (batch, chunk) count rounded up to 8, times
// the head blocks of 4 per chunk (the kernel returns for ids past the last chunk).
unsigned chunk_state_blocks(const SSDK &k, int64_t nq) {
    return (unsigned)((nq + 7) / 8 * 8 * (k.G * ((k.hpg + 3) / 4)));
}

// Chunk output. The forward runs the per-head kernel on the score blocks formed by
// the chunk-state launch; the fp32 recompute of the gradient pass (which forms no
// score blocks) runs the 16-row kernel.
template <int N, int Q>
void launch_out(const SSDK &k, int64_t nq, hipStream_t s) {
    const unsigned rounded = (unsigned)((nq + 7) / 8 * 8);
    hipLaunchKernelGGL((ssd_out_head_kernel<N, Q>), dim3(rounded * (unsigned)k.H), dim3(Q), 0, s, k, nq);
}

template <int N, int Q>
void launch_recompute_out(const SSDK &k, int64_t nq, hipStream_t s) {
    const int nhg = (k.hpg + OutCfg<N>::HG - 1) / OutCfg<N>::HG;
    const int64_t nblocks = (nq + 7) / 8 * 8 * (k.G * nhg * out_split<N, Q>());
    hipLaunchKernelGGL((ssd_chunk_out_kernel<N, Q>), dim3((unsigned)nblocks), dim3(Q * 4 / out_split<N, Q>()), 0, s,
                       k, nhg, nq);
}

template <int N, int Q>
void launch_nq(const SSDK &k, int batch, hipStream_t s) {
    const int64_t nq = (int64_t)batch * k.nc;            // (batch, chunk) pairs
    // chunk states, and the score blocks of the output kernel in extra workgroups
    const unsigned cs_blocks = chunk_state_blocks(k, nq);
    const unsigned sc_blocks = (unsigned)((nq + 7) / 8 * 8 * k.G);
    hipLaunchKernelGGL((ssd_chunk_state_kernel<N, Q, 0>), dim3(cs_blocks + sc_blocks), dim3(kThreads), 0, s, k, nq,
                       (int)sc_blocks);
    const int64_t total = (int64_t)batch * k.H * kP * N / 4;
    hipLaunchKernelGGL(ssd_state_pass_kernel<true>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       k, N, total);
    launch_out<N, Q>(k, nq, s);
}

template <int N>
void launch_n(const SSDK &k, int batch, int Q, hipStream_t s) {
    switch (Q) {
        case 64: launch_nq<N, 64>(k, batch, s); break;
        case 128: launch_nq<N, 128>(k, batch, s); break;
        default: launch_nq<N, 256>(k, batch, s); break;
    }
}

// pieces of the forward for the gradient pass
template <int N, int Q>
void recompute_nq(const SSDK &k, int batch, int what, hipStream_t s) {
    const int64_t nq = (int64_t)batch * k.nc;
    const dim3 cs_grid(chunk_state_blocks(k, nq));
    if (what == 0) {          // split-precision chunk states, then the entering states
        hipLaunchKernelGGL((ssd_chunk_state_kernel<N, Q, 1>), cs_grid, dim3(kThreads), 0, s, k, nq, 0);
        const int64_t total = (int64_t)batch * k.H * kP * N / 4;
        hipLaunchKernelGGL(ssd_state_pass_kernel<false>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                           k, N, total);
    } else if (what == 1) {   // fp32 pre-gate output
        launch_recompute_out<N, Q>(k, nq, s);
    } else {                  // adjoint aggregates (exp(cs_t) weights)
        hipLaunchKernelGGL((ssd_chunk_state_kernel<N, Q, 2>), cs_grid, dim3(kThreads), 0, s, k, nq, 0);
    }
}

template <int N>
void recompute_n(const SSDK &k, int batch, int Q, int what, hipStream_t s) {
    switch (Q) {
        case 64: recompute_nq<N, 64>(k, batch, what, s); break;
        case 128: recompute_nq<N, 128>(k, batch, what, s); break;
        default: recompute_nq<N, 256>(k, batch, what, s); break;
    }
}

}  // namespace

void ssd_recompute_launch(const SSDK &k, int batch, int Q, int N, int what, hipStream_t s) {
    if (N == 64) recompute_n<64>(k, batch, Q, what, s);
    else if (N == 128) recompute_n<128>(k, batch, Q, what, s);
    else recompute_n<256>(k, batch, Q, what, s);
}

ssm_status ssd_launch(const ssm_ssd_args &a, const SSDPlan &plan, hipStream_t s, char *err,
                      size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();
    if (a.seqlen == 0) {
        if (a.h_final) {
            const int64_t n = a.batch * a.nheads * a.headdim * a.dstate;
            hipLaunchKernelGGL(ssd_copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                               s, a.h0, a.h_final, n);
        }
    } else {
        SSDK k{};
        k.x = (const uint16_t *)a.x; k.dt = (const uint16_t *)a.dt;
        k.Bm = (const uint16_t *)a.Bm; k.Cm = (const uint16_t *)a.Cm; k.z = (const uint16_t *)a.z;
        k.dt_bias = a.dt_bias; k.A = a.A; k.Dskip = a.Dskip; k.h0 = a.h0;
        k.y = (uint16_t *)a.y; k.h_final = a.h_final;
        k.states16 = (uint16_t *)((char *)a.workspace + plan.states_offset);
        k.states_last = (float *)((char *)a.workspace + ssd_last_state_offset(a, plan));
        k.sin = (uint16_t *)((char *)a.workspace + plan.sin_offset);
        k.decay = (float *)((char *)a.workspace + plan.decay_offset);
        k.gsc = plan.gsc_bytes ? (float *)((char *)a.workspace + plan.gsc_offset) : nullptr;
        k.L = a.seqlen; k.H = (int32_t)a.nheads; k.nc = (int32_t)plan.nchunks;
        k.softplus = a.dt_softplus ? 1 : 0;
        k.G = a.ngroups > 1 ? (int32_t)a.ngroups : 1;
        k.hpg = (int32_t)(a.nheads / k.G);
        switch (a.dstate) {
            case 64: launch_n<64>(k, (int)a.batch, (int)a.chunk, s); break;
            case 128: launch_n<128>(k, (int)a.batch, (int)a.chunk, s); break;
            default: launch_n<256>(k, (int)a.batch, (int)a.chunk, s); break;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(err, errlen, "ssd_chunked_fwd: kernel launch failed: %s", hipGetErrorString(e));
        return SSM_EHIP;
    }
    return SSM_OK;
}

}  // namespace ssm
