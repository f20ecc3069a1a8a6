// Device code shared by the scalar-A (SSD) kernels: the matrix-core fragment
// helpers, LDS transposes, the per-head step and cumulative log-decay of a chunk,
// and the kernel argument block.
//
// Fragments of v_mfma_f32_16x16x32_bf16 (lane l, r16 = l & 15, kb = l >> 4):
//   A (16 x 32): row r16, k = 8 kb + e (e = 0..7, one 16-byte vector);
//   B (32 x 16): column r16, k = 8 kb + e;
//   D (16 x 16, fp32): rows 4 kb + i (i = 0..3), column r16.
// Two D tiles over consecutive 16-blocks of a dimension j give a lane the 8 values
// j = 16 h + 4 kb + i (h, i in 0..1, 0..3); used as the k values of an A fragment
// they stand for k = 8 kb + 4 h + i, so the matching B operand is stored with its
// k rows permuted by perm_s.
#pragma once

#include <algorithm>

#include "device_common.h"

namespace ssm {

constexpr int kP = 64;          // head dimension handled by these kernels
constexpr int kThreads = 256;   // 4 waves

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// v_mfma_f32_32x32x16_bf16 (lane l, c32 = l & 31, hf = l >> 5): A (32 x 16) row c32,
// k = 8 hf + e; B (16 x 32) column c32, k = 8 hf + e; D (32 x 32, fp32) register v
// holds row 8 (v >> 2) + 4 hf + (v & 3), column c32.
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Buffer resource from a wave-uniform base and size. Every call site passes values
// that are the same in all lanes of the wave; readfirstlane on the base as well
// keeps the resource in SGPRs even where the compiler built the address with
// vector instructions (a resource in VGPRs costs a loop over lanes per access).
__device__ __forceinline__ rsrc_t make_rsrc_u(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return make_rsrc((const void *)((hi << 32) | lo), bytes);
}

// 16 bytes through a buffer resource (0 outside its range)
__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// the same with a wave-uniform part of the offset in the instruction's scalar offset
__device__ __forceinline__ u32x4 load16s(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return pack_bf16x2(lo, hi); }

// (lo halves of a, b) and (hi halves of a, b) as packed bf16 pairs.
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Write a 4 x 8 block (4 rows, 8 columns, each row one u32x4 of packed bf16) to
// LDS transposed: T[c][r0 .. r0+3] for the 8 columns c0 .. c0+7.
__device__ __forceinline__ void store_transposed(const u32x4 (&r)[4], uint16_t *T, int ldt, int c0,
                                                 int r0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x2 lo = u32x2{lo_pair(r[0][j], r[1][j]), lo_pair(r[2][j], r[3][j])};
        const u32x2 hi = u32x2{hi_pair(r[0][j], r[1][j]), hi_pair(r[2][j], r[3][j])};
        *(u32x2 *)&T[(c0 + 2 * j) * ldt + r0] = lo;
        *(u32x2 *)&T[(c0 + 2 * j + 1) * ldt + r0] = hi;
    }
}

struct SSDK {
    const uint16_t *x, *dt, *Bm, *Cm, *z;
    const float *dt_bias, *A, *Dskip, *h0;
    uint16_t *y;
    float *h_final;
    float *states;      // fp32 [B][nc][H][P][N]: state of each chunk from zero (gradient pass)
    uint16_t *states16; // bf16, same layout: the chunk states of the forward
    float *states_last; // fp32 [B][H][P][N]: the forward's last chunk state (feeds h_final only)
    uint16_t *sin;      // bf16 [B][nc][H][P][N]: state entering each chunk
    float *decay;       // fp32 [B][H][nc]: exp(cs_end) of each chunk
    float *sin32;       // optional fp32 copy of the entering states (may alias states)
    float *y32;         // fp32 pre-gate output (B, L, H, P) of the recompute variant
    const uint16_t *xlo;   // optional bf16 lo part of x (adjoint aggregates: dyc = hi + lo)
    float *gsc;         // fp32 score blocks C B^T per (batch, chunk, group) (forward)
    int64_t L;
    int32_t H;
    int32_t nc;
    int32_t softplus;
    int32_t G;          // groups of B, C
    int32_t hpg;        // heads per group
};

// The raw dt of chunk c of head h, as head_dt_cs reads it (steps clamped to the
// sequence): lane l gets steps l*SPL .. l*SPL+SPL-1.
template <int Q>
__device__ __forceinline__ void head_dt_raw(const SSDK &p, int b, int h, int c, float (&raw)[Q / 64]) {
    constexpr int SPL = Q / 64;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int64_t tg = std::min<int64_t>((int64_t)c * Q + lane * SPL + i, p.L - 1);
        raw[i] = to_f32(p.dt[((int64_t)b * p.L + tg) * p.H + h]);
    }
}

// dt and the inclusive in-chunk cumulative log-decay A*dt from the raw dt of
// head_dt_raw. Steps past the sequence get dt = 0. Returns the chunk total (the
// last cs) to every lane.
template <int Q>
__device__ __forceinline__ float head_dt_cs_from(const SSDK &p, int h, int c, const float (&raw)[Q / 64],
                                                 float (&dtv)[Q / 64], float (&cs)[Q / 64]) {
    constexpr int SPL = Q / 64;
    const int lane = threadIdx.x & 63;
    const float *biasp = p.dt_bias ? p.dt_bias : p.A;   // unconditional loads (an absent bias reads A)
    const float biasv = biasp[h], a = p.A[h];
    const float bias = p.dt_bias ? biasv : 0.0f;
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int64_t tg = (int64_t)c * Q + lane * SPL + i;
        const float v = raw[i] + bias;
        const float dt = p.softplus ? softplus_f32(v) : v;
        const float d = tg < p.L ? dt : 0.0f;
        dtv[i] = d;
        run += a * d;
        cs[i] = run;
    }
    float incl = run;   // inclusive scan of lane totals
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    const float excl = incl - run;
#pragma unroll
    for (int i = 0; i < SPL; ++i) cs[i] += excl;
    return __shfl(incl, 63, 64);
}

// dt and the inclusive in-chunk cumulative log-decay A*dt for the steps of chunk
// c of head h; lane l owns steps l*SPL .. l*SPL+SPL-1 (SPL = Q/64). All loads are
// issued first (their latencies overlap: a load under a branch is waited for at
// the branch's end, one at a time).
template <int Q>
__device__ __forceinline__ float head_dt_cs(const SSDK &p, int b, int h, int c, float (&dtv)[Q / 64],
                                            float (&cs)[Q / 64]) {
    float raw[Q / 64];
    head_dt_raw<Q>(p, b, h, c, raw);
    return head_dt_cs_from<Q>(p, h, c, raw, dtv, cs);
}

// position of chunk-local s (its block of 64 aside) in the permuted x rows
__device__ __forceinline__ int perm_s(int sl) {
    return ((sl >> 5) << 5) | (((sl >> 2) & 3) << 3) | (((sl >> 4) & 1) << 2) | (sl & 3);
}

}  // namespace ssm
