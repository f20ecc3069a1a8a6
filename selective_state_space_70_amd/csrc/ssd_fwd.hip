// Scalar-A state-space form (Mamba-2 "SSD") for gfx950, on the matrix cores.
//
// With one scalar decay per head the mixing matrix of a chunk is semiseparable:
// inside a chunk of Q steps, y = (L o C B^T o exp(cs_t - cs_s) o dt_s) x, and the
// influence of everything before the chunk passes through one N x P state per
// head [Mamba-2 page "Mamba-2：把状态空间模型和 Attention 统一到一个数学框架里", Core
// idea step 2 (SSM as a structured attention-like matrix y = (L o M) x) and key
// point 1 (semiseparable: every off-diagonal block is low rank, O(L) storage)].
// With cs_t = sum_{k<=t in chunk} A dt_k:
//   state of chunk c  : S_c = sum_s exp(cs_end - cs_s) dt_s B_s (x) x_s   (N x P)
//   entering state    : Sin_0 = h0, Sin_{c+1} = exp(cs_end,c) Sin_c + S_c
//   output            : y_t = sum_{s<=t} (C_t.B_s) exp(cs_t - cs_s) dt_s x_s
//                            + exp(cs_t) C_t . Sin_c + D x_t,   then * silu(z_t)
//
// Kernels (one call):
//   1. ssd_chunk_state : per (b, chunk, head), S_c on the MFMA units
//      (v_mfma_f32_16x16x32_bf16, K = time), the decay exp(cs_end) of the chunk.
//   2. ssd_state_pass  : sequential over chunks per (b, h, n, p) element.
//   3. ssd_chunk_out   : per (b, chunk, head). For each 16-row time tile the
//      transposed score tile G^T = B C^T is computed on the MFMA units, masked and
//      scaled in registers, rounded to bf16 and used directly as the A operand of
//      Y += M X: the accumulator layout of a 16x16 tile gives each lane 4
//      consecutive s of one t, two tiles give 8, which is an A-operand fragment
//      once X is fetched with the same permutation of s. The carried state enters
//      through Y += exp(cs_t) (C Sin) on the same units.
// The contraction over s is insensitive to which 8 values of s a lane group holds
// as long as the A and B fragments use the same order; that freedom is what lets
// the accumulator fragment be reused without going through LDS.
#include <algorithm>
#include <cstdio>

#include "device_common.h"
#include "internal.h"

namespace ssm {
namespace {

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

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

struct SSDK {
    const uint16_t *x, *dt, *Bm, *Cm, *z;
    const float *dt_bias, *A, *Dskip, *h0;
    uint16_t *y;
    float *h_final;
    float *states;   // [B][nc][H][N][P]
    float *decay;    // [B][H][nc]
    int64_t L;
    int32_t H;
    int32_t nc;
    int32_t softplus;
};

// Inclusive prefix sum over the 256 threads of a block (values of threads past
// the chunk are zero). Uses wave shuffles and one LDS exchange of wave totals.
__device__ __forceinline__ float block_inclusive_scan(float v, float *wave_tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) wave_tot[w] = v;
    __syncthreads();
    float add = 0.0f;
    for (int i = 0; i < w; ++i) add += wave_tot[i];
    __syncthreads();
    return v + add;
}

// dt and the in-chunk cumulative log-decay for step t of chunk c (thread t).
// Returns dt (0 past the end of the sequence) and writes cs to *cs_out.
__device__ __forceinline__ float chunk_dt_cs(const SSDK &p, int b, int h, int c, int Q,
                                             float *wave_tot, float *cs_out) {
    const int t = threadIdx.x;
    const int64_t tg = (int64_t)c * Q + t;
    float dtv = 0.0f;
    if (t < Q && tg < p.L) {
        const float v = to_f32(p.dt[((int64_t)b * p.L + tg) * p.H + h]) +
                        (p.dt_bias ? p.dt_bias[h] : 0.0f);
        dtv = p.softplus ? softplus_f32(v) : v;
    }
    *cs_out = block_inclusive_scan(p.A[h] * dtv, wave_tot);
    return dtv;
}

// ---------------------------------------------------------------- chunk states
template <int N, int Q>
__global__ __launch_bounds__(kThreads) void ssd_chunk_state_kernel(const SSDK p) {
    constexpr int SB = 64;              // time rows staged per step
    constexpr int PAD = 8;              // bf16 padding per LDS row
    constexpr int NT = N / 16;          // n tiles
    constexpr int NT_W = NT / 4;        // n tiles per wave
    __shared__ float wave_tot[4];
    __shared__ float w_s[Q];
    __shared__ __attribute__((aligned(16))) uint16_t BwT[N][SB + PAD];
    __shared__ __attribute__((aligned(16))) uint16_t XT[kP][SB + PAD];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, kb = lane >> 4;

    float cs;
    const float dtv = chunk_dt_cs(p, b, h, c, Q, wave_tot, &cs);
    __shared__ float cs_end_sh;
    if (tid == Q - 1) cs_end_sh = cs;
    __syncthreads();
    const float cs_end = cs_end_sh;
    if (tid < Q) w_s[tid] = fast_exp2((cs_end - cs) * kLog2e) * dtv;
    if (tid == 0) p.decay[((int64_t)b * p.H + h) * p.nc + c] = fast_exp2(cs_end * kLog2e);

    f32x4 acc[NT_W][4];
#pragma unroll
    for (int i = 0; i < NT_W; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t t_base = (int64_t)c * Q;
    for (int s0 = 0; s0 < Q; s0 += SB) {
        __syncthreads();
        // B rows -> BwT[n][s] scaled by w_s (bf16). N*SB/8 vectors of 8 n.
        for (int v = tid; v < SB * N / 8; v += kThreads) {
            const int s = v / (N / 8), ng = v % (N / 8);
            const int64_t tg = t_base + s0 + s;
            u32x4 raw = u32x4{0u, 0u, 0u, 0u};
            if (tg < p.L) raw = *(const u32x4 *)(p.Bm + ((int64_t)b * p.L + tg) * N + ng * 8);
            const float ws = w_s[s0 + s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                BwT[ng * 8 + 2 * e][s] = f32_to_bf16(bf16_lo(raw[e]) * ws);
                BwT[ng * 8 + 2 * e + 1][s] = f32_to_bf16(bf16_hi(raw[e]) * ws);
            }
        }
        // x rows -> XT[p][s]
        for (int v = tid; v < SB * kP / 8; v += kThreads) {
            const int s = v / (kP / 8), pg = v % (kP / 8);
            const int64_t tg = t_base + s0 + s;
            u32x4 raw = u32x4{0u, 0u, 0u, 0u};
            if (tg < p.L)
                raw = *(const u32x4 *)(p.x + (((int64_t)b * p.L + tg) * p.H + h) * kP + pg * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                XT[pg * 8 + 2 * e][s] = (uint16_t)(raw[e] & 0xffffu);
                XT[pg * 8 + 2 * e + 1][s] = (uint16_t)(raw[e] >> 16);
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < SB / 32; ++kk) {
            const int sk = kk * 32 + kb * 8;
            bf16x8 bfr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = as_bf16x8(*(const u32x4 *)&XT[j * 16 + r16][sk]);
#pragma unroll
            for (int i = 0; i < NT_W; ++i) {
                const int nrow = (wv * NT_W + i) * 16 + r16;
                const bf16x8 afr = as_bf16x8(*(const u32x4 *)&BwT[nrow][sk]);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(afr, bfr[j], acc[i][j]);
            }
        }
    }
    // S_c[n][p]: lane holds rows n = tile*16 + 4*kb + e, column p = j*16 + r16
    float *out = p.states + ((((int64_t)b * p.nc + c) * p.H + h) * N) * kP;
#pragma unroll
    for (int i = 0; i < NT_W; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = (wv * NT_W + i) * 16 + 4 * kb + e;
                out[n * kP + j * 16 + r16] = acc[i][j][e];
            }
}

// ---------------------------------------------------------------- state passing
// One thread per (b, h, n, p); slot c becomes the state entering chunk c.
__global__ __launch_bounds__(256) void ssd_state_pass_kernel(const SSDK p, int N, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t per_bh = (int64_t)N * kP;
    const int64_t np = i % per_bh;            // n*P + p
    const int64_t bh = i / per_bh;            // b*H + h
    const int64_t b = bh / p.H, h = bh % p.H;
    const int64_t n = np / kP, pp = np % kP;
    const int64_t hidx = (bh * kP + pp) * N + n;    // (b, h, p, n)
    float s = p.h0 ? p.h0[hidx] : 0.0f;
    const float *dec = p.decay + bh * p.nc;
    for (int c = 0; c < p.nc; ++c) {
        float *slot = p.states + (((b * p.nc + c) * p.H + h) * per_bh) + np;
        const float sc = *slot;
        *slot = s;
        s = fmaf(dec[c], s, sc);
    }
    if (p.h_final) p.h_final[hidx] = s;
}

// ---------------------------------------------------------------- chunk output
template <int N, int Q>
__global__ __launch_bounds__(kThreads) void ssd_chunk_out_kernel(const SSDK p) {
    constexpr int PADX = 8, PADS = 8;
    constexpr int TT = Q / 16;                  // time tiles in a chunk
    __shared__ float wave_tot[4];
    __shared__ float cs_s[Q];
    __shared__ float dt_s[Q];
    __shared__ __attribute__((aligned(16))) uint16_t XT[kP][Q + PADX];
    __shared__ __attribute__((aligned(16))) uint16_t SinT[kP][N + PADS];

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, kb = lane >> 4;
    const int64_t t_base = (int64_t)c * Q;
    const int T = (int)std::min<int64_t>(Q, p.L - t_base);    // valid steps in this chunk

    float cs;
    const float dtv = chunk_dt_cs(p, b, h, c, Q, wave_tot, &cs);
    if (tid < Q) {
        cs_s[tid] = cs;
        dt_s[tid] = dtv;
    }
    // x chunk -> XT[p][s]
    for (int v = tid; v < Q * kP / 8; v += kThreads) {
        const int s = v / (kP / 8), pg = v % (kP / 8);
        u32x4 raw = u32x4{0u, 0u, 0u, 0u};
        if (s < T) raw = *(const u32x4 *)(p.x + (((int64_t)b * p.L + t_base + s) * p.H + h) * kP + pg * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            XT[pg * 8 + 2 * e][s] = (uint16_t)(raw[e] & 0xffffu);
            XT[pg * 8 + 2 * e + 1][s] = (uint16_t)(raw[e] >> 16);
        }
    }
    // entering state Sin[n][p] (fp32) -> SinT[p][n] (bf16)
    const float *sin = p.states + ((((int64_t)b * p.nc + c) * p.H + h) * N) * kP;
    for (int v = tid; v < N * kP / 4; v += kThreads) {
        const int n = v / (kP / 4), pg = v % (kP / 4);
        const float4 s4 = *(const float4 *)(sin + n * kP + pg * 4);
        SinT[pg * 4 + 0][n] = f32_to_bf16(s4.x);
        SinT[pg * 4 + 1][n] = f32_to_bf16(s4.y);
        SinT[pg * 4 + 2][n] = f32_to_bf16(s4.z);
        SinT[pg * 4 + 3][n] = f32_to_bf16(s4.w);
    }
    __syncthreads();

    const uint16_t *Bb = p.Bm + ((int64_t)b * p.L + t_base) * N;
    const uint16_t *Cb = p.Cm + ((int64_t)b * p.L + t_base) * N;
    const float dsk = p.Dskip ? p.Dskip[h] : 0.0f;

    for (int tt = wv; tt < TT; tt += 4) {
        const int t0 = tt * 16;
        if (t0 >= T) break;
        // C rows of this tile as fragments (row t0 + r16, n = 32*k + 8*kb .. +7)
        bf16x8 cfr[N / 32];
        const int trow = std::min(t0 + r16, T - 1);
#pragma unroll
        for (int k = 0; k < N / 32; ++k)
            cfr[k] = as_bf16x8(*(const u32x4 *)(Cb + (int64_t)trow * N + k * 32 + kb * 8));

        // carried state: Y = C Sin, rows scaled by exp(cs_t) afterwards
        f32x4 yacc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < N / 32; ++k)
                a = mfma16x16x32(cfr[k], as_bf16x8(*(const u32x4 *)&SinT[j * 16 + r16][k * 32 + kb * 8]), a);
            yacc[j] = a;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + 4 * kb + e;
            const float sc = fast_exp2(cs_s[std::min(t, Q - 1)] * kLog2e);
#pragma unroll
            for (int j = 0; j < 4; ++j) yacc[j][e] *= sc;
        }

        // diagonal block: s in [0, t0 + 16), 32 at a time
        const int tcol = t0 + r16;                 // the t this lane's G^T column holds
        const float cs_t = cs_s[tcol];
        for (int s0 = 0; s0 < t0 + 16; s0 += 32) {
            f32x4 g[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int srow = std::min(s0 + 16 * u + r16, T - 1);
                f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < N / 32; ++k) {
                    const bf16x8 bfr = as_bf16x8(*(const u32x4 *)(Bb + (int64_t)srow * N + k * 32 + kb * 8));
                    a = mfma16x16x32(bfr, cfr[k], a);
                }
                g[u] = a;
            }
            // mask, decay and dt scale; element (u, e) is s = s0 + 16u + 4kb + e
            uint32_t m[4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float vals[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s0 + 16 * u + 4 * kb + e;
                    float val = 0.0f;
                    if (s <= tcol && s < T)
                        val = g[u][e] * fast_exp2((cs_t - cs_s[s]) * kLog2e) * dt_s[s];
                    vals[e] = val;
                }
                m[2 * u] = pack_bf16(vals[0], vals[1]);
                m[2 * u + 1] = pack_bf16(vals[2], vals[3]);
            }
            const bf16x8 mfr = as_bf16x8(u32x4{m[0], m[1], m[2], m[3]});
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint16_t *xr = &XT[j * 16 + r16][0];
                const u32x2 lo = *(const u32x2 *)(xr + s0 + 4 * kb);
                const u32x2 hi = *(const u32x2 *)(xr + s0 + 16 + 4 * kb);
                const bf16x8 xfr = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                yacc[j] = mfma16x16x32(mfr, xfr, yacc[j]);
            }
        }

        // y = Y + D x, gate, store. Lane holds rows t0 + 4kb + e, column j*16 + r16.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + 4 * kb + e;
            if (t >= T) continue;
            const int64_t rowoff = (((int64_t)b * p.L + t_base + t) * p.H + h) * kP;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int pp = j * 16 + r16;
                const float xv = to_f32(XT[pp][t]);
                float yv = fmaf(dsk, xv, yacc[j][e]);
                if (p.z) yv *= silu_f32(to_f32(p.z[rowoff + pp]));
                p.y[rowoff + pp] = f32_to_bf16(yv);
            }
        }
    }
}

__global__ __launch_bounds__(256) void ssd_copy_state_kernel(const float *h0, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = h0 ? h0[i] : 0.0f;
}

template <int N, int Q>
void launch_nq(const SSDK &k, int batch, hipStream_t s) {
    const dim3 grid((unsigned)k.nc, (unsigned)k.H, (unsigned)batch);
    hipLaunchKernelGGL((ssd_chunk_state_kernel<N, Q>), grid, dim3(kThreads), 0, s, k);
    const int64_t total = (int64_t)batch * k.H * N * kP;
    hipLaunchKernelGGL(ssd_state_pass_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       k, N, total);
    hipLaunchKernelGGL((ssd_chunk_out_kernel<N, Q>), grid, dim3(kThreads), 0, s, k);
}

template <int N>
void launch_n(const SSDK &k, int batch, int Q, hipStream_t s) {
    switch (Q) {
        case 64: launch_nq<N, 64>(k, batch, s); break;
        case 128: launch_nq<N, 128>(k, batch, s); break;
        default: launch_nq<N, 256>(k, batch, s); break;
    }
}

}  // namespace

SSDPlan ssd_plan(const ssm_ssd_args &a) {
    SSDPlan pl{};
    if (a.batch <= 0 || a.seqlen <= 0 || a.chunk <= 0) return pl;
    pl.nchunks = (a.seqlen + a.chunk - 1) / a.chunk;
    const size_t states = (size_t)a.batch * pl.nchunks * a.nheads * a.dstate * a.headdim * sizeof(float);
    pl.states_offset = 0;
    pl.decay_offset = (states + 255) & ~(size_t)255;
    const size_t dec = (size_t)a.batch * a.nheads * pl.nchunks * sizeof(float);
    pl.bytes = pl.decay_offset + ((dec + 255) & ~(size_t)255);
    return pl;
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
        k.states = (float *)((char *)a.workspace + plan.states_offset);
        k.decay = (float *)((char *)a.workspace + plan.decay_offset);
        k.L = a.seqlen; k.H = (int32_t)a.nheads; k.nc = (int32_t)plan.nchunks;
        k.softplus = a.dt_softplus ? 1 : 0;
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
