// Causal depthwise conv1d along time + bias + SiLU (the short convolution of the
// x branch ahead of the scan [Reading page section 5; Hybrid page section 3;
// Juejin page, basic usage: width d_conv = 4]).
//
// Purely HBM-bound: each input and output element crosses HBM once. A lane owns
// a 16-byte vector of adjacent channels (8 bf16 or 4 fp32) of one batch row and
// walks a segment of time, keeping the last K-1 inputs of its channels in
// registers, so every x row is read by one lane only (apart from the K-1 rows of
// history a segment re-reads at its start). Time is cut into segments so that the
// grid fills the chip even for short batches. The lane that runs the last
// segment of a row leaves its window behind as the final state.
#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "device_common.h"
#include "internal.h"

namespace ssm {
namespace {

struct ConvK {
    const void *x, *x0;
    const float *w, *bias;
    void *y, *xf;
    int64_t L;
    int32_t D;
    int32_t seg_len;
    int32_t silu;
};

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

template <typename T, int V>
struct Vec;

// load_raw fetches a lane's vector without converting it (so a block of rows can be
// in flight in few registers); unpack converts it to fp32.
template <>
struct Vec<uint16_t, 8> {
    typedef u32x4 Raw;
    __device__ __forceinline__ static Raw load_raw(const uint16_t *p) { return *(const u32x4 *)p; }
    __device__ __forceinline__ static void unpack(const Raw &v, float (&o)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = bf16_lo(v[i]);
            o[2 * i + 1] = bf16_hi(v[i]);
        }
    }
    __device__ __forceinline__ static void load(const uint16_t *p, float (&o)[8]) { unpack(load_raw(p), o); }
    __device__ __forceinline__ static void store(uint16_t *p, const float (&o)[8]) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
        // y is not read back here: a non-temporal store keeps the caches for the x
        // rows still to come (B8 L2048 D1536: 29.6 -> 27.7 us)
        __builtin_nontemporal_store(v, (u32x4 *)p);
    }
};

template <>
struct Vec<float, 4> {
    typedef f32x4 Raw;
    __device__ __forceinline__ static Raw load_raw(const float *p) { return *(const f32x4 *)p; }
    __device__ __forceinline__ static void unpack(const Raw &v, float (&o)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = v[i];
    }
    __device__ __forceinline__ static void load(const float *p, float (&o)[4]) { unpack(load_raw(p), o); }
    __device__ __forceinline__ static void store(float *p, const float (&o)[4]) {
        __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, (f32x4 *)p);   // as the bf16 store
    }
};

template <typename T>
struct Vec<T, 1> {
    typedef T Raw;
    __device__ __forceinline__ static Raw load_raw(const T *p) { return *p; }
    __device__ __forceinline__ static void unpack(const Raw &v, float (&o)[1]) { o[0] = to_f32(v); }
    __device__ __forceinline__ static void load(const T *p, float (&o)[1]) { o[0] = to_f32(*p); }
    __device__ __forceinline__ static void store(T *p, const float (&o)[1]) { store_val(p, o[0]); }
};

template <typename T, int K, int V>
__global__ __launch_bounds__(64) void conv1d_kernel(const ConvK k) {
    constexpr int U = 4;   // time steps whose loads are issued together (8 measured no faster)
    const int d0 = (blockIdx.x * 64 + threadIdx.x) * V;
    if (d0 >= k.D) return;
    const int64_t b = blockIdx.z;
    const int64_t t0 = (int64_t)blockIdx.y * k.seg_len;
    const int64_t t1 = std::min<int64_t>(k.L, t0 + k.seg_len);
    const T *x = (const T *)k.x, *x0 = (const T *)k.x0;
    T *y = (T *)k.y;

    float w[V][K], bias[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        bias[v] = k.bias ? k.bias[d0 + v] : 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) w[v][j] = k.w[(int64_t)(d0 + v) * K + j];
    }
    // the K-1 inputs before t0 (history rows come from x0, zeros without it)
    float win[K - 1][V];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        const int64_t s = t0 - (K - 1) + j;
        if (s >= 0) {
            Vec<T, V>::load(x + (b * k.L + s) * k.D + d0, win[j]);
        } else if (x0) {
            Vec<T, V>::load(x0 + (b * (K - 1) + (K - 1) + s) * k.D + d0, win[j]);
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v) win[j][v] = 0.0f;
        }
    }

    // Rows come in blocks of U, each block's loads issued before the previous block's
    // stores: the memory counter completes in order, so waiting for a load issued
    // after a store would also wait for the store. Rows past the segment are clamped
    // to its last row (valid, loaded again, not used), so the loads are unconditional.
    typedef typename Vec<T, V>::Raw Raw;
    auto load_block = [&](int64_t tb, Raw (&r)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = std::min<int64_t>(tb + u, t1 - 1);
            r[u] = Vec<T, V>::load_raw(x + (b * k.L + row) * k.D + d0);
        }
    };
    Raw cur_raw[U], nxt_raw[U];
    if (t0 < t1) load_block(t0, cur_raw);
    for (int64_t t = t0; t < t1; t += U) {
        load_block(t + U, nxt_raw);
        float cur[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) Vec<T, V>::unpack(cur_raw[u], cur[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t + u < t1) {
                float o[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    float acc = fmaf(w[v][K - 1], cur[u][v], bias[v]);
#pragma unroll
                    for (int j = 0; j < K - 1; ++j) acc = fmaf(w[v][j], win[j][v], acc);
                    o[v] = k.silu ? silu_f32(acc) : acc;
                }
                Vec<T, V>::store(y + (b * k.L + t + u) * k.D + d0, o);
#pragma unroll
                for (int j = 0; j < K - 2; ++j)
#pragma unroll
                    for (int v = 0; v < V; ++v) win[j][v] = win[j + 1][v];
#pragma unroll
                for (int v = 0; v < V; ++v) win[K - 2][v] = cur[u][v];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) cur_raw[u] = nxt_raw[u];
    }
    // the window now holds the inputs at t1-(K-1) .. t1-1
    if (k.xf && t1 == k.L) {
        T *xf = (T *)k.xf;
#pragma unroll
        for (int j = 0; j < K - 1; ++j) Vec<T, V>::store(xf + (b * (K - 1) + j) * k.D + d0, win[j]);
    }
}

template <typename T, int V>
void launch_tv(const ConvK &k, int K, dim3 grid, hipStream_t s) {
    switch (K) {
        case 2: hipLaunchKernelGGL((conv1d_kernel<T, 2, V>), grid, dim3(64), 0, s, k); break;
        case 3: hipLaunchKernelGGL((conv1d_kernel<T, 3, V>), grid, dim3(64), 0, s, k); break;
        default: hipLaunchKernelGGL((conv1d_kernel<T, 4, V>), grid, dim3(64), 0, s, k); break;
    }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

ssm_status conv_launch(const ssm_conv_args &a, hipStream_t s, char *err, size_t errlen) {
    if (a.batch == 0) return SSM_OK;
    (void)hipGetLastError();
    const int es = a.dtype == SSM_BF16 ? 2 : 4;
    const int vec = 16 / es;
    const bool wide = a.dim % vec == 0 && aligned16(a.x) && aligned16(a.y) && aligned16(a.init_state) &&
                      aligned16(a.final_state);
    const int V = wide ? vec : 1;
    const int64_t lanes = (a.dim + V - 1) / V;
    // enough segments along time for ~256K lanes in flight, at least 32 steps each (a
    // segment re-reads K-1 rows of history, and shorter segments made the B8 L2048
    // D1536 case slower: 35.6 us at 8 steps, 29.8 us at 32)
    int64_t lanes_target = 262144, min_seg = 32;
    if (const char *env = std::getenv("SSM_CONV_LANES")) lanes_target = std::max(1L, std::atol(env));   // tuning override
    if (const char *env = std::getenv("SSM_CONV_MIN_SEG")) min_seg = std::max(1L, std::atol(env));      // tuning override
    const int64_t want = std::max<int64_t>(1, (lanes_target + a.batch * lanes - 1) / (a.batch * lanes));
    const int64_t nseg_max = std::max<int64_t>(1, a.seqlen / min_seg);
    int64_t nseg = std::min<int64_t>(std::min<int64_t>(want, nseg_max), 65535);
    const int64_t seg_len = a.seqlen == 0 ? 0 : (a.seqlen + nseg - 1) / nseg;
    nseg = seg_len == 0 ? 1 : (a.seqlen + seg_len - 1) / seg_len;
    ConvK k{};
    k.x = a.x; k.x0 = a.init_state; k.w = a.weight; k.bias = a.bias;
    k.y = a.y; k.xf = a.final_state;
    k.L = a.seqlen; k.D = (int32_t)a.dim; k.seg_len = (int32_t)seg_len;
    k.silu = a.apply_silu ? 1 : 0;
    const dim3 grid((unsigned)((lanes + 63) / 64), (unsigned)nseg, (unsigned)a.batch);
    if (a.dtype == SSM_BF16) {
        if (wide) launch_tv<uint16_t, 8>(k, (int)a.width, grid, s);
        else launch_tv<uint16_t, 1>(k, (int)a.width, grid, s);
    } else {
        if (wide) launch_tv<float, 4>(k, (int)a.width, grid, s);
        else launch_tv<float, 1>(k, (int)a.width, grid, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::snprintf(err, errlen, "causal_conv1d_fwd: kernel launch failed: %s", hipGetErrorString(e));
        return SSM_EHIP;
    }
    return SSM_OK;
}

}  // namespace ssm
