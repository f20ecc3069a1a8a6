// Device helpers shared by the gfx950 kernels of libssm.so.
//
// Storage types: float (fp32) and uint16_t holding bfloat16 bits. All arithmetic
// is fp32. bf16 -> fp32 is a 16-bit shift (exact); fp32 -> bf16 uses the native
// round-to-nearest-even conversion of gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Pointer into the constant address space: uniform loads through it become
// scalar (s_load) loads, so a value shared by the whole wave (B_t, C_t) lands
// in SGPRs and costs no vector instruction to broadcast. Only used for buffers
// that no kernel of the same launch writes.
typedef const __attribute__((address_space(4))) uint32_t cu32;

__device__ __forceinline__ cu32 *as_const(const void *p) { return (cu32 *)(p); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    __bf16 b = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}
// Two fp32 values as a packed pair of bf16 (lo in bits 0..15), one v_cvt_pk_bf16_f32.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ void store_val(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_val(uint16_t *p, float v) { *p = f32_to_bf16(v); }

// Raw buffer access: the base and size live in a wave-uniform resource (SGPRs),
// the row offset is a uniform byte offset (soffset) and the lane adds a fixed
// byte offset (voffset), so streaming along time needs no vector address math.
// Reads at or past `bytes` return 0 (hardware range check on the vector offset).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // the size is wave-uniform; readfirstlane keeps it in an SGPR even when the
    // compiler computed it with a vector instruction (a resource in VGPRs would
    // force a loop over lanes around every access)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ void buf_load(rsrc_t r, uint32_t voff, uint32_t soff, uint16_t &v) {
    v = __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_load(rsrc_t r, uint32_t voff, uint32_t soff, float &v) {
    v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t voff, uint32_t soff, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_store(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
}

// The same wave-uniform value, opaque to the optimiser (an empty asm statement
// that claims to change it; no instruction is emitted).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
    asm volatile("" : "+s"(v));
    return v;
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float fast_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float fast_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^{-|v|}).
// log1p(u) for u in (0, 1] is taken as log(w) + (u - (w - 1)) with w = 1 + u:
// the second term is the exact rounding error of 1 + u, so small steps keep
// their full relative precision (a plain log(1 + e^v) loses it below ~1e-3).
// max(v, 0) is taken as (v + |v|) / 2, exact, folded into the last FMA (fmaxf would
// cost a NaN-quieting instruction on top of the max).
__device__ __forceinline__ float softplus_f32(float v) {
    const float u = fast_exp2(-fabsf(v) * kLog2e);
    const float w = 1.0f + u;
    const float c = u - (w - 1.0f);
    return fmaf(v + fabsf(v), 0.5f, fmaf(fast_log2(w), kLn2, c));
}

// silu(z) = z / (1 + e^{-z}); for z -> -inf the reciprocal of +inf is 0.
__device__ __forceinline__ float silu_f32(float z) {
    return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// One row of a (L, N) B or C matrix shared by the whole wave, loaded with scalar
// loads and widened to fp32 (SGPR-resident).
template <typename T, int N>
struct SharedRow;

template <int N>
struct SharedRow<uint16_t, N> {
    __device__ __forceinline__ static void load(const uint16_t *row, float (&out)[N]) {
        cu32 *p = as_const(row);
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            const uint32_t w = p[j];
            out[2 * j] = bf16_lo(w);
            out[2 * j + 1] = bf16_hi(w);
        }
    }
};

template <int N>
struct SharedRow<float, N> {
    __device__ __forceinline__ static void load(const float *row, float (&out)[N]) {
        cu32 *p = as_const(row);
#pragma unroll
        for (int j = 0; j < N; ++j) out[j] = __uint_as_float(p[j]);
    }
};

}  // namespace ssm
