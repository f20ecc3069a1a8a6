/*
 * ssm.h — C ABI of the MI355X (gfx950) selective-state-space library (libssm.so).
 *
 * Pages cited (titles as published; sections named as on the page):
 *   [Mamba-2 page]  "Mamba-2：把状态空间模型和 Attention 统一到一个数学框架里"
 *                   (aiplusplus.yigather.com/tech/05-27a2ce5d)
 *   [SSM page]      "状态空间模型与 Mamba：不用注意力读取长序列的方法"
 *                   (ai-trend.me/zh/study/state-space-models/)
 *   [Juejin page]   SSM/Mamba engineering article (juejin.cn/post/7634002571020402707)
 *   [Reading page]  "论文解读：Mamba — 线性时间的序列建模革命" (agent.eake.cn)
 *   [Hybrid page]   "基础知识：Mamba 与混合 SSM 架构" (charles2530.github.io)
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a caller-owned DEVICE pointer to contiguous
 *     row-major memory, last dimension fastest. The library never allocates,
 *     frees or copies device memory on its own; scratch space is the caller's
 *     `workspace`, sized by the matching *_workspace_bytes() query.
 *   - All argument checks run on the host, synchronously, before anything is
 *     enqueued. On any error nothing is launched, outputs are untouched, the
 *     call returns a non-zero ssm_status and ssm_last_error() describes it.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without waiting for it. A device fault surfaces on that stream.
 *   - Outputs must not alias inputs or each other. Apart from the fixed scratch
 *     array of selective_scan_fwd_noalloc (below), the library keeps no mutable
 *     global state (the error text is thread-local), so concurrent calls from
 *     several host threads are safe if their buffers are disjoint.
 *   - Tuning overrides, read from the environment at every call and meant for
 *     measurement only: SSM_SCAN_CHUNKS (time chunks of the scan's split, a
 *     positive integer; it changes the workspace size and the rounding order of
 *     the result, so query the size under the same setting and keep it fixed
 *     between selective_scan_chunk_states and selective_scan_apply), SSM_CONV_LANES
 *     and SSM_CONV_MIN_SEG (lanes in flight and the shortest time segment of
 *     causal_conv1d_fwd; the result is bit-identical under any setting). Unset,
 *     the library picks them itself.
 *   - Storage dtype SSM_BF16 means bfloat16 in memory; all arithmetic is fp32,
 *     the recurrent state is fp32, and bf16 outputs are rounded to nearest-even.
 *   - Byte offsets inside one batch row of a (batch, L, ...) tensor must fit in
 *     31 bits; larger shapes return SSM_ENOTSUP.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 6

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

typedef enum {
    SSM_OK = 0,
    SSM_EINVAL = 1,   /* null required pointer, negative size, misalignment, short workspace */
    SSM_ENOTSUP = 2,  /* well-formed but outside what the kernels implement (N, dtype, size) */
    SSM_EHIP = 3      /* the HIP runtime refused a launch */
} ssm_status;

/*
 * Selective scan (Mamba-1 form), per channel (b, d) with an N-dim fp32 state:
 *   dt_t   = softplus(delta[b,t,d] + delta_bias[d])      (or delta + bias when
 *                                                         delta_softplus == 0)
 *   h_t[n] = exp(dt_t * A[d,n]) * h_{t-1}[n] + dt_t * Bm[b,t,n] * x[b,t,d]
 *   y[b,t,d] = (sum_n Cm[b,t,n] h_t[n] + Dskip[d] * x[b,t,d]) * silu(z[b,t,d])
 *   h_final[b,d,:] = h_L (not gated), the state a later call takes as h0.
 * Sources: the discrete recurrence [Mamba-2 page, Background]; input-dependent
 * Delta, B, C with softplus on Delta [Mamba-2 page, Core idea step 1; Reading
 * page section 3]; the D x skip term [Juejin page, SSM basics]; the SiLU(z) gate
 * [Reading page section 5; Hybrid page section 3]; a per-channel N-dim state
 * [SSM page, how it works]; the state carried across calls for streaming
 * [Juejin page, long-document streaming step(x, state)]. Abar = exp(dt A) and the
 * Euler input term dt B x are the adopted discretisation.
 *
 * Layouts: x, delta, z, y: (batch, L, D), dtype. Bm, Cm: (batch, L, G, N), dtype:
 * G groups of B, C (ngroups; 0 or 1 = one group shared by every channel), channel
 * d reading group d / (D / G); G > 1 needs D / G to be a multiple of 64 (a wave
 * of 64 channels reads one row). A: (D, N) fp32 (diagonal, real; rows of the form
 * A[d,n] = (n+1) A[d,0] are detected on the device and take a faster exact path).
 * delta_bias, Dskip: (D) fp32. h0, h_final: (batch, D, N) fp32.
 * Nullable: z (no gate), delta_bias (0), Dskip (0), h0 (zero state),
 * h_final (not written). Supported: N in {16, 32, 64}; dtype F32 or BF16.
 * batch == 0 is a no-op; L == 0 writes h_final = h0 (or zeros).
 */
typedef struct ssm_scan_args {
    int64_t batch, seqlen, dim, dstate;   /* B, L, D, N */
    int64_t ngroups;                      /* G, groups of Bm/Cm (0 or 1: one) */
    ssm_dtype dtype;                      /* storage of x, delta, z, Bm, Cm, y */
    int32_t delta_softplus;               /* 1: softplus(delta + bias); 0: delta + bias */
    const void *x, *delta, *z;
    const void *Bm, *Cm;
    const float *A;
    const float *delta_bias;
    const float *Dskip;
    const float *h0;
    void *y;
    float *h_final;
    void *workspace;                      /* >= selective_scan_workspace_bytes(), 256-B aligned */
    size_t workspace_bytes;
} ssm_scan_args;

/*
 * Scalar-A state-space form (Mamba-2 "SSD"): H heads of P channels; a head shares
 * one step dt[b,t,h] and one scalar A[h] < 0, B and C are one group shared by all
 * heads, and every channel (h, p) keeps an N-dim state:
 *   dt_t = softplus(dt[b,t,h] + dt_bias[h]);  a_t = exp(dt_t A[h])
 *   S_t[h,p,:] = a_t S_{t-1}[h,p,:] + dt_t x[b,t,h,p] Bm[b,t,:]
 *   y[b,t,h,p] = (Cm[b,t,:] . S_t[h,p,:] + Dskip[h] x[b,t,h,p]) * silu(z[b,t,h,p])
 * computed in chunks of `chunk` steps through the semiseparable-matrix form:
 * inside a chunk y = (L o C B^T o decay o dt) x on the matrix cores, and chunk
 * states carry the rest [Mamba-2 page, Core idea step 2 and key points 1 and 3:
 * the SSM as a structured (semiseparable) attention-like matrix that runs as
 * matrix multiplication; selectivity restricted to keep that structure].
 * Layouts: x, z, y: (batch, L, H, P) dtype; dt: (batch, L, H) dtype; Bm, Cm:
 * (batch, L, G, N) dtype, head h reading group h / (H / G) (ngroups 0 or 1: one
 * group; H must be a multiple of G); dt_bias, A, Dskip: (H) fp32; h0, h_final:
 * (batch, H, P, N) fp32.
 * Nullable: z, dt_bias, Dskip, h0, h_final. Supported: dtype BF16; N in
 * {64, 128, 256}; P == 64; chunk in {64, 128, 256}. Any L >= 0 (the last chunk
 * may be short); results do not depend on `chunk` beyond rounding.
 */
typedef struct ssm_ssd_args {
    int64_t batch, seqlen, nheads, headdim, dstate, chunk;  /* B, L, H, P, N, Q */
    int64_t ngroups;                                        /* G (0 or 1: one group) */
    ssm_dtype dtype;
    int32_t dt_softplus;                  /* 1: softplus(dt + bias); 0: dt + bias */
    const void *x;
    const void *dt;
    const float *dt_bias;
    const float *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    void *y;
    float *h_final;
    void *workspace;                      /* >= ssd_chunked_workspace_bytes(), 256-B aligned */
    size_t workspace_bytes;
} ssm_ssd_args;

/* Enqueue the selective scan. Errors: SSM_EINVAL, SSM_ENOTSUP (before any launch),
 * SSM_EHIP (a launch was refused; earlier kernels of this call may have run). */
ssm_status selective_scan_fwd(const ssm_scan_args *args, hipStream_t stream);

/* The same computation in its two passes, for callers that time or schedule them
 * separately (or exchange chunk states between devices of a sequence-sharded
 * scan, where the state entering a shard is that shard's h0):
 *   selective_scan_chunk_states: the affine map of every time chunk but the last
 *     (its end state from a zero state and its decay), then the composition of
 *     those maps from the start of the sequence to each chunk, into `workspace`
 *     (nothing when the call is not split in time). Independent of h0.
 *   selective_scan_apply: applies each chunk's composed map to h0 to get the
 *     state entering it, then runs every chunk again with readout: writes y
 *     and h_final. Needs the workspace filled by selective_scan_chunk_states with
 *     the same arguments (same sizes, inputs and workspace; h0 may differ).
 * selective_scan_fwd == selective_scan_chunk_states followed by selective_scan_apply.
 * Errors as for selective_scan_fwd. */
ssm_status selective_scan_chunk_states(const ssm_scan_args *args, hipStream_t stream);
ssm_status selective_scan_apply(const ssm_scan_args *args, hipStream_t stream);

/* Host-only check of `args` (no HIP call): the status selective_scan_fwd would
 * return from its argument checks, ignoring the workspace pointer and size. */
ssm_status selective_scan_validate(const ssm_scan_args *args);

/* Workspace bytes selective_scan_fwd needs for these sizes (0 if none, or if the
 * sizes, dtype or state size are invalid). Reads only batch, seqlen, dim, dstate
 * and dtype; the pointers may be NULL. Host-only. */
size_t selective_scan_workspace_bytes(const ssm_scan_args *args);

/* selective_scan_fwd without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Its scratch space is a fixed
 * device array of SSM_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU,
 * held until the process ends; args->workspace and args->workspace_bytes are
 * ignored. Same arguments, results (bit for bit) and errors as
 * selective_scan_fwd, plus SSM_ENOTSUP, before anything is enqueued, when the call
 * needs more scratch than that (selective_scan_workspace_bytes(args) >
 * SSM_NOALLOC_SCRATCH_BYTES; with N = 16 the library's own time split never
 * needs more), and SSM_EHIP when the
 * array's address cannot be obtained on the current device. Every call on one GPU
 * uses that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller. No part of
 * the array needs to start at zero: every value a call reads was written earlier
 * in the same call. */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
ssm_status selective_scan_fwd_noalloc(const ssm_scan_args *args, hipStream_t stream);

/*
 * Gradients of the selective scan (training) for the loss
 *   sum(dy * y) + sum(dh_final * h_final)
 * with y, h_final as selective_scan_fwd computes them from the same inputs. The
 * forward is recomputed, nothing from it is needed. [Mamba-2 page, Core idea:
 * Mamba-1's scan, its training throughput.] Reverse-mode through the recurrence:
 *   dyc_t = dy_t silu(z_t);  g_t = C_t dyc_t + exp(dt_{t+1} A) o g_{t+1}  (adjoint of h_t,
 *   the last step adds dh_final);  dB_t += g_t dt_t x_t, dC_t += dyc_t h_t (summed over
 *   the channels of a group);  dx_t = dyc_t Dskip + dt_t sum_n g_t B_t;
 *   d dt_t = sum_n g_t (B_t x_t + A exp(dt_t A) h_{t-1});  ddelta = d dt * softplus';
 *   dA += g_t dt_t exp(dt_t A) h_{t-1};  dDskip += dyc_t x_t;  dz_t = dy_t (C_t.h_t +
 *   Dskip x_t) silu'(z_t);  dh0 = exp(dt_0 A) o g_0.
 * Forward inputs exactly as ssm_scan_args (same layouts, same nullability; N in
 * {16, 32, 64}). dy: (batch, L, D) dtype. dh_final: (batch, D, N) fp32, nullable (0).
 * Outputs, all written in full (accumulated ones are zeroed first):
 *   dx, ddelta: (batch, L, D) dtype; dz: (batch, L, D) dtype, required iff z != NULL;
 *   dB, dC: (batch, L, G, N) fp32; dA: (D, N) fp32; dDskip, ddelta_bias: (D) fp32,
 *   nullable (not computed); dh0: (batch, D, N) fp32, nullable.
 * Every gradient is deterministic: the sums over channels (dB, dC), chunks and
 * batch rows (dA, dDskip, ddelta_bias) are formed from stored partials in a fixed
 * order, so repeated calls give identical bits.
 */
typedef struct ssm_scan_bwd_args {
    int64_t batch, seqlen, dim, dstate;   /* B, L, D, N */
    int64_t ngroups;
    ssm_dtype dtype;
    int32_t delta_softplus;
    const void *x, *delta, *z;
    const void *Bm, *Cm;
    const float *A, *delta_bias, *Dskip, *h0;
    const void *dy;
    const float *dh_final;
    void *dx, *ddelta, *dz;
    float *dB, *dC, *dA, *dDskip, *ddelta_bias, *dh0;
    void *workspace;                      /* >= selective_scan_bwd_workspace_bytes(), 256-B aligned */
    size_t workspace_bytes;
} ssm_scan_bwd_args;

ssm_status selective_scan_bwd(const ssm_scan_bwd_args *args, hipStream_t stream);

/* Workspace bytes selective_scan_bwd needs (sizes, dtype and dstate only; 0 if invalid). */
size_t selective_scan_bwd_workspace_bytes(const ssm_scan_bwd_args *args);

/* Enqueue the chunked scalar-A (SSD) form. Errors as for selective_scan_fwd. */
ssm_status ssd_chunked_fwd(const ssm_ssd_args *args, hipStream_t stream);

/* Host-only argument check of the SSD form, ignoring the workspace. */
ssm_status ssd_chunked_validate(const ssm_ssd_args *args);

/* Workspace bytes ssd_chunked_fwd needs for these sizes (0 if invalid). Reads only
 * the sizes and dtype; the pointers may be NULL. Host-only. */
size_t ssd_chunked_workspace_bytes(const ssm_ssd_args *args);

/*
 * Gradients of the scalar-A (SSD) form for the loss sum(dy * y) + sum(dh_final *
 * h_final), with y, h_final as ssd_chunked_fwd computes them from the same inputs
 * (recomputed; nothing from the forward is needed) [Mamba-2 page, Core idea:
 * training throughput of the scan; key point 3: the scalar-times-identity decay
 * that keeps the matrix form]. Per head h (channels p, states n), with
 * g_t = dL/dS_t the adjoint state and dyc = dy silu(z):
 *   g_t = C_t (x) dyc_t + a_{t+1} g_{t+1}  (the last step adds dh_final);
 *   dx_t = dt_t g_t B_t + Dskip dyc_t;  dB_t += dt_t g_t^T x_t, dC_t += S_t^T dyc_t
 *   (summed over the heads of a group);  d dt_t = sum_{p,n} g_t (x_t B_t^T + A a_t S_{t-1});
 *   ddt = d dt * softplus';  dA += sum_{t,p,n} g_t dt_t a_t S_{t-1};  dDskip += dyc_t . x_t;
 *   dz_t = dy_t (C_t S_t + Dskip x_t) silu'(z_t);  dh0 = a_0 g_0.
 * Computed chunk by chunk on the matrix cores (dx, dB, dC, the adjoint states);
 * the decay gradients come from fp32 sums of the chunk's (t, s) terms.
 * Forward inputs exactly as ssm_ssd_args (dtype BF16, P == 64, chunk in {64, 128,
 * 256}; N in {64, 128, 256}). dy: (batch, L, H, P) bf16. dh_final: (batch, H, P, N) fp32,
 * nullable (0). Outputs, all written in full:
 *   dx: (batch, L, H, P) bf16; ddt: (batch, L, H) bf16 (gradient of the raw dt);
 *   dz: (batch, L, H, P) bf16, required iff z != NULL; dB, dC: (batch, L, G, N) fp32;
 *   dA: (H) fp32; dDskip, ddt_bias: (H) fp32, nullable (not computed); dh0:
 *   (batch, H, P, N) fp32, nullable.
 * dA, dDskip and ddt_bias are sums of float atomics: equal to the last bits only up
 * to summation order, run to run; dx, ddt, dz, dB, dC and dh0 are deterministic.
 */
typedef struct ssm_ssd_bwd_args {
    int64_t batch, seqlen, nheads, headdim, dstate, chunk;  /* B, L, H, P, N, Q */
    int64_t ngroups;
    ssm_dtype dtype;
    int32_t dt_softplus;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    const void *dy;
    const float *dh_final;
    void *dx, *ddt, *dz;
    float *dB, *dC, *dA, *dDskip, *ddt_bias, *dh0;
    void *workspace;                      /* >= ssd_chunked_bwd_workspace_bytes(), 256-B aligned */
    size_t workspace_bytes;
} ssm_ssd_bwd_args;

ssm_status ssd_chunked_bwd(const ssm_ssd_bwd_args *args, hipStream_t stream);

/* Workspace bytes ssd_chunked_bwd needs (sizes, dtype and whether z is given; 0 if
 * invalid). Host-only. */
size_t ssd_chunked_bwd_workspace_bytes(const ssm_ssd_bwd_args *args);

/*
 * One decode step of the selective scan (a sequence of length 1), the state read
 * and written in place:
 *   dt = softplus(delta[b,d] + delta_bias[d])     (delta + bias if delta_softplus == 0)
 *   state[b,d,n] <- exp(dt A[d,n]) state[b,d,n] + dt Bm[b,n] x[b,d]
 *   y[b,d] = (sum_n Cm[b,n] state[b,d,n] + Dskip[d] x[b,d]) * silu(z[b,d])
 * This is selective_scan_fwd over one token with h0 = state and h_final written
 * back to state [Juejin page, long-document streaming: step(x, state) returns the
 * output and the next state; SSM page, how it works: inference keeps a fixed-size
 * state per channel and advances it token by token].
 * Layouts: x, delta, z, y: (batch, D) dtype; Bm, Cm: (batch, G, N) dtype (channel d
 * reads group d / (D / G)); A: (D, N) fp32; delta_bias, Dskip: (D) fp32; state:
 * (batch, D, N) fp32, 16-byte aligned
 * (the layout of h0 / h_final above). Nullable: z, delta_bias, Dskip.
 * Supported: N in {16, 32, 64, 128, 256}; dtype F32 or BF16. batch == 0 is a no-op.
 */
typedef struct ssm_scan_step_args {
    int64_t batch, dim, dstate;           /* B, D, N */
    int64_t ngroups;                      /* G (0 or 1: one group); D % G == 0 */
    ssm_dtype dtype;                      /* storage of x, delta, z, Bm, Cm, y */
    int32_t delta_softplus;
    const void *x, *delta, *z;
    const void *Bm, *Cm;
    const float *A;
    const float *delta_bias;
    const float *Dskip;
    float *state;                         /* in/out */
    void *y;
} ssm_scan_step_args;

ssm_status selective_state_update(const ssm_scan_step_args *args, hipStream_t stream);

/*
 * One decode step of the scalar-A (SSD) form, state in place: per head h,
 *   dt = softplus(dt[b,h] + dt_bias[h]);  a = exp(dt A[h])
 *   state[b,h,p,n] <- a state[b,h,p,n] + dt Bm[b,n] x[b,h,p]
 *   y[b,h,p] = (sum_n Cm[b,n] state[b,h,p,n] + Dskip[h] x[b,h,p]) * silu(z[b,h,p])
 * [Mamba-2 page, Background: the discrete recurrence, here with one scalar decay
 * per head; Juejin page, step(x, state)]. ssd_chunked_fwd over one token with
 * h0 = state and h_final written back to state.
 * Layouts: x, z, y: (batch, H, P) dtype; dt: (batch, H) dtype; Bm, Cm: (batch, G, N)
 * dtype (head h reads group h / (H / G)); dt_bias, A, Dskip: (H) fp32; state:
 * (batch, H, P, N) fp32, 16-byte aligned.
 * Nullable: z, dt_bias, Dskip. Supported: any P >= 1; N in {16, 32, 64, 128, 256};
 * dtype F32 or BF16.
 */
typedef struct ssm_ssd_step_args {
    int64_t batch, nheads, headdim, dstate;   /* B, H, P, N */
    int64_t ngroups;                          /* G (0 or 1: one group); H % G == 0 */
    ssm_dtype dtype;
    int32_t dt_softplus;
    const void *x;
    const void *dt;
    const float *dt_bias;
    const float *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    float *state;                             /* in/out */
    void *y;
} ssm_ssd_step_args;

ssm_status ssd_state_update(const ssm_ssd_step_args *args, hipStream_t stream);

/*
 * Causal depthwise convolution along time with bias and SiLU, the short Conv1d the
 * x branch passes before the scan [Reading page section 5 and Hybrid page section
 * 3: Conv1d then SiLU ahead of the SSM; Juejin page, basic usage: width d_conv = 4]:
 *   xx = [init_state ; x] along time (zeros when init_state is NULL)
 *   y[b,t,d] = silu(bias[d] + sum_{k<K} weight[d,k] xx[b, t-(K-1)+k, d])
 *   (apply_silu == 0: no SiLU)
 *   final_state[b,:,d] = the last K-1 entries of xx: the init_state of a call that
 *   continues the same sequence.
 * Layouts: x, y: (batch, L, D) dtype; weight: (D, K) fp32; bias: (D) fp32;
 * init_state, final_state: (batch, K-1, D) dtype. Nullable: bias, init_state,
 * final_state. final_state must not alias init_state or x. Supported: K in
 * {2, 3, 4}; dtype F32 or BF16. L == 0 writes final_state = init_state (or zeros).
 */
typedef struct ssm_conv_args {
    int64_t batch, seqlen, dim, width;    /* B, L, D, K */
    ssm_dtype dtype;
    int32_t apply_silu;
    const void *x;
    const float *weight;
    const float *bias;
    const void *init_state;
    void *y;
    void *final_state;
} ssm_conv_args;

ssm_status causal_conv1d_fwd(const ssm_conv_args *args, hipStream_t stream);

/* Static name of a status code ("SSM_OK", ...). */
const char *ssm_status_str(ssm_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *ssm_last_error(void);

/* SSM_ABI_VERSION of the built library. */
int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSM_H */
