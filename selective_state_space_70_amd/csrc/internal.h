// Host-side interfaces between the C ABI (capi.hip) and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// Steps per chunk of the scan gradients (a chunk's states live in VGPRs).
constexpr int kScanBwdChunk = 64;
// Heads per workgroup of the SSD-gradient column kernel (a dx accumulator each)
// and row kernel.
constexpr int kSsdBwdHeadsCol = 2;
constexpr int kSsdBwdHeadsRow = 4;

// How one selective-scan call is split along time.
//   chunks     : number of time chunks G (1 = no split)
//   chunk_len  : steps per chunk (the last one may be shorter)
// Workspace (when G > 1), per chain of 64 channels, two fp32 blocks [G-1][N+1][64]:
// the aggregates (each chunk's end state from a zero state, then its decay: the
// product of its steps' exp(dt A[0]) on the fast path, its summed step otherwise)
// and the prefixes (the composed map entering chunks 1..G-1, same layout).
struct ScanPlan {
    int64_t chunks;
    int64_t chunk_len;
    size_t agg_offset;
    size_t pre_offset;
    size_t bytes;
};

ScanPlan scan_plan(const ssm_scan_args &a);
// Enqueue the kernels of one call; returns SSM_EHIP with `err` filled on a refused launch.
// `passes`: bit 0 = chunk states, bit 1 = apply (readout).
ssm_status scan_launch(const ssm_scan_args &a, const ScanPlan &plan, hipStream_t stream,
                       int passes, char *err, size_t errlen);

// SSD (scalar A per head) plan: chunk states and the carried state per chunk.
struct SSDPlan {
    int64_t nchunks;
    size_t states_offset;   // bf16 [B][nchunks][H][P][N]: chunk states from a zero state
    size_t sin_offset;      // the same buffer: the state entering each chunk, written
                            // over the chunk states by the state pass
    size_t decay_offset;    // fp32 [B][H][nchunks]
    size_t gsc_offset;      // fp32 score blocks: [B][nchunks][G][blocks][1024]
    size_t gsc_bytes;
    size_t bytes;
};

SSDPlan ssd_plan(const ssm_ssd_args &a);
// fp32 [B][H][P][N] after the decays: the last chunk's state (it feeds h_final only)
size_t ssd_last_state_offset(const ssm_ssd_args &a, const SSDPlan &pl);
ssm_status ssd_launch(const ssm_ssd_args &a, const SSDPlan &plan, hipStream_t stream,
                      char *err, size_t errlen);

// Pieces of the SSD forward the gradient pass reruns (what: 0 = split-precision
// chunk states and the entering states, 1 = fp32 pre-gate output, 2 = adjoint
// aggregates with exp(cs_t) weights). N in {64, 128, 256}.
struct SSDK;
void ssd_recompute_launch(const SSDK &k, int batch, int Q, int N, int what, hipStream_t s);

// Gradients of the SSD form (see ssd_bwd.hip for the buffers).
struct SSDBwdPlan {
    int64_t nchunks, slices_col, slices_row;
    int32_t hs_col, hs_row;   // heads per workgroup of the column / row kernels
    size_t sin32_offset;      // fp32 [B][nc][H][P][N]: chunk states, then entering states
    size_t sin_offset;        // bf16 [B][nc][H][P][N]: entering states (forward output recompute)
    size_t decay_offset;      // fp32 [B][H][nc]
    size_t hfin_offset;       // fp32 [B][H][P][N]: final state of the recompute
    size_t gout_offset;       // fp32 [B][nc][H][P][N]: adjoint aggregates, then adjoint at chunk ends
    size_t kc_offset;         // fp32 [B][H][nc][P N / 256]: per-wave shares of <adjoint, state> at each chunk end
    size_t y32_offset;        // fp32 (B, L, H, P): pre-gate output (only with z)
    size_t dych_offset;       // bf16 (B, L, H, P): dy silu(z), hi part (only with z)
    size_t dycl_offset;       // bf16 (B, L, H, P): lo part (only with z)
    size_t q_offset;          // fp32 (B, L, H): sum_p dyc (y - D x)
    size_t dtdd_offset;       // fp32 (B, L, H): dt_t sum_{p,n} g_t x_t B_t
    size_t dd_offset;         // fp32 (B, L, H): sum_{p,n} g_t x_t B_t
    size_t dBp_offset;        // fp32 [slices_col][B][L][G][N]
    size_t dCp_offset;        // fp32 [slices_row][B][L][G][N]
    size_t bytes;
};
SSDBwdPlan ssd_bwd_plan(const ssm_ssd_bwd_args &a);
ssm_status ssd_bwd_launch(const ssm_ssd_bwd_args &a, const SSDBwdPlan &plan, hipStream_t stream,
                          char *err, size_t errlen);

// Gradients of the selective scan: chunks of 64 steps; workspace holds the
// per-chunk aggregates (forward and adjoint) and the composed entering states.
struct ScanBwdPlan {
    int64_t chunks;
    size_t aggF_offset;   // fp32 [chain][chunk][N+1][64]
    size_t aggR_offset;   // fp32 [chain][chunk][N][64]
    size_t hin_offset;    // fp32 [B][chunk][N][D]
    size_t uin_offset;    // fp32 [B][chunk][N][D]
    size_t dApart_offset; // fp32 [B][chunk][D][N]: per-chunk shares of dA
    size_t dDpart_offset; // fp32 [B][chunk][D]: per-chunk shares of dDskip
    size_t dbpart_offset; // fp32 [B][chunk][D]: per-chunk shares of ddelta_bias
    size_t bcpart_offset; // fp32 [B L + 1][waves along D][2N]: per-wave sums of dB_t, dC_t (+ a spare row)
    size_t fast_offset;   // int32 [ceil(D / 64)]: which path each 64 channels take
    size_t bytes;
};
ScanBwdPlan scan_bwd_plan(const ssm_scan_bwd_args &a);
ssm_status scan_bwd_launch(const ssm_scan_bwd_args &a, const ScanBwdPlan &plan, hipStream_t stream,
                           char *err, size_t errlen);

// Set the thread's ssm_last_error() text (printf format); returns `s`.
ssm_status set_last_error(ssm_status s, const char *fmt, ...);

// Decode steps and the short convolution: no workspace, one kernel each.
ssm_status step_launch(const ssm_scan_step_args &a, hipStream_t stream, char *err, size_t errlen);
ssm_status ssd_step_launch(const ssm_ssd_step_args &a, hipStream_t stream, char *err, size_t errlen);
ssm_status conv_launch(const ssm_conv_args &a, hipStream_t stream, char *err, size_t errlen);

}  // namespace ssm
