// Host-side interfaces between the C ABI (capi.hip) and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// How one selective-scan call is split along time.
//   chunks     : number of time chunks G (1 = no split)
//   chunk_len  : steps per chunk (the last one may be shorter)
// Workspace (when G > 1), per chain of 64 channels: aggregates[G-1][N+1][64]
// (fp32 end state from a zero state, then the summed step).
struct ScanPlan {
    int64_t chunks;
    int64_t chunk_len;
    size_t agg_offset;
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
    size_t states_offset;   // fp32 [B][nchunks][H][P][N]: chunk states from a zero state
    size_t sin_offset;      // bf16 [B][nchunks][H][P][N]: state entering each chunk
    size_t decay_offset;    // fp32 [B][H][nchunks]
    size_t bytes;
};

SSDPlan ssd_plan(const ssm_ssd_args &a);
ssm_status ssd_launch(const ssm_ssd_args &a, const SSDPlan &plan, hipStream_t stream,
                      char *err, size_t errlen);

// Gradients of the selective scan: chunks of 64 steps; workspace holds the
// per-chunk aggregates (forward and adjoint) and the composed entering states.
struct ScanBwdPlan {
    int64_t chunks;
    size_t aggF_offset;   // fp32 [chain][chunk][N+1][64]
    size_t aggR_offset;   // fp32 [chain][chunk][N][64]
    size_t hin_offset;    // fp32 [B][chunk][D][N]
    size_t uin_offset;    // fp32 [B][chunk][D][N]
    size_t dApart_offset; // fp32 [B][chunk][D][N]: per-chunk shares of dA
    size_t bytes;
};
ScanBwdPlan scan_bwd_plan(const ssm_scan_bwd_args &a);
ssm_status scan_bwd_launch(const ssm_scan_bwd_args &a, const ScanBwdPlan &plan, hipStream_t stream,
                           char *err, size_t errlen);

// Decode steps and the short convolution: no workspace, one kernel each.
ssm_status step_launch(const ssm_scan_step_args &a, hipStream_t stream, char *err, size_t errlen);
ssm_status ssd_step_launch(const ssm_ssd_step_args &a, hipStream_t stream, char *err, size_t errlen);
ssm_status conv_launch(const ssm_conv_args &a, hipStream_t stream, char *err, size_t errlen);

}  // namespace ssm
