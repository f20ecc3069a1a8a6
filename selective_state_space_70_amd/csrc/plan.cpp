// Host-side plans: how each call is split into chunks and launches, and where
// its scratch buffers sit in the caller's workspace. Plain C++ (no device code),
// shared by the C ABI's workspace queries and the kernel launchers.
#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "internal.h"

namespace ssm {

ScanPlan scan_plan(const ssm_scan_args &a) {
    ScanPlan pl{};
    pl.chunks = 1;
    pl.chunk_len = a.seqlen;
    if (a.seqlen <= 0 || a.batch <= 0 || a.dim <= 0) return pl;
    // One wave per (b, 64 channels, chunk). Aim at ~4096 waves: four per SIMD on
    // the 1024 SIMDs, all resident at once (the main pass fits four per SIMD),
    // which balances the SIMDs and hides memory latency (never more than 4096, so
    // no SIMD gets a fifth wave to run after the others); chunks stay >= 32 steps.
    const int64_t waves = a.batch * ((a.dim + 63) / 64);
    int64_t G = std::max<int64_t>(1, 4096 / waves);
    G = std::min<int64_t>(G, std::max<int64_t>(1, a.seqlen / 32));
    if (const char *env = std::getenv("SSM_SCAN_CHUNKS")) {  // tuning override
        const long v = std::strtol(env, nullptr, 10);
        if (v > 0) G = v;
    }
    G = std::max<int64_t>(1, std::min<int64_t>(G, std::min<int64_t>(a.seqlen, 65535)));
    pl.chunk_len = (a.seqlen + G - 1) / G;
    if (G > 1) pl.chunk_len = (pl.chunk_len + 3) / 4 * 4;
    pl.chunks = (a.seqlen + pl.chunk_len - 1) / pl.chunk_len;
    if (pl.chunks > 1) {
        auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
        const size_t chains = (size_t)a.batch * ((a.dim + 63) / 64);
        const size_t G = (size_t)pl.chunks;
        const size_t blocks = up(chains * (G - 1) * (a.dstate + 1) * 64 * sizeof(float));
        pl.agg_offset = 0;
        pl.pre_offset = blocks;
        pl.bytes = 2 * blocks;
    }
    return pl;
}

// fp32 [B][H][P][N] after the decays: the last chunk's state (it feeds h_final only)
size_t ssd_last_state_offset(const ssm_ssd_args &a, const SSDPlan &pl) {
    return pl.decay_offset + (((size_t)a.batch * a.nheads * pl.nchunks * sizeof(float) + 255) & ~(size_t)255);
}

SSDPlan ssd_plan(const ssm_ssd_args &a) {
    SSDPlan pl{};
    if (a.batch <= 0 || a.seqlen <= 0 || a.chunk <= 0) return pl;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    pl.nchunks = (a.seqlen + a.chunk - 1) / a.chunk;
    const size_t elems = (size_t)a.batch * pl.nchunks * a.nheads * a.dstate * a.headdim;
    pl.states_offset = 0;
    // the entering states overwrite the bf16 chunk states in place (the state pass
    // reads each element before it writes it): one buffer, and a smaller working set
    // for the output launch that reads x again
    pl.sin_offset = pl.states_offset;
    pl.decay_offset = pl.sin_offset + up(elems * sizeof(uint16_t));
    pl.gsc_offset = ssd_last_state_offset(a, pl) + up((size_t)a.batch * a.nheads * a.headdim * a.dstate * sizeof(float));
    // 32 x 32 fp32 blocks of C B^T on and below the diagonal of each chunk
    const size_t tiles = (size_t)(a.chunk + 31) / 32;
    const size_t G = a.ngroups > 1 ? (size_t)a.ngroups : 1;
    pl.gsc_bytes = up((size_t)a.batch * pl.nchunks * G * (tiles * (tiles + 1) / 2) * 1024 * sizeof(float));
    pl.bytes = pl.gsc_offset + pl.gsc_bytes;
    return pl;
}

ScanBwdPlan scan_bwd_plan(const ssm_scan_bwd_args &a) {
    ScanBwdPlan pl{};
    if (a.batch <= 0 || a.seqlen <= 0 || a.dim <= 0) return pl;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const int64_t N = a.dstate;
    pl.chunks = (a.seqlen + kScanBwdChunk - 1) / kScanBwdChunk;
    const size_t chains = (size_t)a.batch * ((a.dim + 63) / 64);
    pl.aggF_offset = 0;
    pl.aggR_offset = up(chains * pl.chunks * (N + 1) * 64 * sizeof(float));
    pl.hin_offset = pl.aggR_offset + up(chains * pl.chunks * N * 64 * sizeof(float));
    const size_t st = (size_t)a.batch * pl.chunks * a.dim * N * sizeof(float);
    pl.uin_offset = pl.hin_offset + up(st);
    pl.dApart_offset = pl.uin_offset + up(st);
    const size_t cd = (size_t)a.batch * pl.chunks * a.dim * sizeof(float);
    pl.dDpart_offset = pl.dApart_offset + up(st);
    pl.dbpart_offset = pl.dDpart_offset + up(cd);
    pl.bcpart_offset = pl.dbpart_offset + up(cd);
    const int64_t waves = (a.dim + 64 * 16 / N - 1) / (64 * 16 / N);   // main-kernel waves along D
    // one (step, wave) row per step and batch row, plus a spare row
    pl.fast_offset = pl.bcpart_offset + up(((size_t)a.batch * a.seqlen + 1) * waves * 2 * N * sizeof(float));
    pl.bytes = pl.fast_offset + up((size_t)((a.dim + 63) / 64) * sizeof(int32_t));
    return pl;
}

SSDBwdPlan ssd_bwd_plan(const ssm_ssd_bwd_args &a) {
    SSDBwdPlan pl{};
    if (a.batch <= 0 || a.seqlen <= 0 || a.chunk <= 0) return pl;
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const int64_t G = a.ngroups > 1 ? a.ngroups : 1;
    const int64_t hpg = a.nheads / G;
    pl.nchunks = (a.seqlen + a.chunk - 1) / a.chunk;
    pl.hs_col = kSsdBwdHeadsCol;
    pl.hs_row = kSsdBwdHeadsRow;
    pl.slices_col = (hpg + kSsdBwdHeadsCol - 1) / kSsdBwdHeadsCol;
    pl.slices_row = (hpg + kSsdBwdHeadsRow - 1) / kSsdBwdHeadsRow;
    const size_t st = (size_t)a.batch * pl.nchunks * a.nheads * a.headdim * a.dstate;
    const size_t blhp = (size_t)a.batch * a.seqlen * a.nheads * a.headdim;
    const size_t blh = (size_t)a.batch * a.seqlen * a.nheads;
    const size_t bln = (size_t)a.batch * a.seqlen * G * a.dstate;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
    pl.sin32_offset = take(st * 4);
    pl.sin_offset = take(st * 2);
    pl.decay_offset = take((size_t)a.batch * a.nheads * pl.nchunks * 4);
    pl.hfin_offset = take((size_t)a.batch * a.nheads * a.headdim * a.dstate * 4);
    pl.gout_offset = take(st * 4);
    pl.kc_offset = take((size_t)a.batch * a.nheads * pl.nchunks * (a.headdim * a.dstate / 256) * 4);
    const bool z = a.z != nullptr;
    pl.y32_offset = take(z ? blhp * 4 : 0);
    pl.dych_offset = take(z ? blhp * 2 : 0);
    pl.dycl_offset = take(z ? blhp * 2 : 0);
    pl.q_offset = take(blh * 4);
    pl.dtdd_offset = take(blh * 4);
    pl.dd_offset = take(blh * 4);
    pl.dBp_offset = take((size_t)pl.slices_col * bln * 4);
    pl.dCp_offset = take((size_t)pl.slices_row * bln * 4);
    pl.bytes = off;
    return pl;
}

}  // namespace ssm
