// Address/undefined-behaviour sanitizer run of the host side of the C ABI (CPU
// only, no GPU call): every argument check, workspace query and plan is driven
// with random sizes drawn from the values around each documented limit (negative,
// zero, one, the limits themselves and just past them, values whose products
// overflow 64 bits) and random null / aligned / misaligned pointers. The
// undefined-behaviour sanitizer aborts on a signed overflow in a size product;
// the entry points are called only when the check rejects the arguments, which
// must happen before any HIP call. Exit status 0 when every result is one of the
// documented statuses and every rejection left a message.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ssm.h"

static uint64_t g_state = 0xD1B54A32D192ED03ull;
static uint64_t rnd() {
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return g_state;
}
static int64_t pick(const int64_t *v, int n) { return v[rnd() % n]; }

static const int64_t kSizes[] = {-1, 0, 1, 2, 3, 7, 16, 63, 64, 65, 100, 128, 255, 256, 257, 4096,
                                 65535, 65536, 131072, (1 << 20), (1 << 30), (1 << 30) + 1,
                                 (int64_t)1 << 31, ((int64_t)1 << 31) - 1, (int64_t)1 << 34,
                                 (int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX, INT64_MIN};
static const int64_t kSmall[] = {-1, 0, 1, 2, 3, 4, 5, 8, 16, 17, 32, 64, 100, 128, 256, 512,
                                 (int64_t)1 << 40, INT64_MAX};
static const int kNS = sizeof kSizes / sizeof kSizes[0];
static const int kNM = sizeof kSmall / sizeof kSmall[0];

static void *ptr() {
    switch (rnd() % 4) {
        case 0: return nullptr;
        case 1: return (void *)(uintptr_t)0x10000;   // never dereferenced on the host
        case 2: return (void *)(uintptr_t)0x10002;
        default: return (void *)(uintptr_t)0x10100;
    }
}
static ssm_dtype dtype() {
    static const int v[] = {SSM_F32, SSM_BF16, SSM_BF16, 7};
    return (ssm_dtype)v[rnd() % 4];
}

static int fails = 0;
static void expect_status(ssm_status s, const char *who) {
    if (s != SSM_OK && s != SSM_EINVAL && s != SSM_ENOTSUP) {
        std::fprintf(stderr, "FAIL: %s returned %d\n", who, (int)s);
        ++fails;
    }
    if (s != SSM_OK && std::strlen(ssm_last_error()) == 0) {
        std::fprintf(stderr, "FAIL: %s rejected without a message\n", who);
        ++fails;
    }
}

int main() {
    const hipStream_t st = nullptr;
    // a null argument block is rejected by every entry point
    expect_status(selective_scan_validate(nullptr), "scan validate(NULL)");
    expect_status(selective_scan_fwd(nullptr, st), "scan fwd(NULL)");
    expect_status(ssd_chunked_validate(nullptr), "ssd validate(NULL)");
    expect_status(ssd_chunked_fwd(nullptr, st), "ssd fwd(NULL)");
    expect_status(selective_scan_bwd(nullptr, st), "scan bwd(NULL)");
    expect_status(ssd_chunked_bwd(nullptr, st), "ssd bwd(NULL)");
    expect_status(selective_state_update(nullptr, st), "step(NULL)");
    expect_status(ssd_state_update(nullptr, st), "ssd step(NULL)");
    expect_status(causal_conv1d_fwd(nullptr, st), "conv(NULL)");
    if (selective_scan_workspace_bytes(nullptr) || ssd_chunked_workspace_bytes(nullptr) ||
        selective_scan_bwd_workspace_bytes(nullptr) || ssd_chunked_bwd_workspace_bytes(nullptr)) {
        std::fprintf(stderr, "FAIL: a workspace query of NULL is not 0\n");
        ++fails;
    }
    long accepted = 0;
    for (int it = 0; it < 200000; ++it) {
        {
            ssm_scan_args a{};
            a.batch = pick(kSmall, kNM); a.seqlen = pick(kSizes, kNS); a.dim = pick(kSizes, kNS);
            a.dstate = pick(kSmall, kNM); a.ngroups = pick(kSmall, kNM); a.dtype = dtype();
            a.x = ptr(); a.delta = ptr(); a.z = ptr(); a.Bm = ptr(); a.Cm = ptr();
            a.A = (const float *)ptr(); a.delta_bias = (const float *)ptr(); a.Dskip = (const float *)ptr();
            a.h0 = (const float *)ptr(); a.y = ptr(); a.h_final = (float *)ptr();
            a.workspace = ptr(); a.workspace_bytes = (size_t)pick(kSizes, kNS);
            (void)selective_scan_workspace_bytes(&a);
            const ssm_status s = selective_scan_validate(&a);
            expect_status(s, "scan validate");
            if (s != SSM_OK) {
                expect_status(selective_scan_fwd(&a, st), "scan fwd");
                expect_status(selective_scan_chunk_states(&a, st), "scan chunk states");
                expect_status(selective_scan_apply(&a, st), "scan apply");
            } else {
                ++accepted;
            }
        }
        {
            ssm_ssd_args a{};
            a.batch = pick(kSmall, kNM); a.seqlen = pick(kSizes, kNS); a.nheads = pick(kSmall, kNM);
            a.headdim = pick(kSmall, kNM); a.dstate = pick(kSmall, kNM); a.chunk = pick(kSmall, kNM);
            a.ngroups = pick(kSmall, kNM); a.dtype = dtype();
            a.x = ptr(); a.dt = ptr(); a.dt_bias = (const float *)ptr(); a.A = (const float *)ptr();
            a.Bm = ptr(); a.Cm = ptr(); a.Dskip = (const float *)ptr(); a.z = ptr();
            a.h0 = (const float *)ptr(); a.y = ptr(); a.h_final = (float *)ptr();
            a.workspace = ptr(); a.workspace_bytes = (size_t)pick(kSizes, kNS);
            (void)ssd_chunked_workspace_bytes(&a);
            const ssm_status s = ssd_chunked_validate(&a);
            expect_status(s, "ssd validate");
            if (s != SSM_OK) expect_status(ssd_chunked_fwd(&a, st), "ssd fwd");
        }
        {
            ssm_scan_bwd_args a{};
            a.batch = pick(kSmall, kNM); a.seqlen = pick(kSizes, kNS); a.dim = pick(kSizes, kNS);
            a.dstate = pick(kSmall, kNM); a.ngroups = pick(kSmall, kNM); a.dtype = dtype();
            a.x = ptr(); a.delta = ptr(); a.z = ptr(); a.Bm = ptr(); a.Cm = ptr(); a.dy = ptr();
            a.A = nullptr; a.dx = ptr(); a.ddelta = ptr(); a.dz = ptr();
            a.dB = (float *)ptr(); a.dC = (float *)ptr(); a.dA = (float *)ptr();
            a.workspace = ptr(); a.workspace_bytes = (size_t)pick(kSizes, kNS);
            (void)selective_scan_bwd_workspace_bytes(&a);
            // no A: rejected unless batch == 0, which returns before any HIP call
            expect_status(selective_scan_bwd(&a, st), "scan bwd");
        }
        {
            ssm_ssd_bwd_args a{};
            a.batch = pick(kSmall, kNM); a.seqlen = pick(kSizes, kNS); a.nheads = pick(kSmall, kNM);
            a.headdim = pick(kSmall, kNM); a.dstate = pick(kSmall, kNM); a.chunk = pick(kSmall, kNM);
            a.ngroups = pick(kSmall, kNM); a.dtype = dtype();
            a.x = ptr(); a.dt = ptr(); a.A = nullptr; a.Bm = ptr(); a.Cm = ptr();
            a.z = ptr(); a.dy = ptr(); a.dx = ptr(); a.ddt = ptr(); a.dz = ptr();
            a.dB = (float *)ptr(); a.dC = (float *)ptr(); a.dA = (float *)ptr();
            a.workspace = ptr(); a.workspace_bytes = (size_t)pick(kSizes, kNS);
            (void)ssd_chunked_bwd_workspace_bytes(&a);
            expect_status(ssd_chunked_bwd(&a, st), "ssd bwd");   // as above: no A
        }
        {
            ssm_scan_step_args a{};
            a.batch = pick(kSizes, kNS); a.dim = pick(kSizes, kNS); a.dstate = pick(kSmall, kNM);
            a.ngroups = pick(kSmall, kNM); a.dtype = dtype();
            a.x = ptr(); a.delta = ptr(); a.z = ptr(); a.Bm = ptr(); a.Cm = ptr();
            a.A = (const float *)ptr(); a.state = (float *)ptr(); a.y = ptr();
            if (!a.x || !a.state || a.dstate == 17 || a.batch <= 0)
                expect_status(selective_state_update(&a, st), "step");
        }
        {
            ssm_ssd_step_args a{};
            a.batch = pick(kSizes, kNS); a.nheads = pick(kSmall, kNM); a.headdim = pick(kSmall, kNM);
            a.dstate = pick(kSmall, kNM); a.ngroups = pick(kSmall, kNM); a.dtype = dtype();
            a.x = ptr(); a.dt = ptr(); a.A = (const float *)ptr(); a.Bm = ptr(); a.Cm = ptr();
            a.z = ptr(); a.state = (float *)ptr(); a.y = ptr();
            if (!a.x || !a.state || a.dstate == 17 || a.batch <= 0)
                expect_status(ssd_state_update(&a, st), "ssd step");
        }
        {
            ssm_conv_args a{};
            a.batch = pick(kSmall, kNM); a.seqlen = pick(kSizes, kNS); a.dim = pick(kSizes, kNS);
            a.width = pick(kSmall, kNM); a.dtype = dtype();
            a.x = ptr(); a.weight = (const float *)ptr(); a.bias = (const float *)ptr();
            a.init_state = ptr(); a.y = ptr(); a.final_state = ptr();
            if (!a.weight || a.width > 4 || a.batch <= 0) expect_status(causal_conv1d_fwd(&a, st), "conv");
        }
    }
    if (fails) {
        std::fprintf(stderr, "%d failures\n", fails);
        return 1;
    }
    std::printf("ABI sanitizer run: ok (%ld scan argument sets accepted)\n", accepted);
    return 0;
}
