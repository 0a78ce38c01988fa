// Drives the C ABI's host validation (kda_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with the kernel launchers replaced by counting
// stand-ins (launch_stubs.cpp).  Every rejected call must return its status
// without reaching a launcher; every accepted one must reach exactly one.
// Sizes include extremes so that the sizing arithmetic is exercised where it
// could overflow.  Exit status 0 when every expectation holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <limits>

#include "../../include/kda.h"

extern int g_launches;

static int failures = 0;

#define EXPECT(call, want, launches)                                                             \
    do {                                                                                         \
        const int before_ = g_launches;                                                          \
        const int got_ = (int)(call);                                                            \
        const int ran_ = g_launches - before_;                                                   \
        if (got_ != (int)(want) || ran_ != (launches)) {                                         \
            fprintf(stderr, "line %d: %s -> status %d (want %d), launches %d (want %d)\n",       \
                    __LINE__, #call, got_, (int)(want), ran_, (int)(launches));                  \
            ++failures;                                                                          \
        }                                                                                        \
    } while (0)

// A host buffer standing in for device memory; never read or written by the
// validation (the sanitizers would report it).
static void* buf(size_t n) {
    void* p = aligned_alloc(256, n < 256 ? 256 : (n + 255) / 256 * 256);
    if (!p) { fprintf(stderr, "out of host memory\n"); exit(2); }
    return p;
}

int main() {
    const float nan = std::numeric_limits<float>::quiet_NaN();
    const float inf = std::numeric_limits<float>::infinity();

    // ---- safe chunk size over the float line
    const float gs[] = {-5.f, -10.f, -1e-30f, -1e-45f, -3.4e38f, -0.f, 0.f, 1.f, nan, inf, -inf};
    const int want_gs[] = {16, 8, -2, -2, 0, -1, -1, -1, -1, -1, -1};
    for (size_t i = 0; i < sizeof(gs) / sizeof(gs[0]); ++i) {
        const int r = kda_safe_chunk_size(gs[i], KDA_BF16);
        if (want_gs[i] != -2 && r != want_gs[i]) {
            fprintf(stderr, "safe_chunk_size(%g) = %d, want %d\n", gs[i], r, want_gs[i]);
            ++failures;
        }
        if (want_gs[i] == -2 && r < 16) {  // tiny |g_min|: a huge (clamped) tile
            fprintf(stderr, "safe_chunk_size(%g) = %d, want >= 16\n", gs[i], r);
            ++failures;
        }
    }

    // ---- workspace sizing at extreme sizes: 0 or a value, never UB
    const int big[] = {0, 1, 4096, 1 << 20, 1 << 30, std::numeric_limits<int>::max()};
    for (int B : big)
        for (int T : big)
            for (int H : big) {
                (void)kda_chunk_fwd_workspace(B, T, H, 128, 128, 64, KDA_BF16);
                (void)kda_chunk_fwd_kernel_count(B, T, H, 128, 128, 32, KDA_F32);
                (void)kda_chunk_bwd_workspace(B, T, H, 128, 128);
                (void)kda_chunk_bwd_grouped_workspace(B, T, H, H, 128, 128, 1);
            }
    (void)kda_chunk_fwd_workspace(-1, 64, 1, 64, 64, 64, KDA_BF16);
    (void)kda_chunk_fwd_workspace(1, -1, 1, 64, 64, 64, KDA_BF16);

    // ---- kda_chunk_fwd
    const int B = 2, T = 100, H = 3, Dk = 64, Dv = 32, C = 32;
    const size_t rows = (size_t)B * T * H;
    void* q = buf(rows * Dk * 2); void* k = buf(rows * Dk * 2); void* v = buf(rows * Dv * 2);
    void* z = buf(rows * Dk * 2); void* br = buf(rows * 2); float* A = (float*)buf(H * 4);
    void* o = buf(rows * Dv * 2);
    float* S = (float*)buf((size_t)B * H * Dk * Dv * 4);
    const size_t wsn = kda_chunk_fwd_workspace(B, T, H, Dk, Dv, C, KDA_BF16);
    void* ws = buf(wsn);
    auto fwd = [&](const void* q_, void* o_, int T_, int chunk, float g_min, unsigned flags, int dt, void* ws_,
                   size_t wsb) {
        return kda_chunk_fwd(q_, k, v, z, br, A, nullptr, o_, S, nullptr, nullptr, B, T_, H, Dk, Dv, chunk, g_min,
                             flags, (kda_dtype)dt, ws_, wsb, nullptr);
    };
    EXPECT(fwd(q, o, T, C, -5.f, 7, 1, ws, wsn), KDA_OK, 1);
    EXPECT(fwd(q, o, T, C, -10.f, 7, 1, ws, wsn), KDA_OK, 1);       // strong gate: element-wise tiles
    EXPECT(fwd(q, o, T, C, nan, 7, 1, ws, wsn), KDA_ERR_GATE, 0);
    EXPECT(fwd(q, o, T, C, 0.f, 7, 1, ws, wsn), KDA_ERR_GATE, 0);
    EXPECT(fwd(q, o, T, C, nan, 15, 1, ws, wsn), KDA_OK, 1);       // v1 gate: g_min unused
    EXPECT(fwd(q, o, T, C, -5.f, 8, 1, ws, wsn), KDA_ERR_DTYPE, 0);
    EXPECT(fwd(q, o, T, C, -5.f, 16, 1, ws, wsn), KDA_ERR_DTYPE, 0);
    EXPECT(fwd(q, o, T, C, -5.f, 7, 2, ws, wsn), KDA_ERR_DTYPE, 0);
    EXPECT(fwd(q, o, T, 48, -5.f, 7, 1, ws, wsn), KDA_ERR_SHAPE, 0);
    EXPECT(fwd(q, o, -1, C, -5.f, 7, 1, ws, wsn), KDA_ERR_SHAPE, 0);
    EXPECT(fwd(nullptr, o, T, C, -5.f, 7, 1, ws, wsn), KDA_ERR_NULL, 0);
    EXPECT(fwd((const char*)q + 8, o, T, C, -5.f, 7, 1, ws, wsn), KDA_ERR_ALIGN, 0);
    EXPECT(fwd(q, nullptr, T, C, -5.f, 7, 1, ws, wsn), KDA_ERR_NULL, 0);
    EXPECT(fwd(q, o, T, C, -5.f, 7, 1, nullptr, wsn), KDA_ERR_WORKSPACE, 0);
    EXPECT(fwd(q, o, T, C, -5.f, 7, 1, ws, wsn - 1), KDA_ERR_WORKSPACE, 0);
    EXPECT(fwd(q, o, T, C, -5.f, 7, 1, (char*)ws + 16, wsn), KDA_ERR_WORKSPACE, 0);
    EXPECT(kda_chunk_fwd(q, k, v, z, br, A, nullptr, o, S, nullptr, nullptr, std::numeric_limits<int>::max(), T,
                         std::numeric_limits<int>::max(), Dk, Dv, C, -5.f, 7, KDA_BF16, ws, wsn, nullptr),
           KDA_ERR_SHAPE, 0);
    EXPECT(kda_chunk_fwd_timed(q, k, v, z, br, A, nullptr, o, S, nullptr, nullptr, B, T, H, Dk, Dv, C, -5.f, 7,
                               KDA_BF16, ws, wsn, nullptr, nullptr, 0),
           KDA_ERR_NULL, 0);
    // grouped heads: HV a multiple of H, a bias only with the in-kernel gate
    EXPECT(kda_chunk_fwd_grouped(q, k, v, z, br, A, A, nullptr, o, S, nullptr, nullptr, B, T, 1, H, Dk, Dv, C,
                                 -5.f, 3, KDA_BF16, ws, wsn, nullptr),
           KDA_ERR_DTYPE, 0);
    EXPECT(kda_chunk_fwd_grouped(q, k, v, z, br, A, nullptr, nullptr, o, S, nullptr, nullptr, B, T, 2, H, Dk, Dv,
                                 C, -5.f, 7, KDA_BF16, ws, wsn, nullptr),
           KDA_ERR_SHAPE, 0);

    // ---- the fused input-side convolution: taps required, all 16-byte aligned
    float* cw = (float*)buf((size_t)H * (2 * Dk + Dv) * 16);
    float* cb = (float*)buf((size_t)H * (2 * Dk + Dv) * 4);
    void* cs = buf((size_t)B * 3 * H * (2 * Dk + Dv) * 2);
    EXPECT(kda_chunk_fwd_conv(q, k, v, z, br, A, nullptr, cw, cb, cs, o, S, B, T, H, Dk, Dv, C, -5.f, 7, KDA_BF16,
                              ws, wsn, nullptr),
           KDA_OK, 1);
    EXPECT(kda_chunk_fwd_conv(q, k, v, z, br, A, nullptr, cw, nullptr, nullptr, o, S, B, T, H, Dk, Dv, C, -5.f, 7,
                              KDA_BF16, ws, wsn, nullptr),
           KDA_OK, 1);
    EXPECT(kda_chunk_fwd_conv(q, k, v, z, br, A, nullptr, nullptr, cb, cs, o, S, B, T, H, Dk, Dv, C, -5.f, 7,
                              KDA_BF16, ws, wsn, nullptr),
           KDA_ERR_NULL, 0);
    EXPECT(kda_chunk_fwd_conv(q, k, v, z, br, A, nullptr, cw + 1, cb, cs, o, S, B, T, H, Dk, Dv, C, -5.f, 7,
                              KDA_BF16, ws, wsn, nullptr),
           KDA_ERR_ALIGN, 0);
    EXPECT(kda_chunk_fwd_conv(q, k, v, z, br, A, nullptr, cw, cb + 1, cs, o, S, B, T, H, Dk, Dv, C, -5.f, 7,
                              KDA_BF16, ws, wsn, nullptr),
           KDA_ERR_ALIGN, 0);
    EXPECT(kda_chunk_fwd_conv(q, k, v, z, br, A, nullptr, cw, cb, (char*)cs + 2, o, S, B, T, H, Dk, Dv, C, -5.f, 7,
                              KDA_BF16, ws, wsn, nullptr),
           KDA_ERR_ALIGN, 0);

    // ---- the layer body with the fused output side: the gate required, y
    // apart from every input, the larger workspace
    {
        void* gate = buf(rows * Dv * 2);
        float* gw = (float*)buf(Dv * 4);
        void* y = buf(rows * Dv * 2);
        const size_t lwn = kda_layer_fwd_workspace(B, T, H, Dk, Dv, C, KDA_BF16);
        void* lws = buf(lwn);
        auto layer = [&](const void* gate_, const float* gw_, void* y_, const float* cw_, void* ws_, size_t wsb) {
            return kda_layer_fwd(q, k, v, z, br, A, nullptr, cw_, nullptr, nullptr, gate_, gw_, y_, S, B, T, H, Dk,
                                 Dv, C, -5.f, 7, KDA_BF16, ws_, wsb, nullptr);
        };
        EXPECT(layer(gate, gw, y, nullptr, lws, lwn), KDA_OK, 1);
        EXPECT(layer(gate, nullptr, y, cw, lws, lwn), KDA_OK, 1);
        EXPECT(layer(nullptr, gw, y, nullptr, lws, lwn), KDA_ERR_NULL, 0);
        EXPECT(layer((char*)gate + 2, gw, y, nullptr, lws, lwn), KDA_ERR_ALIGN, 0);
        EXPECT(layer(gate, gw + 1, y, nullptr, lws, lwn), KDA_ERR_ALIGN, 0);
        EXPECT(layer(gate, gw, gate, nullptr, lws, lwn), KDA_ERR_SHAPE, 0);
        EXPECT(layer(gate, gw, v, nullptr, lws, lwn), KDA_ERR_SHAPE, 0);
        EXPECT(layer(gate, gw, y, nullptr, lws, lwn - 1), KDA_ERR_WORKSPACE, 0);
        EXPECT(layer(gate, gw, y, nullptr, lws, wsn), wsn < lwn ? KDA_ERR_WORKSPACE : KDA_OK, wsn < lwn ? 0 : 1);
        EXPECT(kda_layer_fwd(q, k, v, z, br, A, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, y, S, B, 0, H,
                             Dk, Dv, C, -5.f, 7, KDA_BF16, lws, lwn, nullptr),
               KDA_OK, 1);
        free(gate); free(gw); free(y); free(lws);
    }

    // ---- the allocation-free entry point: its own size limit, no workspace
    EXPECT(kda_chunk_fwd_noalloc(q, k, v, z, br, A, nullptr, o, S, nullptr, nullptr, B, T, H, Dk, Dv, C, -5.f, 7,
                                 KDA_BF16, nullptr),
           KDA_OK, 1);
    EXPECT(kda_chunk_fwd_noalloc(q, k, v, z, br, A, nullptr, o, S, nullptr, nullptr, 1, T, 421, 128, 128, 32, -5.f, 7,
                                 KDA_BF16, nullptr),
           KDA_OK, 1);
    EXPECT(kda_chunk_fwd_noalloc(q, k, v, z, br, A, nullptr, o, S, nullptr, nullptr, 1, T, 422, 128, 128, 32, -5.f, 7,
                                 KDA_BF16, nullptr),
           KDA_ERR_SCRATCH, 0);
    EXPECT(kda_chunk_fwd_noalloc(nullptr, k, v, z, br, A, nullptr, o, S, nullptr, nullptr, B, T, H, Dk, Dv, C, -5.f,
                                 7, KDA_BF16, nullptr),
           KDA_ERR_NULL, 0);

    // ---- kda_step
    EXPECT(kda_step(q, k, v, z, br, A, S, o, B, H, Dk, Dv, -5.f, 7, KDA_BF16, nullptr), KDA_OK, 1);
    EXPECT(kda_step(q, k, v, z, br, A, nullptr, o, B, H, Dk, Dv, -5.f, 7, KDA_BF16, nullptr), KDA_ERR_NULL, 0);
    EXPECT(kda_step(q, k, v, z, br, nullptr, S, o, B, H, Dk, Dv, -5.f, 7, KDA_BF16, nullptr), KDA_ERR_NULL, 0);
    EXPECT(kda_step(q, k, v, z, br, nullptr, S, o, B, H, Dk, Dv, -5.f, 3, KDA_BF16, nullptr), KDA_OK, 1);
    EXPECT(kda_step(q, k, v, z, br, A, S, o, B, H, Dk, 48, -5.f, 7, KDA_BF16, nullptr), KDA_ERR_SHAPE, 0);
    EXPECT(kda_step_grouped(q, k, v, z, br, A, nullptr, S, o, B, 2, 3, Dk, Dv, -5.f, 7, KDA_BF16, nullptr),
           KDA_ERR_SHAPE, 0);

    // ---- kda_segment_compose: S_prefix may not overlap its inputs
    const int ns = 3;
    float* M = (float*)buf((size_t)ns * B * H * Dk * Dk * 4);
    float* St = (float*)buf((size_t)ns * B * H * Dk * Dv * 4);
    float* Sp = (float*)buf((size_t)ns * B * H * Dk * Dv * 4);
    EXPECT(kda_segment_compose(ns, M, St, S, Sp, B, H, Dk, Dv, nullptr), KDA_OK, 1);
    EXPECT(kda_segment_compose(ns, M, St, S, St, B, H, Dk, Dv, nullptr), KDA_ERR_SHAPE, 0);
    EXPECT(kda_segment_compose(ns, M, St, Sp + 64, Sp, B, H, Dk, Dv, nullptr), KDA_ERR_SHAPE, 0);
    EXPECT(kda_segment_compose(ns, M, St, nullptr, M + 64, B, H, Dk, Dv, nullptr), KDA_ERR_SHAPE, 0);
    EXPECT(kda_segment_compose(-1, M, St, S, Sp, B, H, Dk, Dv, nullptr), KDA_ERR_SHAPE, 0);

    // ---- kda_segment_fixup
    void* P = buf(rows * Dk * 2);
    EXPECT(kda_segment_fixup(1, P, S, nullptr, o, B, T, H, Dk, Dv, KDA_BF16, nullptr), KDA_OK, 1);
    EXPECT(kda_segment_fixup(2, P, S, nullptr, o, 1, T, H, Dk, Dv, KDA_BF16, nullptr), KDA_ERR_NULL, 0);

    // ---- kda_short_conv and kda_output_gate
    const int Cc = H * Dk;
    float* w = (float*)buf((size_t)Cc * 16);
    void* x = buf((size_t)B * T * Cc * 2); void* y = buf((size_t)B * T * Cc * 2);
    void* win = buf((size_t)B * 3 * Cc * 2);
    EXPECT(kda_short_conv(x, w, nullptr, nullptr, win, y, B, T, Cc, 1, KDA_BF16, nullptr), KDA_OK, 1);
    EXPECT(kda_short_conv(x, w, nullptr, nullptr, win, x, B, T, Cc, 1, KDA_BF16, nullptr), KDA_ERR_SHAPE, 0);
    EXPECT(kda_short_conv(x, w, nullptr, win, win, y, B, T, Cc, 1, KDA_BF16, nullptr), KDA_ERR_SHAPE, 0);
    EXPECT(kda_short_conv(x, w, nullptr, win, win, y, B, 8, Cc, 1, KDA_BF16, nullptr), KDA_OK, 1);
    EXPECT(kda_short_conv(x, w, nullptr, nullptr, nullptr, y, B, T, Cc + 4, 1, KDA_BF16, nullptr), KDA_ERR_SHAPE, 0);
    EXPECT(kda_output_gate(o, v, nullptr, o, B, T, H, Dv, KDA_BF16, nullptr), KDA_OK, 1);
    EXPECT(kda_output_gate(o, v, nullptr, (char*)o + 64, B, T, H, Dv, KDA_BF16, nullptr), KDA_ERR_SHAPE, 0);

    // ---- kda_chunk_bwd: outputs overlap nothing
    const size_t bwn = kda_chunk_bwd_workspace(B, T, H, Dk, Dv);
    void* bws = buf(bwn);
    void* dq = buf(rows * Dk * 2); void* dk = buf(rows * Dk * 2); void* dv = buf(rows * Dv * 2);
    void* dz = buf(rows * Dk * 2); void* db = buf(rows * 2); float* dA = (float*)buf(H * 4);
    float* dS0 = (float*)buf((size_t)B * H * Dk * Dv * 4);
    void* dout = buf(rows * Dv * 2);
    auto bwd = [&](void* dq_, void* dv_, float* dS0_, float g_min, void* ws_, size_t wsb) {
        return kda_chunk_bwd(q, k, v, z, br, A, S, dout, nullptr, dq_, dk, dv_, dz, db, dA, dS0_, B, T, H, Dk, Dv,
                             g_min, 7, KDA_BF16, ws_, wsb, nullptr);
    };
    EXPECT(bwd(dq, dv, dS0, -5.f, bws, bwn), KDA_OK, 1);
    EXPECT(bwd(dq, dv, dS0, -10.f, bws, bwn), KDA_OK, 1);
    EXPECT(bwd(q, dv, dS0, -5.f, bws, bwn), KDA_ERR_SHAPE, 0);
    EXPECT(bwd(dq, dout, dS0, -5.f, bws, bwn), KDA_ERR_SHAPE, 0);
    EXPECT(bwd(dq, dv, S, -5.f, bws, bwn), KDA_ERR_SHAPE, 0);
    EXPECT(bwd(dq, dq, dS0, -5.f, bws, bwn), KDA_ERR_SHAPE, 0);
    EXPECT(bwd(dq, dv, (float*)bws, -5.f, bws, bwn), KDA_ERR_SHAPE, 0);
    EXPECT(bwd(dq, dv, dS0, -5.f, bws, bwn - 1), KDA_ERR_WORKSPACE, 0);

    for (int s = 0; s <= 8; ++s)  // every status has a description
        if (!kda_status_string((kda_status)s)) { fprintf(stderr, "status %d has no string\n", s); ++failures; }

    if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
    else printf("validation driver: all expectations hold\n");
    return failures ? 1 : 0;
}
