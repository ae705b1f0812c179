// Host-side checks of the C ABI's argument validation, run under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only) on a machine without a GPU. Every call below
// is rejected before any HIP call: the status must be an error and the per-thread message
// must be set. The size queries run over a grid of sizes, up to the documented caps.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "dspark.h"

static int failures = 0;

static void expect_error(int status, const char* what) {
    const char* msg = dspark_last_error();
    if (status == DSPARK_OK || msg == nullptr || std::strlen(msg) == 0) {
        std::printf("FAIL %s: status %d message '%s'\n", what, status, msg ? msg : "(null)");
        ++failures;
    }
    (void)dspark_status_string(status);
}

int main() {
    void* fake = reinterpret_cast<void*>(0x1000);
    void* odd = reinterpret_cast<void*>(0x1004);
    const float* ff = static_cast<const float*>(fake);
    const int32_t* fi = static_cast<const int32_t*>(fake);
    float* wf = static_cast<float*>(fake);
    int32_t* wi = static_cast<int32_t*>(fake);

    for (int s = -2; s < 12; ++s) (void)dspark_status_string(s);
    if (dspark_version() <= 0) { std::printf("FAIL version\n"); ++failures; }

    // size queries over a grid of sizes (overflow-free arithmetic up to the caps)
    const int Bs[] = {1, 7, 512, 4096, 1 << 16, 1 << 24};
    const int Vs[] = {1, 8, 129280, 151936, 1 << 20};
    const int Gs[] = {1, 16, 64};
    for (int B : Bs)
        for (int V : Vs)
            for (int G : Gs) {
                (void)dspark_markov_draft_workspace_bytes(B, V, 256, G);
                (void)dspark_verify_workspace_bytes(B, V, G);
                (void)dspark_tv_labels_workspace_bytes(B, V, G);
                (void)dspark_verify_tv_workspace_bytes(B, V, G);
                (void)dspark_verify_markov_workspace_bytes(B, V, 256, G);
            }
    for (int R : {1, 64, 512, 16384})
        for (int G : {1, 16, 64}) {
            (void)dspark_schedule_workspace_bytes(R, G, 1 << 20);
            (void)dspark_conf_ring_bytes(R, G);
            (void)dspark_sts_fit_workspace_bytes(R, G, 64);
        }

    // draft
    expect_error(dspark_markov_draft(0, 8, 4, 2, ff, fake, fake, 0, fi, ff, wi, nullptr, nullptr,
                                     nullptr, fake, 1 << 30, nullptr), "draft B=0");
    expect_error(dspark_markov_draft(2, 8, 4, 65, ff, fake, fake, 0, fi, ff, wi, nullptr, nullptr,
                                     nullptr, fake, 1 << 30, nullptr), "draft gamma cap");
    expect_error(dspark_markov_draft(2, 8, 4, 2, ff, fake, fake, 7, fi, ff, wi, nullptr, nullptr,
                                     nullptr, fake, 1 << 30, nullptr), "draft dtype");
    expect_error(dspark_markov_draft(2, 8, 4, 2, nullptr, fake, fake, 0, fi, ff, wi, nullptr,
                                     nullptr, nullptr, fake, 1 << 30, nullptr), "draft U null");
    expect_error(dspark_markov_draft(2, 8, 4, 2, ff, fake, fake, 0, fi, ff, wi, nullptr, nullptr,
                                     nullptr, fake, 8, nullptr), "draft workspace");
    expect_error(dspark_markov_draft_ex(2, 8, 4, 2, ff, fake, fake, 0, fi, ff, wi, nullptr, nullptr,
                                        nullptr, fake, 1 << 30, nullptr, 6), "draft option bits");
    expect_error(dspark_markov_draft_ex(2, 8, 4, 2, ff, fake, fake, 0, fi, ff, wi, nullptr, nullptr,
                                        nullptr, fake, 8, nullptr, DSPARK_DRAFT_PER_POSITION),
                 "draft_ex workspace");
    // verify, TV, fused
    expect_error(dspark_verify(0, 8, 2, ff, ff, 6, nullptr, nullptr, fi, nullptr, ff, ff, wi, wi,
                               nullptr, nullptr, fake, 1 << 30, nullptr), "verify B=0");
    expect_error(dspark_verify(2, 8, 2, nullptr, ff, 6, nullptr, nullptr, fi, nullptr, ff, ff, wi,
                               wi, nullptr, nullptr, fake, 1 << 30, nullptr), "verify Ld null");
    expect_error(dspark_verify(2, 8, 2, ff, ff, 6, nullptr, nullptr, fi, nullptr, ff, ff, wi, wi,
                               nullptr, nullptr, fake, 4, nullptr), "verify workspace");
    expect_error(dspark_tv_labels(2, 8, 2, nullptr, ff, 6, nullptr, nullptr, nullptr, nullptr, wf,
                                  fake, 1 << 30, nullptr), "tv Ld null");
    expect_error(dspark_verify_tv(2, 0, 2, ff, ff, 6, nullptr, nullptr, fi, nullptr, ff, ff, wi, wi,
                                  nullptr, nullptr, wf, fake, 1 << 30, nullptr), "verify_tv V=0");
    expect_error(dspark_verify_markov(2, 8, 8, 2, ff, fake, fake, 0, fi, fi, ff, ff, 6, nullptr,
                                      nullptr, ff, ff, wi, wi, wf, wf, fake, 1 << 30, nullptr),
                 "verify_markov fp32 factors");
    expect_error(dspark_verify_markov(2, 8, 8, 2, ff, fake, fake, 1, fi, fi, nullptr, ff, 6,
                                      nullptr, nullptr, ff, ff, wi, wi, wf, wf, fake, 1 << 30,
                                      nullptr), "verify_markov ld_lse null");
    // schedule and the lag ring
    expect_error(dspark_schedule(0, 4, ff, nullptr, ff, 40, 0, wi, nullptr, nullptr, nullptr,
                                 nullptr, fake, 1 << 30, nullptr), "schedule R=0");
    expect_error(dspark_schedule(8, 4, ff, nullptr, ff, 7, 0, wi, nullptr, nullptr, nullptr,
                                 nullptr, fake, 1 << 30, nullptr), "schedule Bmax < R");
    expect_error(dspark_schedule(8, 4, ff, nullptr, ff, 40, 9, wi, nullptr, nullptr, nullptr,
                                 nullptr, fake, 1 << 30, nullptr), "schedule mode");
    const size_t rb = dspark_conf_ring_bytes(4, 4);
    expect_error(dspark_conf_ring_init(4, 4, nullptr, rb, nullptr), "ring init null");
    expect_error(dspark_conf_ring_init(4, 4, odd, rb, nullptr), "ring init misaligned");
    expect_error(dspark_conf_ring_push(4, 4, fake, rb - 1, ff, nullptr), "ring push small");
    expect_error(dspark_conf_ring_push(4, 4, fake, rb, nullptr, nullptr), "ring push conf null");
    expect_error(dspark_schedule_lagged(4, 4, fake, rb, nullptr, ff, 3, 0, wi, nullptr, nullptr,
                                        nullptr, nullptr, fake, 1 << 30, nullptr), "lagged Bmax");
    // STS
    expect_error(dspark_sts_fit(0, 4, ff, fi, nullptr, ff, 8, 15, 0, wf, wf, wf, nullptr, fake,
                                1 << 30, nullptr), "sts N=0");
    expect_error(dspark_sts_fit(16, 4, ff, fi, nullptr, ff, 8, 17, 0, wf, wf, wf, nullptr, fake,
                                1 << 30, nullptr), "sts bins cap");
    std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
