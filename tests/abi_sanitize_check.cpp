// abi_sanitize_check.cpp -- drives the host side of the C ABI (include/dtree.h)
// through every path that needs no GPU: handle creation with valid and
// invalid configurations, workspace sizes, error strings, timing argument
// checks, argument validation of every enqueueing entry point (null and
// misaligned pointers, missing or short workspace) and the B = 0 no-ops.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// code by tests/test_sanitizers.py, so that an out-of-bounds access, leak or
// undefined operation in these paths is reported.  No call below reaches the
// HIP runtime: validation fails, or B = 0, before anything is enqueued.
// Exit status 0 = every check passed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dtree.h"

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

static dt_config cfg(int B, int L, int V, int E, int H, int M, int n, dt_dtype dt = DT_BF16) {
    dt_config c;
    memset(&c, 0, sizeof c);
    c.B = B; c.L = L; c.V = V; c.E = E; c.H = H; c.M = M; c.n = n;
    c.temperature = 0.f;
    c.dtype = dt;
    c.near_tie_eps = 1e-5f;
    c.full_vocab = 0;
    return c;
}

int main() {
    // creation: the limits, and configurations each limit rejects
    const dt_config good[] = {cfg(2, 4, 100, 32, 32, 8, 6), cfg(1, 64, 1000, 32, 32, 32, 32),
                              cfg(1, 4, 1000, 32, 32, 64, 64), cfg(3, 4, 100, 32, 4096, 8, 6),
                              cfg(0, 4, 100, 32, 32, 8, 6), cfg(5, 3, 37, 8, 12, 37, 9, DT_F32)};
    for (const dt_config& c : good) {
        dt_handle* h = nullptr;
        CHECK(dt_create(&c, &h) == DT_OK && h != nullptr);
        CHECK(c.B == 0 ? true : dt_workspace_bytes(h) > 0);
        dt_destroy(h);
    }
    dt_config bad[] = {cfg(2, 0, 100, 32, 32, 8, 6), cfg(2, 4, 0, 32, 32, 8, 6), cfg(2, 4, 100, 32, 32, 0, 6),
                       cfg(2, 4, 100, 32, 32, 8, 0), cfg(-1, 4, 100, 32, 32, 8, 6), cfg(2, 4, 100, 32, 32, 101, 6),
                       cfg(2, 4, 1000, 32, 32, 65, 6), cfg(2, 4, 100, 32, 32, 8, 65), cfg(2, 65, 100, 32, 32, 8, 6),
                       cfg(2, 4, 100, 48, 32, 8, 6), cfg(2, 4, 100, 32, 8192, 8, 6), cfg(1, 64, 1000, 32, 32, 64, 64),
                       cfg(2, 4, 100, 6, 32, 8, 6, DT_F32)};
    bad[0].temperature = -1.f;
    for (const dt_config& c : bad) {
        dt_handle* h = (dt_handle*)&failures;  // overwritten with NULL on failure
        CHECK(dt_create(&c, &h) != DT_OK && h == nullptr);
        CHECK(strlen(dt_last_error(nullptr)) > 0);
    }
    {
        dt_config c = cfg(2, 4, 100, 32, 32, 8, 6);
        c.dtype = (dt_dtype)7;
        dt_handle* h = nullptr;
        CHECK(dt_create(&c, &h) == DT_ERR_INVALID_ARG);
        c = cfg(2, 4, 100, 32, 32, 8, 6);
        c.full_vocab = 2;
        CHECK(dt_create(&c, &h) == DT_ERR_INVALID_ARG);
        CHECK(dt_create(nullptr, &h) == DT_ERR_INVALID_ARG);
        CHECK(dt_create(&c, nullptr) == DT_ERR_INVALID_ARG);
    }
    for (int s = 0; s >= -5; --s) CHECK(dt_status_string((dt_status)s) != nullptr);
    dt_destroy(nullptr);

    // argument validation of the enqueueing entry points: fake addresses are
    // never dereferenced, every call below fails before any HIP call
    const dt_config c = cfg(2, 4, 100, 32, 32, 8, 6);
    dt_handle* h = nullptr;
    CHECK(dt_create(&c, &h) == DT_OK);
    const size_t need = dt_workspace_bytes(h);
    void* fake = (void*)0x10000;
    void* odd = (void*)0x10004;
    int32_t* fi = (int32_t*)fake;
    float* ff = (float*)fake;
    uint8_t* fu8 = (uint8_t*)fake;
    uint32_t* fu32 = (uint32_t*)fake;
    CHECK(dt_build(h, fake, need, fake, fake, fake, fake, nullptr, nullptr, nullptr, nullptr, fi, fi, fi, ff, fu8,
                   fi, fu32, nullptr) == DT_ERR_INVALID_ARG);  // C missing
    CHECK(strstr(dt_last_error(h), "null") != nullptr);
    CHECK(dt_build(h, fake, need, fake, odd, fake, fake, nullptr, nullptr, fake, nullptr, fi, fi, fi, ff, fu8, fi,
                   fu32, nullptr) == DT_ERR_INVALID_ARG);  // misaligned embedding
    CHECK(dt_build(h, nullptr, need, fake, fake, fake, fake, nullptr, nullptr, fake, nullptr, fi, fi, fi, ff, fu8,
                   fi, fu32, nullptr) == DT_ERR_WORKSPACE);
    CHECK(dt_build(h, fake, need - 1, fake, fake, fake, fake, nullptr, nullptr, fake, nullptr, fi, fi, fi, ff, fu8,
                   fi, fu32, nullptr) == DT_ERR_WORKSPACE);
    CHECK(dt_build(h, (char*)fake + 16, need, fake, fake, fake, fake, nullptr, nullptr, fake, nullptr, fi, fi, fi,
                   ff, fu8, fi, fu32, nullptr) == DT_ERR_WORKSPACE);  // workspace alignment
    CHECK(dt_build_noalloc(h, nullptr, fake, fake, fake, nullptr, nullptr, fake, nullptr, fi, fi, fi, ff, fu8, fi,
                           fu32, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_build_noalloc(h, fake, fake, fake, fake, nullptr, nullptr, fake, (const float*)odd, fi, fi, fi, ff, fu8,
                           fi, fu32, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_build_marginal(h, fake, need, nullptr, fi, fi, fi, ff, fu8, fi, fu32, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_build_marginal(h, fake, need, odd, fi, fi, fi, ff, fu8, fi, fu32, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_build_folded(h, fake, need, fake, nullptr, fake, nullptr, fake, nullptr, fi, fi, fi, ff, fu8, fi, fu32,
                          nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_build_folded(h, nullptr, need, fake, ff, fake, nullptr, fake, nullptr, fi, fi, fi, ff, fu8, fi, fu32,
                          nullptr) == DT_ERR_WORKSPACE);
    CHECK(dt_fold_input(h, nullptr, fake, nullptr, ff, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_fold_input(h, fake, fake, nullptr, (float*)odd, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_topm(h, fake, need, nullptr, fi, ff, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_topm(h, nullptr, need, fake, fi, ff, nullptr) == DT_ERR_WORKSPACE);
    CHECK(dt_topm_tail(h, fake, need, fake, fi, ff, nullptr, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_gru_step(h, fake, need, fake, ff, fake, fake, nullptr, nullptr, nullptr, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_gru_step(h, fake, need, fake, ff, fake, fake, nullptr, nullptr, ff, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_correct(h, fi, ff, fake, (const float*)odd, fi, fi, ff, nullptr) == DT_ERR_INVALID_ARG);
    CHECK(dt_correct(h, nullptr, ff, fake, ff, fi, fi, ff, nullptr) == DT_ERR_INVALID_ARG);
    for (int i = 0; i < 7; ++i) {
        int32_t* a[7] = {fi, fi, fi, fi, fi, fi, fi};
        a[i] = nullptr;
        CHECK(dt_accept_greedy(h, a[0], a[1], a[2], a[3], a[4], a[5], a[6], nullptr) == DT_ERR_INVALID_ARG);
    }
    CHECK(dt_accept_greedy(nullptr, fi, fi, fi, fi, fi, fi, fi, nullptr) == DT_ERR_INVALID_ARG);
    // timing argument checks (no event is created at level 0)
    CHECK(dt_timing_enable(h, 3, 10) == DT_ERR_INVALID_ARG);
    CHECK(dt_timing_enable(h, 1, -1) == DT_ERR_INVALID_ARG);
    CHECK(dt_timing_enable(h, 0, 0) == DT_OK);
    int nout = -1;
    float ms[4];
    CHECK(dt_timing_read(h, 9, ms, 4, &nout) == DT_ERR_INVALID_ARG);
    CHECK(dt_timing_read(h, 0, nullptr, 4, &nout) == DT_ERR_INVALID_ARG);
    CHECK(dt_timing_read(h, 0, ms, 4, &nout) == DT_OK && nout == 0);
    CHECK(dt_timing_read(h, 4, nullptr, 0, &nout) == DT_OK && nout == 0);
    dt_destroy(h);

    // dt_build_noalloc: a configuration whose scratch exceeds the static
    // array is rejected before any HIP call
    const dt_config big = cfg(256, 16, 151936, 2560, 1024, 64, 64);
    CHECK(dt_create(&big, &h) == DT_OK);
    CHECK(dt_build_noalloc(h, fake, fake, fake, fake, nullptr, nullptr, fake, nullptr, fi, fi, fi, ff, fu8, fi, fu32,
                           nullptr) == DT_ERR_UNSUPPORTED);
    CHECK(strstr(dt_last_error(h), "scratch") != nullptr);
    dt_destroy(h);

    // B = 0: nothing to enqueue, every pointer may be NULL
    const dt_config z = cfg(0, 4, 100, 32, 32, 8, 6);
    CHECK(dt_create(&z, &h) == DT_OK);
    CHECK(dt_build(h, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DT_OK);
    CHECK(dt_build_marginal(h, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr) == DT_OK);
    CHECK(dt_build_noalloc(h, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DT_OK);
    CHECK(dt_topm(h, nullptr, 0, nullptr, nullptr, nullptr, nullptr) == DT_OK);
    CHECK(dt_topm_tail(h, nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr) == DT_OK);
    CHECK(dt_accept_greedy(h, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DT_OK);
    CHECK(dt_build_folded(h, nullptr, 0, nullptr, ff, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, nullptr, nullptr, nullptr) == DT_OK);
    dt_destroy(h);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ABI sanitizer check: every host path ran clean\n");
    return 0;
}
