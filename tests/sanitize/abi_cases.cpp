// Driver for the sanitizer build of the C entry points' host code
// (gated_causal_attention_amd/csrc/resolvent_abi.cpp), test infrastructure.
// The kernel launchers are replaced by the stubs below, which check that each
// launch they receive carries a workspace layout that fits the workspace the
// caller passed and count the launches; nothing touches a device.  Every entry
// point is called with valid arguments and with each class of invalid one
// (negative and empty shapes, unsupported sizes and dtypes, null and misaligned
// pointers, short workspaces, non-finite switches, an overflowing logit
// scale).  Built with -fsanitize=address,undefined; any report, a wrong status
// or a launch that should not have happened fails the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "layout.h"
#include "resolvent.h"

namespace resolvent {
static int launches = 0;
static size_t ws_given = 0;
static void took(size_t need) {
    ++launches;
    if (need > ws_given) {
        std::printf("launch with a workspace layout of %zu bytes > %zu given\n", need, ws_given);
        std::exit(3);
    }
}
int launch_gates(const Layout &L, const float *, const float *, double, unsigned char *,
                 int32_t *, void *, int64_t) {
    took(L.total);
    return 0;
}
int launch_chain(const ChainLayout &C, const float *, const float *, const void *, bool, double,
                 float *, float *, unsigned char *, int32_t *, void *) {
    took(C.total);
    return 0;
}
int launch_decode(const DecodeLayout &DL, const void *, const void *, const float *,
                  const float *, const void *, int64_t, bool, bool, double, float, float, int,
                  bool, float *, float *, unsigned char *, int32_t *, void *) {
    took(DL.total);
    return 0;
}
int launch_path_product(const double *, const double *, int64_t, int64_t, double *, double *,
                        void *) {
    took(0);
    return 0;
}
int launch_operator(const OperatorLayout &OL, const void *, const void *, const float *,
                    const float *, bool, double, float, float, int, bool, float *, float *,
                    unsigned char *, int32_t *, void *) {
    took(OL.total);
    return 0;
}
int launch_chain_step(float *, float *, const float *, const float *, const void *, bool, double,
                      int64_t, int64_t, int32_t *, void *) {
    took(0);
    return 0;
}
int launch_forward(const Problem &P, void *, void *const *) {
    took(P.L.total);
    return 0;
}
}  // namespace resolvent

static int failures = 0;
static void expect(int32_t got, int32_t want, int launched, const char *what) {
    const int did = resolvent::launches;
    resolvent::launches = 0;
    if (got != want || did != launched) {
        std::printf("%s: status %d (want %d), launches %d (want %d)\n", what, got, want, did,
                    launched);
        ++failures;
    }
}

int main() {
    using resolvent::ws_given;
    // one 256-byte aligned arena stands in for every device buffer: the stubs
    // never dereference it
    std::vector<unsigned char> arena(1 << 20);
    unsigned char *base = arena.data() + (256 - reinterpret_cast<uintptr_t>(arena.data()) % 256);
    void *p = base;
    float *f = reinterpret_cast<float *>(base);
    int32_t *st = reinterpret_cast<int32_t *>(base);
    void *odd = base + 2;
    hipStream_t s = nullptr;
    const double inf = INFINITY, nan = NAN;

    for (int32_t qdt : {RESOLVENT_BF16, RESOLVENT_F32})
        for (int64_t d : {64, 128})
            for (int64_t n : {1, 255, 256, 257, 8192}) {
                const int32_t vdt = RESOLVENT_F32;
                const size_t need = resolvent_workspace_bytes(2, 3, n, d, qdt, vdt);
                if (need == 0) { std::printf("no workspace size for n=%lld\n", (long long)n); ++failures; }
                ws_given = need;
                expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 2, 3, n, d, qdt, vdt, f, f, p, need,
                                         st, s), RESOLVENT_OK, 1, "forward");
                expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 2, 3, n, d, qdt, vdt, f, f, p,
                                         need - 1, st, s), RESOLVENT_BAD_ARG, 0, "short workspace");
                expect(resolvent_forward(p, p, f, f, p, nan, 1, 1, 2, 3, n, d, qdt, vdt, f, f, p,
                                         need, st, s), RESOLVENT_NONFINITE, 0, "nan beta");
                expect(resolvent_forward(p, p, f, f, p, 1, 1e300, 1, 2, 3, n, d, qdt, vdt, f, f, p,
                                         need, st, s), RESOLVENT_NONFINITE, 0, "overflowing scale");
                expect(resolvent_forward(odd, p, f, f, p, 1, 1, 1, 2, 3, n, d, qdt, vdt, f, f, p,
                                         need, st, s), RESOLVENT_BAD_ARG, 0, "misaligned q");
                expect(resolvent_forward(p, nullptr, f, f, p, 1, 1, 1, 2, 3, n, d, qdt, vdt, f, f,
                                         p, need, st, s), RESOLVENT_BAD_ARG, 0, "null k");
                const size_t gneed =
                    resolvent_workspace_bytes_grouped(2, 4, 2, n, d, 64, qdt, vdt);
                ws_given = gneed;
                expect(resolvent_forward_grouped(p, p, f, f, p, 0.5, 0.7, 0.5, 2, 4, 2, n, d, 64,
                                                 qdt, vdt, f, f, p, gneed, st, s),
                       RESOLVENT_OK, 1, "grouped");
                expect(resolvent_forward_grouped(p, p, f, f, p, 1, 1, 1, 2, 4, 3, n, d, 64, qdt,
                                                 vdt, f, f, p, gneed, st, s),
                       RESOLVENT_BAD_SHAPE, 0, "heads not a multiple of k/v heads");
                const size_t dneed = resolvent_decode_workspace_bytes(2, 4, 2, n, d, d, qdt, vdt);
                ws_given = dneed;
                expect(resolvent_decode(p, p, f, f, p, 1, 1, 1, 2, 4, 2, n, n + 5, d, d, qdt, vdt,
                                        f, f, p, dneed, st, s), RESOLVENT_OK, 1, "decode");
                expect(resolvent_decode(p, p, f, f, p, 1, 1, 1, 2, 4, 2, n, n - 1, d, d, qdt, vdt,
                                        f, f, p, dneed, st, s), RESOLVENT_BAD_SHAPE, 0,
                       "cache smaller than n");
                if (n <= 4096) {
                    const size_t oneed = resolvent_operator_workspace_bytes(1, 2, n, d, qdt);
                    ws_given = oneed;
                    expect(resolvent_operator(p, p, f, f, 0, 1, 0.3, 1, 2, n, d, qdt, f, f, p,
                                              oneed, st, s), RESOLVENT_OK, 1, "operator");
                    expect(resolvent_operator(p, p, f, f, inf, 1, 0.3, 1, 2, n, d, qdt, f, f, p,
                                              oneed, st, s), RESOLVENT_NONFINITE, 0,
                           "operator inf beta");
                }
            }
    ws_given = 0;
    expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 0, 3, 100, 64, RESOLVENT_BF16, RESOLVENT_BF16,
                             f, f, nullptr, 0, st, s), RESOLVENT_OK, 0, "empty batch");
    expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 1, 3, 100, 0, RESOLVENT_BF16, RESOLVENT_BF16,
                             f, f, p, 0, st, s), RESOLVENT_BAD_SHAPE, 0, "head_dim 0");
    expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 1, 3, 100, 96, RESOLVENT_BF16, RESOLVENT_BF16,
                             f, f, p, 1 << 20, st, s), RESOLVENT_UNSUPPORTED, 0, "head_dim 96");
    expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 1, 3, -1, 64, RESOLVENT_BF16, RESOLVENT_BF16,
                             f, f, p, 1 << 20, st, s), RESOLVENT_BAD_SHAPE, 0, "negative n");
    expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 1, 1, (int64_t(1) << 22) + 1, 64,
                             RESOLVENT_BF16, RESOLVENT_BF16, f, f, p, 1 << 20, st, s),
           RESOLVENT_UNSUPPORTED, 0, "sequence too long");
    expect(resolvent_forward(p, p, f, f, p, 1, 1, 1, 1, 1, 100, 64, RESOLVENT_F32, RESOLVENT_BF16,
                             f, f, p, 1 << 20, st, s), RESOLVENT_UNSUPPORTED, 0, "fp32 q with bf16 v");
    {
        const size_t cneed = resolvent_chain_workspace_bytes(2, 3, 1000, 128);
        ws_given = cneed;
        expect(resolvent_chain(f, f, p, 1, 2, 3, 1000, 128, RESOLVENT_BF16, f, f, p, cneed, st, s),
               RESOLVENT_OK, 1, "chain");
        expect(resolvent_chain(f, f, p, nan, 2, 3, 1000, 128, RESOLVENT_BF16, f, f, p, cneed, st,
                               s), RESOLVENT_NONFINITE, 0, "chain nan g");
        expect(resolvent_chain(f, f, p, 1, 2, 3, 1000, 100, RESOLVENT_BF16, f, f, p, cneed, st, s),
               RESOLVENT_UNSUPPORTED, 0, "chain width not a multiple of 64");
        expect(resolvent_chain_step(f, f, f, f, p, 0.5, 2, 3, 128, RESOLVENT_F32, st, s),
               RESOLVENT_OK, 1, "chain step");
        expect(resolvent_chain_step(f, f, f, f, odd, 0.5, 2, 3, 128, RESOLVENT_F32, st, s),
               RESOLVENT_BAD_ARG, 0, "chain step misaligned v");
    }
    expect(resolvent_path_product(reinterpret_cast<double *>(base), reinterpret_cast<double *>(base),
                                  3, 100, reinterpret_cast<double *>(base),
                                  reinterpret_cast<double *>(base), s), RESOLVENT_OK, 1,
           "path product");
    expect(resolvent_path_product(nullptr, nullptr, 3, 100, nullptr, nullptr, s),
           RESOLVENT_BAD_ARG, 0, "path product null");
    int32_t bq = 0, bk = 0;
    resolvent_tile_shape(&bq, &bk);
    for (int32_t code = -1; code <= 6; ++code)
        if (resolvent_status_str(code) == nullptr) ++failures;
    std::printf("abi cases done (tile %d x %d), %d failures\n", bq, bk, failures);
    return failures != 0;
}
