// Host check of the fused kernel's direct global->LDS copies: every 16-byte
// source range that a workgroup can ask for lies inside its tensor.  It walks
// every key tile of every shape given on the command line (all tiles a
// workgroup of any query tile stages, the logit check included), every row
// and every 16-byte chunk, using the same helpers as the kernel.
#include <cstdio>
#include <cstdlib>

#include "layout.h"

using namespace resolvent;

static int check(int64_t B, int64_t H, int64_t n, int64_t d, int esz, bool bf16_path) {
    const Layout L = make_layout(B, H, n, d, bf16_path);
    const int64_t row_bytes = d * esz;
    const int kch = int(row_bytes / 16);
    const int64_t tensor = L.BH * n * row_bytes;
    const int64_t vt_bytes = L.BH * d * L.n_pad * 2;
    int bad = 0;
    for (int64_t bh = 0; bh < L.BH; bh += (L.BH > 2 ? L.BH - 1 : 1))
        for (int64_t t = 0; t < L.n_kt; ++t) {
            for (int r = 0; r < BK; ++r)
                for (int c = 0; c < kch; ++c) {
                    const int64_t off = tile_row_src(bh, n, t, r, row_bytes, c);
                    if (off < 0 || off + 16 > tensor) {
                        if (bad++ < 5)
                            std::printf("k/v out of range: n=%lld d=%lld t=%lld r=%d off=%lld\n",
                                        (long long)n, (long long)d, (long long)t, r, (long long)off);
                    }
                }
            if (bf16_path)
                for (int dd = 0; dd < d; ++dd)
                    for (int c = 0; c < BK * 2 / 16; ++c) {
                        const int64_t off = vt_src(bh, d, L.n_pad, t, dd, c);
                        if (off < 0 || off + 16 > vt_bytes) {
                            if (bad++ < 5)
                                std::printf("v^T out of range: n=%lld t=%lld d=%d c=%d\n",
                                            (long long)n, (long long)t, dd, c);
                        }
                    }
        }
    return bad;
}

int main(int argc, char **argv) {
    int bad = 0, cases = 0;
    for (int a = 1; a + 3 < argc; a += 4) {
        const int64_t B = std::atoll(argv[a]), H = std::atoll(argv[a + 1]);
        const int64_t n = std::atoll(argv[a + 2]), d = std::atoll(argv[a + 3]);
        bad += check(B, H, n, d, 2, true);   // bf16 q, k; bf16 v^T copy
        bad += check(B, H, n, d, 4, false);  // fp32 q, k, v
        ++cases;
    }
    std::printf("%d shapes, %d out-of-range ranges\n", cases, bad);
    return bad ? 1 : 0;
}
