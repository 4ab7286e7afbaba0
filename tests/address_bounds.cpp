// Host check of the fused kernel's direct global->LDS copies: every source
// range that a workgroup can ask for lies inside its tensor (K, V, v^T) or
// inside the workspace (the gate planes).  It walks
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
                    // the kernels' form: head base + 32-bit in-head offset
                    const int64_t alt = bh * n * row_bytes +
                                        int64_t(tile_row_off(n, t, r, row_bytes)) + 16 * c;
                    if (alt != off && bad++ < 5)
                        std::printf("k/v 32-bit offset mismatch: n=%lld t=%lld r=%d\n",
                                    (long long)n, (long long)t, r);
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
                        const int64_t alt =
                            bh * d * L.n_pad * 2 + int64_t(vt_row_off(L.n_pad, t, dd)) + 16 * c;
                        if (alt != off && bad++ < 5)
                            std::printf("v^T 32-bit offset mismatch: n=%lld t=%lld d=%d\n",
                                        (long long)n, (long long)t, dd);
                        if (off < 0 || off + 16 > vt_bytes) {
                            if (bad++ < 5)
                                std::printf("v^T out of range: n=%lld t=%lld d=%d c=%d\n",
                                            (long long)n, (long long)t, dd, c);
                        }
                    }
            // gate planes: S_j (planes 3..5) and a_{j+1} (planes 0..2), 4 bytes a lane
            for (int own = 0; own < 2; ++own)
                for (int p = own ? 0 : 3; p < (own ? 3 : 6); ++p)
                    for (int lane = 0; lane < BK; ++lane) {
                        const int64_t off =
                            int64_t(L.gate[p]) + 4 * gate_src(bh, L.n_pad, t, lane, own != 0);
                        if (off < 0 || off + 4 > int64_t(L.total)) {
                            if (bad++ < 5)
                                std::printf("gate plane %d out of range: n=%lld t=%lld lane=%d\n",
                                            p, (long long)n, (long long)t, lane);
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
