// Host check of the fused kernel's direct global->LDS copies: every source
// range that a workgroup can ask for lies inside its tensor (K, V) or
// inside the workspace (the gate planes).  It walks
// every key tile of every shape given on the command line (all tiles a
// workgroup of any query tile stages, the logit check included), every row
// and every 16-byte chunk, using the same helpers as the kernel.  For the
// bf16 tiles it also walks the copy instructions lane by lane: each reads a
// chunk inside the tensor, each (row, chunk) of a tile is copied once, into
// the LDS slot where the matrix-operand reads look for it, and a 16-lane
// group of an operand read touches 16 different bank groups.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "layout.h"

using namespace resolvent;

// Every k/v head the kernels address (bh below runs over k/v heads: the
// query heads' kv_head()), with Hkv k/v heads and dv value channels.
static int check(int64_t B, int64_t H, int64_t n, int64_t d, int esz, bool bf16_path,
                 int64_t Hkv, int64_t dv) {
    const Layout L = make_layout(B, H, n, d, bf16_path, Hkv, dv);
    const int64_t row_bytes = d * esz;
    const int kch = int(row_bytes / 16);
    const int64_t tensor = L.BHkv * n * row_bytes;
    const int64_t vrow_bytes = dv * esz;
    const int64_t vtensor = L.BHkv * n * vrow_bytes;
    int bad = 0;
    // the query heads map onto k/v heads inside the batch entry
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t kv = b * L.Hkv + h / (H / L.Hkv);
            if ((kv < 0 || kv >= L.BHkv) && bad++ < 5)
                std::printf("query head (%lld,%lld) maps to k/v head %lld of %lld\n",
                            (long long)b, (long long)h, (long long)kv, (long long)L.BHkv);
        }
    for (int64_t bh = 0; bh < L.BHkv; bh += (L.BHkv > 2 ? L.BHkv - 1 : 1))
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
            if (!bf16_path)  // fp32 V rows of dv channels
                for (int r = 0; r < BK; ++r)
                    for (int c = 0; c < int(vrow_bytes / 16); ++c) {
                        const int64_t off = bh * n * vrow_bytes +
                                            int64_t(tile_row_off(n, t, r, vrow_bytes)) + 16 * c;
                        if ((off < 0 || off + 16 > vtensor) && bad++ < 5)
                            std::printf("v out of range: n=%lld dv=%lld t=%lld r=%d\n",
                                        (long long)n, (long long)dv, (long long)t, r);
                    }
            // the padded copies of fwd_pad_kernel, lane by lane: K rows from k and
            // value rows from the bf16 values (v itself, or v rounded to bf16 in
            // the workspace when it comes as fp32: both [BHkv][n][dv]); a tile
            // reaching past key n-1 takes head-relative, clamped offsets
            if (bf16_path) {
                const int64_t head_k = bh * n * row_bytes, head_v = bh * n * dv * 2;
                const int ksl = d == 128 ? pad_kslots<128>() : pad_kslots<64>();
                const int vsl = dv == 128 ? pad_vslots<128>() : pad_vslots<64>();
                const bool ragged = (t + 1) * BK > n;
                auto src = [&](int j, int lane) -> int64_t {
                    if (d == 128)
                        return dv == 128 ? pad_copy_src<128, 128>(j, lane) : pad_copy_src<128, 64>(j, lane);
                    return dv == 128 ? pad_copy_src<64, 128>(j, lane) : pad_copy_src<64, 64>(j, lane);
                };
                for (int j = 0; j < ksl + vsl; ++j)
                    for (int lane = 0; lane < 64; ++lane) {
                        int64_t lo, hi, off;
                        if (j < ksl) {
                            lo = head_k;
                            hi = head_k + n * row_bytes;
                            if (ragged)
                                off = head_k + (d == 128 ? pad_kcopy_src_ragged<128>(j, lane, n, t)
                                                         : pad_kcopy_src_ragged<64>(j, lane, n, t));
                            else
                                off = head_k + t * BK * row_bytes + src(j, lane);
                        } else {
                            lo = head_v;
                            hi = head_v + n * dv * 2;
                            if (ragged)
                                off = head_v + (dv == 128 ? pad_vcopy_src_ragged<128>(j - ksl, lane, n, t)
                                                          : pad_vcopy_src_ragged<64>(j - ksl, lane, n, t));
                            else
                                off = head_v + t * BK * dv * 2 + src(j, lane);
                        }
                        if ((off < lo || off + 16 > hi) && bad++ < 5)
                            std::printf("padded copy out of its head: n=%lld d=%lld dv=%lld t=%lld "
                                        "j=%d lane=%d\n", (long long)n, (long long)d, (long long)dv,
                                        (long long)t, j, lane);
                        if (bh * n * dv * 2 + n * dv * 2 > L.BHkv * n * dv * 2 && bad++ < 5)
                            std::printf("value head past the tensor: bh=%lld\n", (long long)bh);
                    }
            }
        }
    // gate planes of every query head: S_j (planes 3..5) and a_{j+1} (planes
    // 0..2), 4 bytes a lane
    for (int64_t bh = 0; bh < L.BH; bh += (L.BH > 2 ? L.BH - 1 : 1))
        for (int64_t t = 0; t < L.n_kt; ++t)
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
    // the tile-product copies: lanes 0 and 1 read 16 bytes each of the
    // key tile's (A_re, A_im, A_m, 0) doubles
    for (int64_t bh = 0; bh < L.BH; bh += (L.BH > 2 ? L.BH - 1 : 1))
        for (int64_t t = 0; t < L.n_kt; ++t)
            for (int lane = 0; lane < 2; ++lane) {
                const int64_t off = int64_t(L.tile4) + 32 * (bh * L.n_kt + t) + 16 * lane;
                if ((off < int64_t(L.tile4) || off + 16 > int64_t(L.tile4) + 32 * L.BH * L.n_kt ||
                     off + 16 > int64_t(L.total)) &&
                    bad++ < 5)
                    std::printf("tile product out of range: n=%lld t=%lld lane=%d\n",
                                (long long)n, (long long)t, lane);
            }
    return bad;
}

// The padded bf16 tiles of fwd_pad_kernel (d = D, value width DV), independent
// of the shape: every copy instruction j < NC is issued by some copying wave;
// the 64 slots of instruction j (lane L -> slot 64 j + L) hold, for a
// non-padding slot, exactly the (row, chunk) the slot stands for, every
// (row, chunk) of the K and value tiles is held by exactly one non-padding
// slot, every K operand read stays inside the K tile and each of its 16-lane
// groups touches 16 distinct bank groups (16-byte units modulo 16).  The value
// reads are simulated with the transposing read's lane exchange (lane i of a
// 16-lane group receives element i & 3 of the 8-byte pieces that lanes
// (i >> 2) + 4 e address): lane l must receive the keys
// kb + 16 kc + 8 s + 4 (l >> 5) + e of channel 32 db + (l & 31), from
// non-padding slots inside the value tile (value row q holding key
// pad_vrow_key(q)), with no two lanes of a half wave on one bank (64 banks of
// 4 bytes).
template <int D, int DV>
static int check_pad_layout() {
    constexpr int KSL = pad_kslots<D>(), VSL = pad_vslots<DV>(), NC = pad_copies<D, DV>();
    constexpr int CPW = pad_copies_per_wave<D, DV>();
    constexpr int kbytes = 1024 * pad_kcopies<D>(), vbytes = 1024 * pad_vcopies<DV>();
    constexpr int VSTR = 16 * VSL;
    int bad = 0;
    auto fail = [&](const char *what, int a, int b) {
        if (bad++ < 10) std::printf("pad layout d=%d dv=%d: %s (%d, %d)\n", D, DV, what, a, b);
    };
    std::vector<int> issued(NC, 0);
    for (int w = 1; w < NWAVES; ++w)
        for (int i = 0; i < CPW; ++i) {
            const int j = pad_copy_j<D, DV>(w, i);
            if (j < 0 || j >= NC) fail("copy index", w, i);
            else issued[j] += 1;
        }
    for (int j = 0; j < NC; ++j)
        if (!issued[j]) fail("copy never issued", j, 0);
    if (1024 * NC != kbytes + vbytes) fail("copies do not tile the buffer", NC, 0);
    if (BK * VSTR != vbytes) fail("value rows do not fill the value tile", VSTR, vbytes);
    // which slot holds (row, chunk): from the copies (source side)
    std::vector<int> kslot(BK * (D / 8), -1), vslot(BK * (DV / 8), -1);
    for (int j = 0; j < NC; ++j)
        for (int lane = 0; lane < 64; ++lane) {
            const int p = 64 * j + lane;
            const uint32_t src = pad_copy_src<D, DV>(j, lane);
            if (j < KSL) {
                const int r = int(src / (D * 2)), c = int(src % (D * 2)) / 16;
                if (r < 0 || r >= BK || c < 0 || c >= D / 8) { fail("K copy source", j, lane); continue; }
                if (p % KSL != KSL - 1) {  // not the padding slot
                    if (kslot[r * (D / 8) + c] != -1) fail("K chunk copied twice", r, c);
                    kslot[r * (D / 8) + c] = p;
                    if (p / KSL != r || p % KSL != c) fail("K slot holds another chunk", r, c);
                }
            } else {
                const int q = p - 64 * KSL;
                const int r = int(src / (DV * 2)), c = int(src % (DV * 2)) / 16;
                if (r < 0 || r >= BK || c < 0 || c >= DV / 8) { fail("value copy source", j, lane); continue; }
                if (q % VSL < DV / 8) {  // not a padding slot
                    if (vslot[r * (DV / 8) + c] != -1) fail("value chunk copied twice", r, c);
                    vslot[r * (DV / 8) + c] = p;
                    // value row q / VSL holds key pad_vrow_key(q / VSL) whole
                    if (pad_vrow_key(q / VSL) != r || q % VSL != c)
                        fail("value slot holds another chunk", r, c);
                }
            }
        }
    for (size_t x = 0; x < kslot.size(); ++x)
        if (kslot[x] < 0) fail("K chunk never copied", int(x / (D / 8)), int(x % (D / 8)));
    for (size_t x = 0; x < vslot.size(); ++x)
        if (vslot[x] < 0) fail("value chunk never copied", int(x / (DV / 8)), int(x % (DV / 8)));
    // K operand reads (reader side)
    for (int kb = 0; kb < BK; kb += 32)
        for (int st = 0; st < D / 16; ++st)
            for (int g = 0; g < 4; ++g) {
                const int h = g >> 1;
                unsigned used = 0;
                for (int q = 0; q < 16; ++q) {
                    const int qi = 16 * (g & 1) + q;
                    const int off = pad_kread<D>(kb, st, qi, h);
                    if (off < 0 || off + 16 > kbytes) fail("K read outside the K tile", kb, st);
                    else if (off != 16 * kslot[(kb + qi) * (D / 8) + 2 * st + h])
                        fail("K read misses its chunk", kb + qi, 2 * st + h);
                    used |= 1u << ((off / 16) % 16);
                }
                if (used != 0xFFFFu) fail("K read bank groups", kb, int(used));
            }
    // value operand reads: the transposing 8-byte reads, simulated
    int worst_bank = 0;
    for (int kb = 0; kb < BK; kb += 32)
        for (int kc = 0; kc < 2; ++kc)
            for (int db = 0; db < DV / 32; ++db)
                for (int s = 0; s < 2; ++s) {
                    int row[64], ch[64];
                    for (int lane = 0; lane < 64; ++lane) {
                        const int off = pad_vread_tr<D, DV>(kb, kc, db, s, lane);
                        row[lane] = ch[lane] = -1;
                        if (off < kbytes || off + 8 > kbytes + vbytes || off % 8) {
                            fail("value read outside the value tile", kb, lane);
                            continue;
                        }
                        const int o = off - kbytes, q = o / VSTR, cb = o % VSTR;
                        if (cb + 8 > DV * 2) { fail("value read in a padding slot", q, cb); continue; }
                        const int r = pad_vrow_key(q);  // the key value row q holds
                        if (o / 16 != vslot[r * (DV / 8) + cb / 16] - 64 * KSL)
                            fail("value read misses its chunk", r, cb / 16);
                        row[lane] = r;
                        ch[lane] = cb / 2;
                    }
                    for (int half = 0; half < 2; ++half) {
                        std::vector<int> bank(64, 0);
                        for (int lane = 32 * half; lane < 32 * half + 32; ++lane) {
                            const int off = pad_vread_tr<D, DV>(kb, kc, db, s, lane);
                            for (int b = 0; b < 2; ++b) worst_bank = std::max(worst_bank, ++bank[(off / 4 + b) % 64]);
                        }
                    }
                    for (int lane = 0; lane < 64; ++lane) {
                        const int g = lane >> 4, i = lane & 15;
                        for (int e = 0; e < 4; ++e) {
                            const int srcl = 16 * g + (i >> 2) + 4 * e;
                            const int key = row[srcl], chan = ch[srcl] < 0 ? -1 : ch[srcl] + (i & 3);
                            const int want_key = kb + 16 * kc + 8 * s + 4 * (lane >> 5) + e;
                            const int want_ch = 32 * db + (lane & 31);
                            if (key != want_key || chan != want_ch) fail("value lane gets another element", lane, e);
                        }
                    }
                }
    if (worst_bank > 1) fail("value read: lanes of a half wave on one bank", worst_bank, 0);
    return bad;
}

// The decode step's reads and writes (decode_part_kernel,
// decode_merge_kernel), walked lane by lane: every 16-byte load of q, k and v
// lies inside its tensor, every key row 0..n-1 of a query head's k/v head is
// read whole by the chunks of that head, every gate 0..n-1 is read once, and
// the chunk product, scale and partial indexes stay inside their workspace
// regions.  esz_q / esz_v: element bytes of q,k / v; cap: positions per head.
static int check_decode(int64_t B, int64_t H, int64_t Hkv, int64_t n, int64_t cap, int64_t d,
                        int64_t dv, int esz_q, int esz_v) {
    const DecodeLayout DL = make_decode_layout(B, H, Hkv, n, d, dv);
    const int64_t BH = DL.BH, BHkv = B * Hkv, n_ch = DL.n_ch;
    const int ke = 16 / esz_q, kl = int(d) / ke, kr_n = 64 / kl;
    const int ve = 16 / esz_v, vl = int(dv) / ve, vr_n = 64 / vl;
    const int64_t kbytes = BHkv * cap * d * esz_q, vbytes = BHkv * cap * dv * esz_v;
    const int64_t pf = dec_part_floats(dv), i = n - 1;
    const size_t per = 3 * sizeof(double) * size_t(BH) * size_t(n_ch);
    int bad = 0;
    auto fail = [&](const char *what, int64_t bh, int64_t x) {
        if (bad++ < 10)
            std::printf("decode B=%lld H=%lld Hkv=%lld n=%lld d=%lld dv=%lld: %s (bh %lld, %lld)\n",
                        (long long)B, (long long)H, (long long)Hkv, (long long)n, (long long)d,
                        (long long)dv, what, (long long)bh, (long long)x);
    };
    if (n_ch * DEC_CHUNK < n || (n_ch - 1) * DEC_CHUNK >= n) fail("chunk count", 0, n_ch);
    if (DL.prod + per > DL.scale || DL.scale + size_t(16 * BH * n_ch) > DL.part)
        fail("product/scale regions", 0, 0);
    if (DL.part + size_t(4 * BH * n_ch * pf) > DL.total) fail("partials region", 0, 0);
    if ((DL.part % 16) || (pf % 4)) fail("partials not 16-byte aligned", 0, 0);
    const int seg = int((n_ch + 255) / 256);
    std::vector<int> cseen(size_t(n_ch), 0);
    for (int t = 0; t < 256; ++t) {  // decode_merge_kernel's segments cover every chunk once
        const int64_t c0 = std::min<int64_t>(int64_t(t) * seg, n_ch), c1 = std::min<int64_t>(c0 + seg, n_ch);
        for (int64_t c = c0; c < c1; ++c) cseen[size_t(c)] += 1;
    }
    for (int64_t c = 0; c < n_ch; ++c)
        if (cseen[size_t(c)] != 1) fail("merge segment", 0, c);
    for (int64_t bh = 0; bh < BH; ++bh) {
        const int64_t kvh = (bh / H) * Hkv + (bh % H) / (H / Hkv);
        if (kvh < 0 || kvh >= BHkv) fail("k/v head", bh, kvh);
        std::vector<int> kseen(size_t(n) * (d * esz_q / 16), 0),
            vseen(size_t(n) * (dv * esz_v / 16), 0), useen(size_t(n), 0);
        for (int64_t ch = 0; ch < n_ch; ++ch) {
            if (bh * n_ch + ch >= BH * n_ch) fail("chunk index", bh, ch);
            for (int lane = 0; lane < 64; ++lane) {
                const int64_t qoff = (bh * d + (lane % kl) * ke) * esz_q;
                if (qoff < 0 || qoff + 16 > BH * d * esz_q) fail("q load", bh, lane);
                const int64_t po = (bh * n_ch + ch) * pf;
                if (lane < vl && po + 4 + dv + (lane % vl) * ve + ve > BH * n_ch * pf)
                    fail("partial write", bh, lane);
                // the merge reads chunk ch's partial with CPL channels a lane
                const int cpl = int(dv / 64);
                if (po + 4 + dv + lane * cpl + cpl > BH * n_ch * pf) fail("merge read", bh, lane);
            }
            for (int tt = DEC_CT - 1; tt >= 0; --tt) {
                const int64_t t0 = ch * DEC_CHUNK + tt * BK;
                if (t0 > i) continue;
                const int cnt = int(i - t0 + 1 < BK ? i - t0 + 1 : BK);
                for (int lane = 0; lane < 64; ++lane) {
                    if (t0 + lane < n) {
                        if (bh * cap + t0 + lane >= BH * cap) fail("u read (part)", bh, lane);
                        useen[size_t(t0 + lane)] += 1;
                    }
                    for (int x = 0; x < BK / kr_n; ++x) {
                        const int r = x * kr_n + lane / kl, row = r < cnt ? r : cnt - 1;
                        const int64_t off = (kvh * cap + t0 + row) * d * esz_q + (lane % kl) * ke * esz_q;
                        if (r >= BK) fail("logit slot", bh, r);
                        if (off < 0 || off + 16 > kbytes) fail("k load", bh, off);
                        else kseen[size_t((t0 + row) * (d * esz_q / 16) + lane % kl)] = 1;
                    }
                    for (int x = 0; x < BK / vr_n; ++x) {
                        const int r = x * vr_n + lane / vl, row = r < cnt ? r : cnt - 1;
                        const int64_t off = (kvh * cap + t0 + row) * dv * esz_v + (lane % vl) * ve * esz_v;
                        if (off < 0 || off + 16 > vbytes) fail("v load", bh, off);
                        else vseen[size_t((t0 + row) * (dv * esz_v / 16) + lane % vl)] = 1;
                    }
                }
            }
        }
        for (size_t c = 0; c < kseen.size(); ++c)
            if (!kseen[c]) fail("k chunk never read", bh, int64_t(c));
        for (size_t c = 0; c < vseen.size(); ++c)
            if (!vseen[c]) fail("v chunk never read", bh, int64_t(c));
        for (size_t c = 0; c < useen.size(); ++c)  // every gate checked exactly once
            if (useen[c] != 1) fail("position's gate not checked once", bh, int64_t(c));
    }
    return bad;
}

// The exports: every load of operator_row_kernel (q row i, k rows j <= i,
// gates a_{j+1} with j < i) and store (w row i) stays inside its tensor, and
// path_product_kernel stores every entry of each matrix exactly once.
static int check_exports(int64_t B, int64_t H, int64_t n, int64_t d, int esz) {
    const int64_t BH = B * H;
    const int ke = 16 / esz, kl = int(d) / ke, kr_n = 64 / kl;
    int bad = 0;
    auto fail = [&](const char *what, int64_t a, int64_t b) {
        if (bad++ < 10)
            std::printf("exports B=%lld H=%lld n=%lld d=%lld: %s (%lld, %lld)\n", (long long)B,
                        (long long)H, (long long)n, (long long)d, what, (long long)a, (long long)b);
    };
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t i = 0; i < n; ++i) {
            for (int lane = 0; lane < 64; ++lane) {
                const int64_t qoff = ((bh * n + i) * d + (lane % kl) * ke) * esz;
                if (qoff + 16 > BH * n * d * esz) fail("q load", i, lane);
            }
            for (int64_t t = i / BK; t >= 0; --t) {
                const int64_t t0 = t * BK;
                const int cnt = int(i - t0 + 1 < BK ? i - t0 + 1 : BK);
                for (int lane = 0; lane < 64; ++lane) {
                    for (int x = 0; x < BK / kr_n; ++x) {
                        const int r = x * kr_n + lane / kl, row = r < cnt ? r : cnt - 1;
                        const int64_t off = ((bh * n + t0 + row) * d + (lane % kl) * ke) * esz;
                        if (t0 + row > i || off < 0 || off + 16 > BH * n * d * esz)
                            fail("k load", i, t0 + row);
                    }
                    const int64_t j = t0 + lane;
                    if (j < i && (j + 1 >= n || bh * n + j + 1 >= BH * n)) fail("gate read", i, j);
                    if (lane < cnt && (j > i || (bh * n + i) * n + j >= BH * n * n))
                        fail("w store", i, j);
                }
            }
        }
    // path_product_kernel on one matrix
    const int64_t n_rb = (n + 63) / 64;
    std::vector<int> seen(size_t(n) * size_t(n), 0);
    for (int64_t rb = 0; rb < n_rb; ++rb) {
        const int64_t r0 = rb * 64, rows = std::min<int64_t>(64, n - r0);
        for (int64_t cb = rb; cb >= 0; --cb) {
            const int64_t c0 = cb * 64, cols = std::min<int64_t>(64, n - c0);
            for (int r = 0; r < 64; ++r) {
                if (c0 + r + 1 < n && c0 + r + 1 < 0) fail("gate stage", cb, r);
                if (r < cols)
                    for (int64_t rr = 0; rr < rows; ++rr) seen[size_t((r0 + rr) * n + c0 + r)] += 1;
            }
        }
        for (int64_t c0 = (rb + 1) * 64; c0 < n; c0 += 64)
            for (int r = 0; r < 64; ++r)
                if (c0 + r < n)
                    for (int64_t rr = 0; rr < rows; ++rr) seen[size_t((r0 + rr) * n + c0 + r)] += 1;
    }
    for (size_t x = 0; x < seen.size(); ++x)
        if (seen[x] != 1) fail("path product entry not stored once", int64_t(x / n), int64_t(x % n));
    return bad;
}

// The chain scan's 16-byte aggregate (chain_agg16_kernel: every value row
// 0..n-1 of a head read whole, loads and aggregate stores inside their
// arrays) and the segments of chain_carry_kernel (every tile folded by
// exactly one segment).  esz: element bytes of v.
static int check_chain(int64_t B, int64_t H, int64_t n, int64_t dv, int esz) {
    const ChainLayout C = make_chain_layout(B, H, n, dv);
    const Layout &L = C.g;
    const int ve = 16 / esz, vl = int(dv) / ve, vr_n = 64 / vl;
    int bad = 0;
    auto fail = [&](const char *what, int64_t a, int64_t b) {
        if (bad++ < 10)
            std::printf("chain B=%lld H=%lld n=%lld dv=%lld: %s (%lld, %lld)\n", (long long)B,
                        (long long)H, (long long)n, (long long)dv, what, (long long)a, (long long)b);
    };
    for (int64_t bh = 0; bh < L.BH; ++bh) {
        std::vector<int> seen(size_t(n) * size_t(vl), 0);
        for (int64_t t = 0; t < L.n_kt; ++t) {
            const int64_t p0 = t * BK;
            const int cnt = int(n - p0 < BK ? n - p0 : BK);
            if (cnt <= 0) continue;
            for (int lane = 0; lane < 64; ++lane) {
                for (int x = 0; x < BK / vr_n; ++x) {
                    const int r = x * vr_n + lane / vl, row = r < cnt ? r : cnt - 1;
                    const int64_t off = ((bh * n + p0 + row) * dv + (lane % vl) * ve) * esz;
                    if (off < 0 || off + 16 > L.BH * n * dv * esz) fail("v load", t, lane);
                    else seen[size_t((p0 + row) * vl + lane % vl)] = 1;
                }
                if (lane < cnt && bh * L.n_pad + p0 + lane >= L.BH * L.n_pad) fail("s read", t, lane);
                if (lane < vl && (bh * L.n_kt + t) * dv + (lane % vl) * ve + ve > L.BH * L.n_kt * dv)
                    fail("agg store", t, lane);
            }
        }
        for (size_t x = 0; x < seen.size(); ++x)
            if (!seen[x]) fail("value chunk never read", bh, int64_t(x));
    }
    const int cw = 8, len = int((L.n_kt + cw - 1) / cw);
    std::vector<int> tseen(size_t(L.n_kt), 0);
    for (int s = 0; s < cw; ++s) {
        const int64_t lo = std::min<int64_t>(int64_t(s) * len, L.n_kt);
        const int64_t hi = std::min<int64_t>(lo + len, L.n_kt);
        for (int64_t t = lo; t < hi; ++t) tseen[size_t(t)] += 1;
    }
    for (int64_t t = 0; t < L.n_kt; ++t)
        if (tseen[size_t(t)] != 1) fail("carry segment", 0, t);
    return bad;
}

// The work queues of the bf16 forward (queue_item): for every item order and
// either queue count, the entries of all queues up to their ends are every
// query tile exactly once, heaviest first inside a queue under order 0, and
// the first entry past a queue's end is -1.
static int check_queues(int64_t B, int64_t H, int64_t n) {
    const Layout L = make_layout(B, H, n, 64, true);
    const int64_t BH = L.BH, n_qt = L.n_qt;
    int bad = 0;
    for (int nq : {1, 8}) {
        if (BH % nq != 0) continue;
        for (int order = 0; order < 3; ++order) {
            const int64_t q0 = order == 2 ? n_qt / 4 : 0;
            std::vector<int> seen(size_t(BH * n_qt), 0);
            for (int x = 0; x < nq; ++x) {
                int64_t prev_qt = n_qt;
                for (uint32_t k = 0;; ++k) {
                    const int64_t it = queue_item(x, k, nq, BH, n_qt, order, q0);
                    if (it < 0) {
                        if (int64_t(k) != BH / nq * n_qt && bad++ < 5)
                            std::printf("queue %d of %d ends at %u\n", x, nq, k);
                        break;
                    }
                    if ((it >= BH * n_qt || (it / n_qt) % nq != x) && bad++ < 5) {
                        std::printf("queue %d entry %u: item %lld\n", x, k, (long long)it);
                        break;
                    }
                    ++seen[size_t(it)];
                    if (order == 0) {
                        if (it % n_qt > prev_qt && bad++ < 5)
                            std::printf("queue %d entry %u not heaviest first\n", x, k);
                        prev_qt = it % n_qt;
                    }
                }
            }
            for (int64_t i = 0; i < BH * n_qt; ++i)
                if (seen[size_t(i)] != 1 && bad++ < 5)
                    std::printf("query tile %lld queued %d times (nq %d order %d)\n",
                                (long long)i, seen[size_t(i)], nq, order);
        }
    }
    return bad;
}

int main(int argc, char **argv) {
    int bad = check_pad_layout<128, 128>() + check_pad_layout<128, 64>() +
              check_pad_layout<64, 128>() + check_pad_layout<64, 64>();
    int cases = 0;
    for (int a = 1; a + 3 < argc; a += 4) {
        const int64_t B = std::atoll(argv[a]), H = std::atoll(argv[a + 1]);
        const int64_t n = std::atoll(argv[a + 2]), d = std::atoll(argv[a + 3]);
        for (int64_t dv = 64; dv <= 128; dv += 64)
            for (int64_t Hkv : {H, int64_t(1)}) {
                bad += check(B, H, n, d, 2, true, Hkv, dv);   // bf16 q, k, v
                bad += check(B, H, n, d, 4, false, Hkv, dv);  // fp32 q, k, v
                if (H % Hkv == 0 && n <= 40000) {
                    bad += check_decode(B, H, Hkv, n, n, d, dv, 2, 2);
                    bad += check_decode(B, H, Hkv, n, n + 37, d, dv, 2, 4);
                    bad += check_decode(B, H, Hkv, n, n, d, dv, 4, 4);
                }
            }
        for (int64_t cdv : {int64_t(64), int64_t(128), int64_t(256)}) {
            bad += check_chain(B, H, n, cdv, 2);
            if (cdv <= 128) bad += check_chain(B, H, n, cdv, 4);
        }
        bad += check_queues(B, H, n);
        if (n <= 1100) {
            bad += check_exports(B, H, n, d, 2);
            bad += check_exports(B, H, n, d, 4);
        }
        ++cases;
    }
    std::printf("%d shapes, %d problems\n", cases, bad);
    return bad ? 1 : 0;
}
