// export_kernels.hip -- the materialising exports of the "Resolvent Operator"
// page's Rust API on gfx950, for inspection at small n (both write an [n, n]
// matrix per head):
//   path_product_kernel   G_ij = a_{j+1} ... a_i (G_ii = 1, 0 above the
//                         diagonal) from given complex gates, f64, each row
//                         accumulated from k = i down to k = j + 1 (the
//                         order the page fixes), so the result is the same to
//                         the bit as that definition evaluated in that order
//   op_gates_kernel       the gates a_k of every position (f64) for
//   operator_row_kernel   W_ij = G_ij e^{qk s_ij} / Z_i^beta of one row per
//                         wave (section "Object"): a first pass over the row's
//                         key tiles forms the shift and the normaliser, a
//                         second writes the weights (float32, 0 above the
//                         diagonal)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "layout.h"

namespace resolvent {
namespace {

using namespace dev;

constexpr int32_t kExpNonFinite = 1;
constexpr int PT = 64;  // rows (and columns) of a path-product tile

// One workgroup of PT threads per (matrix, block of PT rows); thread r owns
// row r0 + r.  Column blocks are taken from the diagonal block down to 0: in
// each the thread extends its running product one column to the left at a
// time into an LDS tile, which the workgroup then stores row by row (PT
// consecutive doubles per store).  Column blocks right of the diagonal block
// are zeros.
__global__ __launch_bounds__(PT) void path_product_kernel(const double *a_re, const double *a_im,
                                                          int64_t n, int64_t n_rb, double *g_re,
                                                          double *g_im) {
#pragma clang fp contract(off)
    __shared__ double tr[PT][PT + 1], ti[PT][PT + 1];
    __shared__ double sr[PT], si[PT];
    const int r = threadIdx.x;
    const int64_t mat = blockIdx.x / n_rb, rb = blockIdx.x % n_rb;
    const int64_t r0 = rb * PT, i = r0 + r;
    const double *ar = a_re + mat * n, *ai = a_im + mat * n;
    double *gr = g_re + mat * n * n, *gi = g_im + mat * n * n;
    const int64_t rows = n - r0 < PT ? n - r0 : PT;
    double pr = 1.0, pi = 0.0;  // the running product of this row
    for (int64_t cb = rb; cb >= 0; --cb) {
        const int64_t c0 = cb * PT;
        // the gates a_{j+1} of this column block (a_n is past the end: unused)
        sr[r] = c0 + r + 1 < n ? ar[c0 + r + 1] : 0.0;
        si[r] = c0 + r + 1 < n ? ai[c0 + r + 1] : 0.0;
        __syncthreads();
        for (int jj = PT - 1; jj >= 0; --jj) {
            const int64_t j = c0 + jj;
            double vr = 0.0, vi = 0.0;
            if (j == i) {
                vr = 1.0;
            } else if (j < i) {  // G_ij = G_i,j+1 a_{j+1}
                const double xr = pr * sr[jj] - pi * si[jj];
                const double xi = pr * si[jj] + pi * sr[jj];
                pr = xr;
                pi = xi;
                vr = pr;
                vi = pi;
            }
            tr[r][jj] = vr;
            ti[r][jj] = vi;
        }
        __syncthreads();
        const int64_t cols = n - c0 < PT ? n - c0 : PT;
        if (r < cols)
            for (int64_t rr = 0; rr < rows; ++rr) {
                gr[(r0 + rr) * n + c0 + r] = tr[rr][r];
                gi[(r0 + rr) * n + c0 + r] = ti[rr][r];
            }
        __syncthreads();
    }
    for (int64_t c0 = (rb + 1) * PT; c0 < n; c0 += PT)  // right of the diagonal block
        if (c0 + r < n)
            for (int64_t rr = 0; rr < rows; ++rr) {
                gr[(r0 + rr) * n + c0 + r] = 0.0;
                gi[(r0 + rr) * n + c0 + r] = 0.0;
            }
}

struct OpArgs {
    const void *q, *k;              // [BH][n][d]
    const float *u, *theta;         // [BH][n]
    double *a_re, *a_im, *a_m;      // gates [BH][n] (workspace)
    double *s_re, *s_im, *s_m;      // a_{p+1} ... a_{t0+64} in p's tile [BH][n] (workspace)
    float *w_re, *w_im;             // [BH][n][n]
    int32_t *status;
    double g;
    int64_t BH, n;
    float c, beta, one_minus_beta;
    int beta_mode, qk_zero;
};

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int OB = 64;  // rows of a query block = keys of a key tile

// An opaque 0: offsetting a table's index by it each tile keeps the compiler
// from hoisting that table's loop-invariant LDS reads into registers.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

__device__ __forceinline__ float4 cg_f4(Cg a) { return {float(a.re), float(a.im), float(a.m), 0.f}; }

// Inclusive scans of 64 lanes' gates in f64: prefix (lane l gets x_0 ... x_l)
// and suffix (lane l gets x_l ... x_63).
__device__ __forceinline__ Cg scan_prefix(Cg x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const Cg y = {__shfl_up(x.re, o), __shfl_up(x.im, o), __shfl_up(x.m, o)};
        if (lane >= o) x = cg_mul(y, x);
    }
    return x;
}
__device__ __forceinline__ Cg scan_suffix(Cg x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const Cg y = cg_down(x, o);
        if (lane + o < 64) x = cg_mul(x, y);
    }
    return x;
}

// Gates of every position, one wave per 64-position tile (4 tiles per
// workgroup), and for each position p of tile t0 the product of the gates
// after it to one past the tile's end, a_{p+1} ... a_{t0+64} (f64 suffix scan;
// gates past n count as 1).  Refuses a non-finite u, theta or g theta (the
// status word was cleared by the kernel before it).
__global__ __launch_bounds__(256) void op_gates_kernel(OpArgs A) {
    const int lane = threadIdx.x & 63;
    const int64_t n = A.n, nt = (n + OB - 1) / OB;
    const int64_t tile = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (tile >= A.BH * nt) return;  // whole waves
    const int64_t bh = tile / nt, t0 = (tile % nt) * OB, p = t0 + lane, x = bh * n + p;
    bool bad = false;
    Cg a = cg_one();
    if (p < n) {
        a = gate_of(A.u[x], A.theta[x], A.g, bad);
        A.a_re[x] = a.re;
        A.a_im[x] = a.im;
        A.a_m[x] = a.m;
    }
    Cg b = cg_down(a, 1);  // a_{p+1}
    if (lane == OB - 1) {  // the first gate of the next tile
        bool unused = false;
        b = p + 1 < n ? gate_of(A.u[x + 1], A.theta[x + 1], A.g, unused) : cg_one();
    }
    if (p + 1 >= n) b = cg_one();
    const Cg sfx = scan_suffix(b, lane);
    if (p < n) {
        A.s_re[x] = sfx.re;
        A.s_im[x] = sfx.im;
        A.s_m[x] = sfx.m;
    }
    if (bad) A.status[0] = kExpNonFinite;
}

__global__ __launch_bounds__(64) void clear_word_kernel(int32_t *w) {
    if (threadIdx.x == 0) w[0] = 0;
}

// W of one block of 64 rows per workgroup of 4 waves (section "Object"):
// blockIdx.x = (blocks from the last) * BH + bh, so the longest rows start
// first.  Key tiles of 64 go from the block's own tile down to 0; wave w
// takes rows 32 (w/2) .. +32 and keys 32 (w%2) .. +32 of each 64 x 64 tile.
// The logits come from one 32x32 MFMA product per wave (the key tile in LDS,
// q in registers); lane (c, h) holds row c of the wave's rows and, in
// register r, key 8 (r/4) + 4h + r%4 of its keys, so a lane's four registers
// r = 4a .. 4a+3 are four consecutive keys of one row: one 16-byte store per
// plane.  The row's running largest live logit and normaliser are per lane.
// Below the own tile the path product factors as G_ij = P_i (C S_j) -- P_i
// the gates r0+1 .. i, C those from the tile's end to r0, S_j the suffix
// inside the tile (gates kernel) -- f64 scans rounded to f32 once and
// multiplied per entry in f32; a zero gate still gives an exact 0.  On the
// own tile the 32x32 diagonal sub-blocks take each row's running product
// across its keys (f64), and the lower-left sub-block splits at row 32.
// Pass 0 forms the shift M and the normaliser z of every row; pass 1
// recomputes the same logits and products and writes
// W_ij = G_ij 2^((L - M) + f), f = log2 of the row scale 2^((1-beta) M) z^-beta.
template <bool QF32, int D>
__global__ __launch_bounds__(256, 2) void operator_block_kernel(OpArgs A) {
    constexpr int ESZ = QF32 ? 4 : 2;
    constexpr int KH = D / 2;               // elements of a row each lane half covers
    constexpr int NCH = D * ESZ / 16;       // 16-byte chunks of a key row
    constexpr int ROWB = D * ESZ + 16;      // padded LDS key row (conflict-free reads)
    constexpr int NQ = KH * ESZ / 16;       // 16-byte words of q a lane holds
    __shared__ __align__(16) unsigned char ks[OB * ROWB];
    __shared__ float4 cs[OB];       // C S_j of the tile's keys (f32)
    __shared__ float4 pr[OB];       // P_i of the block's rows
    __shared__ float4 p2[OB / 2];   // rows 32..63: gates r0+33 .. i
    __shared__ float4 s1[OB / 2];   // keys 0..31: gates j+1 .. r0+32
    __shared__ double ga[3][OB];    // the block's gates a_{r0+l} (re, im, |a|)
    __shared__ float gd[2][3][32][33];  // G of the two 32x32 diagonal sub-blocks [row][key]
    __shared__ float2 part[OB];     // (M, z) of keys 32..63, per row
    __shared__ float2 mf[OB];       // (M, f) per row
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr = w >> 1, wc = w & 1, h = lane >> 5, c32 = lane & 31;
    // positions fit in int (n <= 65536); head offsets are 64-bit
    const int n = int(A.n);
    const int nb = (n + OB - 1) / OB;
    const int64_t bh = int64_t(blockIdx.x) % A.BH;
    const int qb = nb - 1 - int(int64_t(blockIdx.x) / A.BH);
    const int r0 = qb * OB;
    const double *ar = A.a_re + bh * n, *ai = A.a_im + bh * n, *am = A.a_m + bh * n;
    const double *sre = A.s_re + bh * n, *sim = A.s_im + bh * n, *smo = A.s_m + bh * n;
    const char *kbase = static_cast<const char *>(A.k) + bh * n * (D * ESZ);
    bool bad = false;

    // the block's gates and their scans (wave 0)
    if (w == 0) {
        const int p = r0 + lane;
        const Cg a = p < n ? Cg{ar[p], ai[p], am[p]} : cg_one();
        ga[0][lane] = a.re;
        ga[1][lane] = a.im;
        ga[2][lane] = a.m;
        pr[lane] = cg_f4(scan_prefix(lane == 0 ? cg_one() : a, lane));
        // split at 32: rows 32.. take gates r0+33 .. i; keys ..31 gates j+1 .. r0+32
        const Cg x2 = lane <= 32 ? cg_one() : a;
        const Cg q2 = scan_prefix(x2, lane);
        if (lane >= 32) p2[lane - 32] = cg_f4(q2);
        const Cg x1 = (lane >= 1 && lane <= 32) ? a : cg_one();
        const Cg q1 = scan_suffix(x1, lane);  // lane l: gates l .. 32 (l >= 1)
        const Cg s = cg_lane(q1, lane + 1 < 64 ? lane + 1 : 63);
        if (lane < 32) s1[lane] = cg_f4(s);
    }

    // q of the lane's row 32 wr + c, elements KH h ..
    const int irel = 32 * wr + c32, i = r0 + irel;
    uint4 qw[NQ];
    {
        const int qrow = min(i, n - 1);
        const char *qp = static_cast<const char *>(A.q) + ((bh * n + qrow) * D + KH * h) * ESZ;
#pragma unroll
        for (int x = 0; x < NQ; ++x) qw[x] = *reinterpret_cast<const uint4 *>(qp + 16 * x);
        float qv[16 / ESZ];
#pragma unroll
        for (int x = 0; x < NQ; ++x) {
            unpack16<QF32>(qw[x], qv);
#pragma unroll
            for (int e = 0; e < 16 / ESZ; ++e)
                if (!isfinite(qv[e])) bad = true;
        }
    }
    __syncthreads();
    if (wr == wc) {  // the diagonal sub-blocks: row c's running product over its keys
        const int base = 32 * wr;
        Cg R = {0.0, 0.0, 0.0};
        for (int kk = 31; kk >= 0; --kk) {
            if (kk == c32)
                R = cg_one();
            else if (kk < c32)
                R = cg_mul(R, Cg{ga[0][base + kk + 1], ga[1][base + kk + 1], ga[2][base + kk + 1]});
            if (((kk >> 2) & 1) == h) {
                gd[wr][0][c32][kk] = float(R.re);
                gd[wr][1][c32][kk] = float(R.im);
                gd[wr][2][c32][kk] = float(R.m);
            }
        }
    }
    __syncthreads();
    const float4 prow = pr[irel];               // P_i of the lane's row
    const float4 p2row = p2[c32];               // (rows 32..: used by waves with wr = 1)
    const bool row_ok = i < n;
    float M = -INFINITY, z = 0.f;
    // the lane row's output rows (64-bit base, 32-bit column offsets)
    float *const wre = A.w_re + (bh * n + i) * n, *const wim = A.w_im + (bh * n + i) * n;
    const bool vec4 = (n & 3) == 0;             // rows start 16-byte aligned

    constexpr int KX = OB * NCH / 256;
    constexpr bool KPRE = !(QF32 && D == 128);  // prefetch the next tile (registers allow)
    auto load_k = [&](int t, uint4 (&v)[KX]) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < KX; ++x) {
            const int ci = tid + 256 * x, row = ci / NCH, ch = ci % NCH;
            v[x] = uint4{0u, 0u, 0u, 0u};
            if (t * OB + row < n)
                v[x] = *reinterpret_cast<const uint4 *>(
                    kbase + uint32_t((t * OB + row) * (D * ESZ) + 16 * ch));
        }
    };
    // four consecutive keys j0.. of the lane's row (W_re, W_im planes)
    auto store4 = [&](int j0, const float (&re)[4], const float (&im)[4])
        __attribute__((always_inline)) {
        if (vec4 && j0 + 3 < n) {
            *reinterpret_cast<float4 *>(wre + j0) = make_float4(re[0], re[1], re[2], re[3]);
            *reinterpret_cast<float4 *>(wim + j0) = make_float4(im[0], im[1], im[2], im[3]);
        } else {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                if (j0 + e4 < n) {
                    wre[j0 + e4] = re[e4];
                    wim[j0 + e4] = im[e4];
                }
        }
    };
    // the two passes as separate code: each keeps only its own registers live
    auto run_pass = [&](auto pass_c) __attribute__((always_inline)) {
        constexpr int pass = decltype(pass_c)::value;
        Cg carry = cg_one();                  // wave 0: gates from the tile's end + 1 to r0
        Cg sj = cg_one(), sj_next = cg_one(); // wave 0: in-tile suffix of key t0 + lane
        Cg ft = cg_one(), ft_next = cg_one(); // wave 0: a_{t0+1} ... a_{t0+64}
        uint4 kv[KX];
        if constexpr (KPRE) load_k(qb, kv);
        for (int t = qb; t >= 0; --t) {
            const int t0 = t * OB;
            const bool own = (t == qb);
            if constexpr (!KPRE) load_k(t, kv);
#pragma unroll
            for (int x = 0; x < KX; ++x) {
                const int ci = tid + 256 * x, row = ci / NCH, ch = ci % NCH;
                if (own && pass == 0) {  // each key is checked once, by its own block
                    float kf[16 / ESZ];
                    unpack16<QF32>(kv[x], kf);
#pragma unroll
                    for (int e = 0; e < 16 / ESZ; ++e)
                        if (!isfinite(kf[e])) bad = true;
                }
                *reinterpret_cast<uint4 *>(ks + row * ROWB + 16 * ch) = kv[x];
            }
            if (w == 0 && !own) cs[lane] = cg_f4(cg_mul(carry, sj));
            __syncthreads();
            if (t > 0) {  // the next tile's words; wave 0: its key suffixes, its product
                if constexpr (KPRE) load_k(t - 1, kv);
                if (w == 0) {
                    const int jn = t0 - OB + lane;
                    sj_next = Cg{sre[jn], sim[jn], smo[jn]};
                    ft_next = Cg{sre[t0 - OB], sim[t0 - OB], smo[t0 - OB]};
                }
            }

            // S^T of the wave's sub-block: A = 32 keys (LDS), B = 32 rows (q)
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
            if (!A.qk_zero) {
                const unsigned char *kp = ks + (32 * wc + c32) * ROWB + KH * ESZ * h;
                if constexpr (!QF32) {
                    // fragments read two ahead of the product that uses them
                    bf16x8 kb[2];
                    kb[0] = *reinterpret_cast<const bf16x8 *>(kp);
                    kb[1] = *reinterpret_cast<const bf16x8 *>(kp + 16);
#pragma unroll
                    for (int s = 0; s < NQ; ++s) {
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            kb[s & 1], __builtin_bit_cast(bf16x8, qw[s]), acc, 0, 0, 0);
                        if (s + 2 < NQ) kb[s & 1] = *reinterpret_cast<const bf16x8 *>(kp + 16 * (s + 2));
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < NQ; ++s) {
                        const float4 kf = *reinterpret_cast<const float4 *>(kp + 16 * s);
                        const float4 qf = __builtin_bit_cast(float4, qw[s]);
                        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qf.x, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qf.y, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qf.z, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qf.w, acc, 0, 0, 0);
                    }
                }
            }

            const int oz = opaque_zero();
            const int jb = t0 + 32 * wc + 4 * h;  // key of register 0; register r: jb + 8 (r/4) + r%4
            if (!own) {
                // below the block: every key is causal; G_ij = P_i (C S_j)
                const float4 *ctab = cs + 32 * wc + oz + 4 * h;
                if constexpr (pass == 0) {
                    float L[16], gmv[16], chk = 0.f, tmax = -INFINITY;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        gmv[r] = prow.z * ctab[8 * (r >> 2) + (r & 3)].z;
                        L[r] = 0.f;
                        if (!A.qk_zero) {
#pragma clang fp contract(off)
                            L[r] = acc[r] * A.c;
                        }
                        chk = fmaf(L[r], 0.f, chk);  // NaN once any logit is not finite
                        tmax = fmaxf(tmax, gmv[r] > 0.f ? L[r] : -INFINITY);
                    }
                    if (row_ok) {
                        if (!isfinite(chk)) bad = true;
                        if (tmax > M) {
                            z *= M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - tmax);
                            M = tmax;
                        }
#pragma unroll
                        for (int r = 0; r < 16; ++r)  // a dead entry adds 0
                            z = fmaf(gmv[r], gmv[r] > 0.f ? __builtin_amdgcn_exp2f(L[r] - M) : 0.f, z);
                    }
                } else if (row_ok) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        float wv_re[4], wv_im[4];
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            const int r = 4 * a + e4;
                            const float4 c = ctab[8 * a + e4];
                            float L = 0.f;
                            if (!A.qk_zero) {
#pragma clang fp contract(off)
                                L = acc[r] * A.c;
                            }
                            const float e = prow.z * c.z > 0.f
                                                ? __builtin_amdgcn_exp2f((L - M) + z) : 0.f;
                            wv_re[e4] = scale_keep_zero(prow.x * c.x - prow.y * c.y, e);
                            wv_im[e4] = scale_keep_zero(prow.x * c.y + prow.y * c.x, e);
                        }
                        store4(jb + 8 * a, wv_re, wv_im);
                    }
                }
            } else {
            // own tile: path products of the lane's 16 entries (re, im, |G|)
            float gr[16], gi[16], gm[16];
            if (wr != wc) {
                if (wr == 0) {  // keys above every row of the sub-block
#pragma unroll
                    for (int r = 0; r < 16; ++r) gr[r] = gi[r] = gm[r] = 0.f;
                } else {  // rows 32.., keys ..31: (gates r0+33 .. i)(gates j+1 .. r0+32)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float4 c = s1[oz + 8 * (r >> 2) + 4 * h + (r & 3)];
                        gr[r] = p2row.x * c.x - p2row.y * c.y;
                        gi[r] = p2row.x * c.y + p2row.y * c.x;
                        gm[r] = p2row.z * c.z;
                    }
                }
            } else {  // diagonal sub-block (products formed once per block)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = oz + 8 * (r >> 2) + 4 * h + (r & 3);
                    gr[r] = gd[wr][0][c32][kk];
                    gi[r] = gd[wr][1][c32][kk];
                    gm[r] = gd[wr][2][c32][kk];
                }
            }
            if constexpr (pass == 0) {
                // this tile's largest live logit of the row, then one rescale
                float L[16], tmax = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = jb + 8 * (r >> 2) + (r & 3);
                    const bool key = j <= i && row_ok;
                    L[r] = 0.f;
                    if (!A.qk_zero) {
#pragma clang fp contract(off)
                        L[r] = acc[r] * A.c;
                    }
                    if (key && !isfinite(L[r])) bad = true;
                    const bool live = key && gm[r] > 0.f;
                    if (!live) gm[r] = 0.f;
                    tmax = live ? fmaxf(tmax, L[r]) : tmax;
                }
                if (tmax > M) {
                    z *= M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - tmax);
                    M = tmax;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)  // a dead entry has gm = 0: adds 0
                    z = fmaf(gm[r], gm[r] > 0.f ? __builtin_amdgcn_exp2f(L[r] - M) : 0.f, z);
            } else if (row_ok) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    float wv_re[4], wv_im[4];
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const int r = 4 * a + e4, j = jb + 8 * a + e4;
                        float L = 0.f;
                        if (!A.qk_zero) {
#pragma clang fp contract(off)
                            L = acc[r] * A.c;
                        }
                        const bool live = j <= i && gm[r] > 0.f;
                        const float e = live ? __builtin_amdgcn_exp2f((L - M) + z) : 0.f;
                        wv_re[e4] = scale_keep_zero(gr[r], e);
                        wv_im[e4] = scale_keep_zero(gi[r], e);
                    }
                    store4(jb + 8 * a, wv_re, wv_im);
                }
            }
            }
            if (w == 0 && !own) carry = cg_mul(ft, carry);  // C for the tile below
            sj = sj_next;
            ft = ft_next;
            __syncthreads();  // the tile buffers are rewritten next
        }
        if constexpr (pass == 0) {
            // merge (M, z) over the two lane halves, then the two waves of the row
            {
                const float Mo = __shfl_xor(M, 32), zo = __shfl_xor(z, 32);
                const float Mn = fmaxf(M, Mo);
                if (Mn != -INFINITY) z = z * exp2f(M - Mn) + zo * exp2f(Mo - Mn);
                M = Mn;
            }
            if (wc == 1 && h == 0) part[irel] = make_float2(M, z);
            __syncthreads();
            if (wc == 0 && h == 0) {
                const float2 o = part[irel];
                const float Mn = fmaxf(M, o.x);
                const float zt = z * exp2f(M - Mn) + o.y * exp2f(o.x - Mn);
                float f;
                if (A.beta_mode == 1)
                    f = -log2f(zt);
                else if (A.beta_mode == 0)
                    f = Mn;
                else
                    f = A.one_minus_beta * Mn - A.beta * log2f(zt);
                mf[irel] = make_float2(Mn, f);
            }
            __syncthreads();
            const float2 x = mf[irel];  // pass 1: M = the row's shift, z = f
            M = x.x;
            z = x.y;
        }
    };
    run_pass(std::integral_constant<int, 0>{});
    run_pass(std::integral_constant<int, 1>{});
    // columns right of the block's own tile are zeros
    const int c0 = r0 + OB, rows = min(OB, n - r0);
    if (c0 < n) {
        float *zr = A.w_re + (bh * n + r0) * n, *zi = A.w_im + (bh * n + r0) * n;
        if (vec4) {
            const int n4 = (n - c0) / 4;
            for (int x = tid; x < rows * n4; x += 256) {
                const int rr = x / n4, c = c0 + 4 * (x % n4);
                *reinterpret_cast<float4 *>(zr + int64_t(rr) * n + c) = make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<float4 *>(zi + int64_t(rr) * n + c) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        } else {
            for (int rr = 0; rr < rows; ++rr)
                for (int jj = c0 + tid; jj < n; jj += 256) {
                    zr[int64_t(rr) * n + jj] = 0.f;
                    zi[int64_t(rr) * n + jj] = 0.f;
                }
        }
    }
    if (__any(bad) && lane == 0) A.status[0] = kExpNonFinite;
}

template <bool QF32, int D>
void launch_blocks(const OpArgs &A, hipStream_t st) {
    const int64_t nb = (A.n + OB - 1) / OB;
    hipLaunchKernelGGL((operator_block_kernel<QF32, D>), dim3((unsigned)(A.BH * nb)), dim3(256),
                       0, st, A);
}

}  // namespace

int launch_path_product(const double *a_re, const double *a_im, int64_t batch, int64_t n,
                        double *g_re, double *g_im, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t n_rb = (n + PT - 1) / PT;
    hipLaunchKernelGGL(path_product_kernel, dim3((unsigned)(batch * n_rb)), dim3(PT), 0, st, a_re,
                       a_im, n, n_rb, g_re, g_im);
    return (int)hipGetLastError();
}

int launch_operator(const OperatorLayout &OL, const void *q, const void *k, const float *u,
                    const float *theta, bool qk_f32, double g, float c, float beta,
                    int beta_mode, bool qk_zero, float *w_re, float *w_im, unsigned char *ws,
                    int32_t *status, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    OpArgs A;
    A.q = q;
    A.k = k;
    A.u = u;
    A.theta = theta;
    A.a_re = reinterpret_cast<double *>(ws + OL.a_re);
    A.a_im = reinterpret_cast<double *>(ws + OL.a_im);
    A.a_m = reinterpret_cast<double *>(ws + OL.a_m);
    A.s_re = reinterpret_cast<double *>(ws + OL.s_re);
    A.s_im = reinterpret_cast<double *>(ws + OL.s_im);
    A.s_m = reinterpret_cast<double *>(ws + OL.s_m);
    A.w_re = w_re;
    A.w_im = w_im;
    A.status = status;
    A.g = g;
    A.BH = OL.BH;
    A.n = OL.n;
    A.c = c;
    A.beta = beta;
    A.one_minus_beta = 1.0f - beta;
    A.beta_mode = beta_mode;
    A.qk_zero = qk_zero ? 1 : 0;
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(64), 0, st, status);
    const int64_t tiles = OL.BH * ((OL.n + OB - 1) / OB);
    hipLaunchKernelGGL(op_gates_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, st, A);
    const int key = (qk_f32 ? 2 : 0) + (OL.d == 128 ? 1 : 0);
    switch (key) {
        case 0: launch_blocks<false, 64>(A, st); break;
        case 1: launch_blocks<false, 128>(A, st); break;
        case 2: launch_blocks<true, 64>(A, st); break;
        case 3: launch_blocks<true, 128>(A, st); break;
    }
    return (int)hipGetLastError();
}

}  // namespace resolvent
