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
    float *w_re, *w_im;             // [BH][n][n]
    int32_t *status;
    double g;
    int64_t BH, n;
    float c, beta, one_minus_beta;
    int beta_mode, qk_zero;
};

// Gates of every position, one thread each; refuses a non-finite u, theta or
// g theta (the status word was cleared by the kernel before it).
__global__ __launch_bounds__(256) void op_gates_kernel(OpArgs A) {
    const int64_t x = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (x >= A.BH * A.n) return;
    bool bad = false;
    const Cg a = gate_of(A.u[x], A.theta[x], A.g, bad);
    A.a_re[x] = a.re;
    A.a_im[x] = a.im;
    A.a_m[x] = a.m;
    if (bad) A.status[0] = kExpNonFinite;
}

__global__ __launch_bounds__(64) void clear_word_kernel(int32_t *w) {
    if (threadIdx.x == 0) w[0] = 0;
}

// One wave per (head, row i): blockIdx.x = bh n + i.  Key tiles are taken from
// the row's own tile down to 0; lane j of a tile holds key t0 + j.  Key rows
// are read KL lanes to a row (16 bytes a lane) and their dot products reduced
// across those lanes; the gates after each key come from a suffix product
// across lanes of b_j = a_{j+1} (1 from j = i on) times the product of the
// later tiles.  Pass 0 forms the shift M (largest live logit) and the
// normaliser; pass 1 recomputes the same logits and products and writes
// W_ij = G_ij 2^(L_j - M) exp2((1-beta) M) z^-beta (one exponential per entry).
template <bool QF32, int D>
__global__ __launch_bounds__(64) void operator_row_kernel(OpArgs A) {
    constexpr int KE = QF32 ? 4 : 8, KL = D / KE, KR = 64 / KL, KI = BK / KR;
    constexpr int KB = QF32 ? 4 : 2;
    __shared__ float dots[BK];
    const int lane = threadIdx.x;
    const int64_t bh = blockIdx.x / A.n, i = blockIdx.x % A.n;
    const int kc = (lane % KL) * KE, kr = lane / KL;
    const uint32_t koff = uint32_t(kc * KB);
    const char *kbase = static_cast<const char *>(A.k) + bh * A.n * (D * KB);
    const double *ar = A.a_re + bh * A.n, *ai = A.a_im + bh * A.n, *am = A.a_m + bh * A.n;
    float *wr = A.w_re + (bh * A.n + i) * A.n, *wi = A.w_im + (bh * A.n + i) * A.n;
    bool bad = false;
    float qv[KE];
    unpack16<QF32>(load16<QF32>(A.q, (bh * A.n + i) * D + kc), qv);
#pragma unroll
    for (int e = 0; e < KE; ++e)
        if (!isfinite(qv[e])) bad = true;
    const int ti = int(i / BK);
    float M = -INFINITY, z = 0.f, f = 0.f;
    for (int pass = 0; pass < 2; ++pass) {
        Cg carry = cg_one();  // the gates from the current tile's end to i
        for (int t = ti; t >= 0; --t) {
            const int64_t t0 = int64_t(t) * BK;
            const int cnt = i - t0 + 1 < BK ? int(i - t0 + 1) : BK;
            const char *kt = kbase + t0 * (D * KB);
            uint4 kw[KI];
#pragma unroll
            for (int x = 0; x < KI; ++x) {
                const int row = x * KR + kr < cnt ? x * KR + kr : cnt - 1;
                kw[x] = *reinterpret_cast<const uint4 *>(kt + (uint32_t(row) * (D * KB) + koff));
            }
#pragma unroll
            for (int x = 0; x < KI; ++x) {
                float kx[KE];
                unpack16<QF32>(kw[x], kx);
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < KE; ++e) {
                    if (!isfinite(kx[e])) bad = true;
                    part = fmaf(qv[e], kx[e], part);
                }
#pragma unroll
                for (int o = 1; o < KL; o <<= 1) part += __shfl_xor(part, o);
                if (lane % KL == 0) dots[x * KR + kr] = part;
            }
            __syncthreads();
            const bool key = lane < cnt;
            float L = 0.f;
            if (!A.qk_zero) {
#pragma clang fp contract(off)
                L = dots[lane] * A.c;
                if (key && !isfinite(L)) bad = true;
            }
            __syncthreads();  // dots is rewritten by the next tile
            const int64_t j = t0 + lane;
            Cg sfx = j < i ? Cg{ar[j + 1], ai[j + 1], am[j + 1]} : cg_one();
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const Cg x = cg_down(sfx, o);
                if (lane + o < 64) sfx = cg_mul(sfx, x);
            }
            const Cg G = cg_mul(sfx, carry);
            carry = cg_mul(cg_lane(sfx, 0), carry);
            const float gm = float(G.m);
            const bool live = key && gm > 0.0f;
            if (pass == 0) {
                const float tmax = wave_max(live ? L : -INFINITY);
                if (tmax > M) {
                    z *= M == -INFINITY ? 0.f : exp2f(M - tmax);
                    M = tmax;
                }
                if (live) z = fmaf(gm, exp2f(L - M), z);
            } else if (key) {
                // one exponential per entry, 2^((L - M) + log2 f): no product of an
                // underflowed and an overflowed factor
                const float e = live ? exp2f((L - M) + f) : 0.f;
                wr[j] = scale_keep_zero(float(G.re), e);
                wi[j] = scale_keep_zero(float(G.im), e);
            }
        }
        if (pass == 0) {  // f: log2 of the row's scale 2^((1-beta) M) z^-beta
            const float zt = wave_sum(z);
            if (A.beta_mode == 1)
                f = -log2f(zt);
            else if (A.beta_mode == 0)
                f = M;
            else
                f = A.one_minus_beta * M - A.beta * log2f(zt);
        }
    }
    for (int64_t j = i + 1 + lane; j < A.n; j += 64) {  // above the diagonal
        wr[j] = 0.f;
        wi[j] = 0.f;
    }
    if (__any(bad) && lane == 0) A.status[0] = kExpNonFinite;
}

template <bool QF32, int D>
void launch_rows(const OpArgs &A, hipStream_t st) {
    hipLaunchKernelGGL((operator_row_kernel<QF32, D>), dim3((unsigned)(A.BH * A.n)), dim3(64), 0,
                       st, A);
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
    hipLaunchKernelGGL(op_gates_kernel, dim3((unsigned)((OL.BH * OL.n + 255) / 256)), dim3(256),
                       0, st, A);
    const int key = (qk_f32 ? 2 : 0) + (OL.d == 128 ? 1 : 0);
    switch (key) {
        case 0: launch_rows<false, 64>(A, st); break;
        case 1: launch_rows<false, 128>(A, st); break;
        case 2: launch_rows<true, 64>(A, st); break;
        case 3: launch_rows<true, 128>(A, st); break;
    }
    return (int)hipGetLastError();
}

}  // namespace resolvent
