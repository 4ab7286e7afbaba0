// chain_kernels.hip -- the path-product corner of the resolvent head as an
// O(n dv) scan (gfx950).
//
// At switches (beta, qk, g) = (0, 0, g) every weight of the head is its path
// product, W_ij = G_ij (e^0 = 1 and Z^0 = 1; "Resolvent Operator" page,
// section "Object"), so the readout is
//     O_i = sum_{j<=i} G_ij V_j,
// the gated chain y_i = a_i y_{i-1} + V_i of the section "The path-product
// corner is a resolvent", per value channel, started at y_0 = V_0 (a_0 is
// never read, so the chain's first term is the value itself).  This is a
// first-order complex linear recurrence in each channel; it is scanned in the
// 64-position key tiles of the forward pass:
//   chain_agg16_kernel  each tile's end value from a zero carry-in, per
//   (chain_agg_kernel   channel: agg_t = sum_{j in t} S_j V_j (S_j the
//    for other widths)  exclusive suffix product inside the tile)
//   chain_carry_kernel  the carry into each tile, folded over the earlier
//                       tiles in f64 with the whole-tile gate products:
//                       Y_t = A_t Y_{t-1} + agg_t, in 8 segments per head
//   chain_out_kernel    each tile's chain from its carry, writing O
// The gates a_k, the suffix products S_j and the tile products A_t (f64) come
// from gates_kernel, the forward pass's own, so a closed gate (a_k = 0) cuts
// the chain exactly.  HBM traffic: v twice, O once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.h"

namespace resolvent {
namespace {

struct ChainArgs {
    const void *v;              // [BH][n][dv], bf16 or float32
    const float *a_re, *a_im;   // gate planes [BH][n_pad]
    const float *s_re, *s_im;   // exclusive in-tile suffix products [BH][n_pad]
    const double *t_re, *t_im;  // whole-tile gate products [BH][n_kt]
    float2 *agg, *carry;        // [BH][n_kt][dv]
    float *o_re, *o_im;         // [BH][n][dv]
    int64_t n, n_pad;
    int n_kt, dv;
};

template <bool VF32>
__device__ __forceinline__ float load_v(const void *v, int64_t idx) {
    if constexpr (VF32) {
        return static_cast<const float *>(v)[idx];
    } else {
        const uint16_t b = static_cast<const uint16_t *>(v)[idx];
        return __uint_as_float(uint32_t(b) << 16);
    }
}

// Values of channels idx and idx+1 (idx even; v aligned for the pair).
template <bool VF32>
__device__ __forceinline__ float2 load_v2(const void *v, int64_t idx) {
    if constexpr (VF32) {
        return *reinterpret_cast<const float2 *>(static_cast<const float *>(v) + idx);
    } else {
        const uint32_t b = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(v) + idx);
        return make_float2(__uint_as_float(b << 16), __uint_as_float(b & 0xFFFF0000u));
    }
}

typedef __attribute__((address_space(4))) const float cfloat;  // read via the scalar cache

// The values of CPL channels at position index idx (clamped into the tile).
template <bool VF32, int CPL>
__device__ __forceinline__ void load_vals(const void *v, int64_t idx, float (&x)[CPL]) {
    if constexpr (CPL == 2) {
        const float2 x2 = load_v2<VF32>(v, idx);
        x[0] = x2.x;
        x[1] = x2.y;
    } else {
        x[0] = load_v<VF32>(v, idx);
    }
}

// The end value of each tile's chain from a zero carry-in, per channel:
//     agg_t = sum_{j in t} S_j V_j,   S_j = a_{j+1} ... a_{end of t}
// (the exclusive suffix product inside the tile, from gates_kernel) -- a
// reduction with no dependence between positions, so all of a tile's value
// loads are in flight at once.  Positions past n hold no value.  Same grid
// and lanes as chain_out_kernel.  A whole tile takes a path without
// per-position guards (with them the compiler serialises the loads).
template <bool VF32, int CPL, bool FULL>
__device__ __forceinline__ void agg_sum(const ChainArgs &A, cfloat *sr, cfloat *si, int64_t vb,
                                        int cnt, float (&acc_r)[CPL], float (&acc_i)[CPL]) {
    constexpr int HALF = BK / 2;
#pragma unroll
    for (int h0 = 0; h0 < BK; h0 += HALF) {
        float x[HALF][CPL];
#pragma unroll
        for (int q = 0; q < HALF; ++q) {
            const int p = FULL ? h0 + q : (h0 + q < cnt ? h0 + q : cnt - 1);
            load_vals<VF32, CPL>(A.v, vb + int64_t(p) * A.dv, x[q]);
        }
#pragma unroll
        for (int q = 0; q < HALF; ++q) {
            const float gr = sr[h0 + q], gi = si[h0 + q];
            const bool live = FULL || h0 + q < cnt;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const float xv = live ? x[q][e] : 0.f;
                acc_r[e] = fmaf(gr, xv, acc_r[e]);
                acc_i[e] = fmaf(gi, xv, acc_i[e]);
            }
        }
    }
}

template <bool VF32, int CPL>
__global__ __launch_bounds__(64) void chain_agg_kernel(ChainArgs A) {
    const int64_t bh = blockIdx.x / A.n_kt;
    const int t = int(blockIdx.x % A.n_kt);
    const int c = (int(blockIdx.y) * 64 + int(threadIdx.x)) * CPL;
    const int64_t p0 = int64_t(t) * BK;
    const int cnt = int(A.n - p0 < BK ? A.n - p0 : BK);
    const int64_t ci = (bh * A.n_kt + t) * A.dv + c;
    float acc_r[CPL], acc_i[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        acc_r[e] = 0.f;
        acc_i[e] = 0.f;
    }
    if (cnt > 0) {
        cfloat *sr = (cfloat *)(uintptr_t)(A.s_re + bh * A.n_pad + p0);
        cfloat *si = (cfloat *)(uintptr_t)(A.s_im + bh * A.n_pad + p0);
        const int64_t vb = (bh * A.n + p0) * A.dv + c;
        if (cnt == BK)
            agg_sum<VF32, CPL, true>(A, sr, si, vb, cnt, acc_r, acc_i);
        else
            agg_sum<VF32, CPL, false>(A, sr, si, vb, cnt, acc_r, acc_i);
    }
#pragma unroll
    for (int e = 0; e < CPL; ++e) A.agg[ci + e] = make_float2(acc_r[e], acc_i[e]);
}

// The same aggregate with whole 16-byte value loads: one wave per (head,
// tile) covers all DVW channels; VL lanes read a row (VE channels a lane), so
// one load instruction covers VR rows and the tile takes VI of them, all in
// flight at once.  Lane (r, c) accumulates its VE channels over the rows
// r, r + VR, ...; the suffix factor of a row comes from the lane holding that
// position (a lane shuffle), and the VR row groups are summed at the end.
template <bool VF32, int DVW>
__global__ __launch_bounds__(64) void chain_agg16_kernel(ChainArgs A) {
    constexpr int VE = VF32 ? 4 : 8, VL = DVW / VE, VR = 64 / VL, VI = BK / VR;
    static_assert(VL >= 1 && VL <= 64 && 64 % VL == 0, "row split");
    const int lane = threadIdx.x;
    const int64_t bh = blockIdx.x / A.n_kt;
    const int t = int(blockIdx.x % A.n_kt);
    const int64_t p0 = int64_t(t) * BK;
    const int cnt = int(A.n - p0 < BK ? A.n - p0 : BK);
    const int vc = (lane % VL) * VE, vr = lane / VL;
    float acc_r[VE], acc_i[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        acc_r[e] = 0.f;
        acc_i[e] = 0.f;
    }
    if (cnt > 0) {
        const char *vb = static_cast<const char *>(A.v) + ((bh * A.n + p0) * DVW + vc) * (VF32 ? 4 : 2);
        uint4 w[VI];
#pragma unroll
        for (int x = 0; x < VI; ++x) {
            const int row = x * VR + vr < cnt ? x * VR + vr : cnt - 1;
            w[x] = *reinterpret_cast<const uint4 *>(vb + int64_t(row) * DVW * (VF32 ? 4 : 2));
        }
        // this lane's position's suffix factor (0 past the tile's last value)
        const float sl_r = lane < cnt ? A.s_re[bh * A.n_pad + p0 + lane] : 0.f;
        const float sl_i = lane < cnt ? A.s_im[bh * A.n_pad + p0 + lane] : 0.f;
#pragma unroll
        for (int x = 0; x < VI; ++x) {
            const int row = x * VR + vr;
            const float gr = __shfl(sl_r, row), gi = __shfl(sl_i, row);
            const uint32_t u[4] = {w[x].x, w[x].y, w[x].z, w[x].w};
            float xv[VE];
            if constexpr (VF32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[e] = __uint_as_float(u[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xv[2 * e] = __uint_as_float(u[e] << 16);
                    xv[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
                }
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                acc_r[e] = fmaf(gr, xv[e], acc_r[e]);
                acc_i[e] = fmaf(gi, xv[e], acc_i[e]);
            }
        }
    }
#pragma unroll
    for (int o = VL; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            acc_r[e] += __shfl_xor(acc_r[e], o);
            acc_i[e] += __shfl_xor(acc_i[e], o);
        }
    if (lane < VL) {
        float2 *ag = A.agg + (bh * A.n_kt + t) * DVW + vc;
#pragma unroll
        for (int e = 0; e < VE; e += 2)
            *reinterpret_cast<float4 *>(ag + e) =
                make_float4(acc_r[e], acc_i[e], acc_r[e + 1], acc_i[e + 1]);
    }
}

// One wave per (key tile t, head bh) -- flattened as blockIdx.x = bh n_kt + t
// -- and channel group blockIdx.y of 64 CPL channels; lane L runs the CPL
// independent chains of channels 64 CPL y + CPL L + e.  The tile's positions
// go in chunks of CH: the values of chunk k+1 are requested before chunk k is
// computed and stored, so a wait for chunk k's values never waits for the
// stores before it (loads and stores share one counter).  The gates are
// uniform: read through the scalar cache.
template <bool VF32, int CPL, bool FULL>
__device__ __forceinline__ void out_scan(const ChainArgs &A, cfloat *ar, cfloat *ai, int64_t vb,
                                         int cnt, float (&yr)[CPL], float (&yi)[CPL]) {
    constexpr int CH = 16;
    const void *__restrict__ v = A.v;
    float *__restrict__ ore = A.o_re;
    float *__restrict__ oim = A.o_im;
    float cur[CH][CPL], nxt[CH][CPL];
#pragma unroll
    for (int q = 0; q < CH; ++q)
        load_vals<VF32, CPL>(v, vb + int64_t(FULL ? q : (q < cnt ? q : cnt - 1)) * A.dv, cur[q]);
#pragma unroll
    for (int k0 = 0; k0 < BK; k0 += CH) {
        if (FULL ? k0 + CH < BK : k0 + CH < cnt) {
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                const int p = FULL ? k0 + CH + q : (k0 + CH + q < cnt ? k0 + CH + q : cnt - 1);
                load_vals<VF32, CPL>(v, vb + int64_t(p) * A.dv, nxt[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int p = k0 + q;
            if (FULL || p < cnt) {
                const float gr = ar[p], gi = ai[p];
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const float nr = gr * yr[e] - gi * yi[e] + cur[q][e];
                    const float ni = gr * yi[e] + gi * yr[e];
                    yr[e] = nr;
                    yi[e] = ni;
                }
                const int64_t idx = vb + int64_t(p) * A.dv;
                if constexpr (CPL == 2) {
                    *reinterpret_cast<float2 *>(ore + idx) = make_float2(yr[0], yr[1]);
                    *reinterpret_cast<float2 *>(oim + idx) = make_float2(yi[0], yi[1]);
                } else {
                    ore[idx] = yr[0];
                    oim[idx] = yi[0];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < CH; ++q)
#pragma unroll
            for (int e = 0; e < CPL; ++e) cur[q][e] = nxt[q][e];
    }
}

template <bool VF32, int CPL>
__global__ __launch_bounds__(64) void chain_out_kernel(ChainArgs A) {
    const int64_t bh = blockIdx.x / A.n_kt;
    const int t = int(blockIdx.x % A.n_kt);
    const int c = (int(blockIdx.y) * 64 + int(threadIdx.x)) * CPL;
    const int64_t p0 = int64_t(t) * BK;
    const int cnt = int(A.n - p0 < BK ? A.n - p0 : BK);
    if (cnt <= 0) return;  // a padding tile past n
    cfloat *ar = (cfloat *)(uintptr_t)(A.a_re + bh * A.n_pad + p0);
    cfloat *ai = (cfloat *)(uintptr_t)(A.a_im + bh * A.n_pad + p0);
    const int64_t vb = (bh * A.n + p0) * A.dv + c;
    const int64_t ci = (bh * A.n_kt + t) * A.dv + c;
    float yr[CPL], yi[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        const float2 cy = A.carry[ci + e];
        yr[e] = cy.x;
        yi[e] = cy.y;
    }
    if (cnt == BK)
        out_scan<VF32, CPL, true>(A, ar, ai, vb, cnt, yr, yi);
    else
        out_scan<VF32, CPL, false>(A, ar, ai, vb, cnt, yr, yi);
}

// The carries into the tiles, in f64: one workgroup of CW waves per (head,
// 64-channel group), lane = channel.  The tiles are split into CW
// consecutive segments; wave s folds its segment from a zero carry-in
// (Y <- A_t Y + agg_t) and records the segment's end value and product; after
// a barrier it folds the earlier segments' records into its own carry-in and
// walks its segment again writing the carries.  The fetches run 16 tiles
// ahead of the dependent steps.
constexpr int CW = 8;
__global__ __launch_bounds__(64 * CW) void chain_carry_kernel(ChainArgs A) {
    constexpr int NB = 16;
    __shared__ double seg_y[2][CW][64];
    __shared__ double seg_p[2][CW];
    const int lane = threadIdx.x % 64, s = threadIdx.x / 64;
    const int64_t bh = blockIdx.x;
    const int c = int(blockIdx.y) * 64 + lane;
    const double *__restrict__ tr = A.t_re + bh * A.n_kt;
    const double *__restrict__ ti = A.t_im + bh * A.n_kt;
    const float2 *__restrict__ agg = A.agg + bh * A.n_kt * A.dv + c;
    float2 *__restrict__ carry = A.carry + bh * A.n_kt * A.dv + c;
    const int len = (A.n_kt + CW - 1) / CW;
    const int t_lo = s * len < A.n_kt ? s * len : A.n_kt;
    const int t_hi = t_lo + len < A.n_kt ? t_lo + len : A.n_kt;
    // pass 0: the segment's own fold (with its product); pass 1: the carries
    double yr = 0.0, yi = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
        double qr = 1.0, qi = 0.0;  // the segment's gate product
        if (pass == 1) {
            __syncthreads();
            yr = 0.0;
            yi = 0.0;
            for (int r = 0; r < s; ++r) {  // Y <- P_r Y + y_r over the earlier segments
                const double pr = seg_p[0][r], pi = seg_p[1][r];
                const double nr = pr * yr - pi * yi + seg_y[0][r][lane];
                const double ni = pr * yi + pi * yr + seg_y[1][r][lane];
                yr = nr;
                yi = ni;
            }
        }
        for (int t0 = t_lo; t0 < t_hi; t0 += NB) {
            float2 e[NB];
            double pr[NB], pi[NB];
#pragma unroll
            for (int x = 0; x < NB; ++x) {
                const int t = t0 + x < t_hi ? t0 + x : t_hi - 1;
                e[x] = agg[int64_t(t) * A.dv];
                pr[x] = tr[t];
                pi[x] = ti[t];
            }
#pragma unroll
            for (int x = 0; x < NB; ++x) {
                if (t0 + x < t_hi) {
                    if (pass == 1) carry[int64_t(t0 + x) * A.dv] = make_float2((float)yr, (float)yi);
                    const double nr = pr[x] * yr - pi[x] * yi + (double)e[x].x;
                    const double ni = pr[x] * yi + pi[x] * yr + (double)e[x].y;
                    yr = nr;
                    yi = ni;
                    if (pass == 0) {
                        const double mr = pr[x] * qr - pi[x] * qi;
                        qi = pr[x] * qi + pi[x] * qr;
                        qr = mr;
                    }
                }
            }
        }
        if (pass == 0) {
            seg_y[0][s][lane] = yr;
            seg_y[1][s][lane] = yi;
            if (lane == 0) {
                seg_p[0][s] = qr;
                seg_p[1][s] = qi;
            }
        }
    }
}

}  // namespace

int launch_chain(const ChainLayout &C, const float *u, const float *theta, const void *v,
                 bool v_f32, double g, float *o_re, float *o_im, unsigned char *ws,
                 int32_t *status, void *stream) {
    const Layout &L = C.g;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int err = launch_gates(L, u, theta, g, ws, status, stream);
    if (err) return err;
    ChainArgs A;
    A.v = v;
    A.a_re = reinterpret_cast<const float *>(ws + L.gate[0]);
    A.a_im = reinterpret_cast<const float *>(ws + L.gate[1]);
    A.s_re = reinterpret_cast<const float *>(ws + L.gate[3]);
    A.s_im = reinterpret_cast<const float *>(ws + L.gate[4]);
    A.t_re = reinterpret_cast<const double *>(ws + L.tile[0]);
    A.t_im = reinterpret_cast<const double *>(ws + L.tile[1]);
    A.agg = reinterpret_cast<float2 *>(ws + C.agg);
    A.carry = reinterpret_cast<float2 *>(ws + C.carry);
    A.o_re = o_re;
    A.o_im = o_im;
    A.n = L.n;
    A.n_pad = L.n_pad;
    A.n_kt = (int)L.n_kt;
    A.dv = (int)C.dv;
    const dim3 heads((unsigned)L.BH, (unsigned)(C.dv / 64));
    const dim3 wide((unsigned)(L.BH * L.n_kt));
    // the aggregate with 16-byte loads when a row of values splits evenly over
    // the lanes and v is 16-byte aligned
    const bool v16 = reinterpret_cast<uintptr_t>(v) % 16 == 0;
    bool agg_done = true;
    if (v16 && !v_f32 && C.dv == 64)
        hipLaunchKernelGGL((chain_agg16_kernel<false, 64>), wide, dim3(64), 0, st, A);
    else if (v16 && !v_f32 && C.dv == 128)
        hipLaunchKernelGGL((chain_agg16_kernel<false, 128>), wide, dim3(64), 0, st, A);
    else if (v16 && !v_f32 && C.dv == 256)
        hipLaunchKernelGGL((chain_agg16_kernel<false, 256>), wide, dim3(64), 0, st, A);
    else if (v16 && v_f32 && C.dv == 64)
        hipLaunchKernelGGL((chain_agg16_kernel<true, 64>), wide, dim3(64), 0, st, A);
    else if (v16 && v_f32 && C.dv == 128)
        hipLaunchKernelGGL((chain_agg16_kernel<true, 128>), wide, dim3(64), 0, st, A);
    else
        agg_done = false;
    // two channels per lane (8-byte stores) when the channels come in whole
    // 128s and the outputs allow it: fewer waves, two independent chains each
    const bool pairs = C.dv % 128 == 0 && reinterpret_cast<uintptr_t>(o_re) % 8 == 0 &&
                       reinterpret_cast<uintptr_t>(o_im) % 8 == 0 &&
                       reinterpret_cast<uintptr_t>(v) % (v_f32 ? 8 : 4) == 0;
    const dim3 tiles((unsigned)(L.BH * L.n_kt), (unsigned)(C.dv / (pairs ? 128 : 64)));
    if (!agg_done) {
        if (pairs && v_f32)
            hipLaunchKernelGGL((chain_agg_kernel<true, 2>), tiles, dim3(64), 0, st, A);
        else if (pairs)
            hipLaunchKernelGGL((chain_agg_kernel<false, 2>), tiles, dim3(64), 0, st, A);
        else if (v_f32)
            hipLaunchKernelGGL((chain_agg_kernel<true, 1>), tiles, dim3(64), 0, st, A);
        else
            hipLaunchKernelGGL((chain_agg_kernel<false, 1>), tiles, dim3(64), 0, st, A);
    }
    hipLaunchKernelGGL(chain_carry_kernel, heads, dim3(64 * CW), 0, st, A);
    if (pairs && v_f32)
        hipLaunchKernelGGL((chain_out_kernel<true, 2>), tiles, dim3(64), 0, st, A);
    else if (pairs)
        hipLaunchKernelGGL((chain_out_kernel<false, 2>), tiles, dim3(64), 0, st, A);
    else if (v_f32)
        hipLaunchKernelGGL((chain_out_kernel<true, 1>), tiles, dim3(64), 0, st, A);
    else
        hipLaunchKernelGGL((chain_out_kernel<false, 1>), tiles, dim3(64), 0, st, A);
    return (int)hipGetLastError();
}

}  // namespace resolvent
