// resolvent_kernels.hip -- HIP kernels (gfx950 / CDNA4) of the resolvent
// operator head forward pass, and their launcher.
//
// The head is the one defined on the "Resolvent Operator" page (teerth.dev,
// Aether-Lang/integrated/resolvent), section "Object"; Z^beta is evaluated in
// the log domain with a shift by the largest live logit as in its section
// "Evaluation and refusals".  The path product G_ij = prod_{k=j+1..i} a_k is
// only ever formed as a product -- never via a logarithm or a division (Lean
// table of the page, no_prefix_scan_represents_a_zero_gate) -- so a closed
// gate yields exact zeros.  For a query tile [i0, i0+BQ) and a key tile t that
// lies wholly before it,
//     G_ij = S_j * C_t * P_i,
// with S_j the exclusive suffix product of the gates inside key tile t, C_t
// the product of every gate between the end of tile t and i0 (carried from
// tile to tile as the key loop runs backwards), and P_i the inclusive prefix
// product inside the query tile.  P_i is applied once to the accumulators
// after the loop; the keys of the query tile itself use G_ij formed explicitly
// by a running product per row, multiplying a_i, a_{i-1}, ..., a_{j+1} in the
// order the page's "Rust API" section fixes.
//
// Kernels, in launch order on the caller's stream:
//   vt_kernel / clear_status_kernel  status := OK; (bf16 path) v -> bf16 v^T
//   gates_kernel                     blend + gate in f64, in-tile scans
//   fwd_kernel                       the fused forward (MFMA)
//   logit_check_kernel               exact logit-overflow refusal, only for
//                                    heads whose |q|,|k| extrema allow one
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "layout.h"

namespace resolvent {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int32_t kNonFinite = 1;
constexpr uint32_t kInfBits = 0x7F800000u;
constexpr int NTHREADS = NWAVES * 64;

// Storage order of keys inside a group of 16: slot p holds key perm16(p)
// (an involution swapping bits 2 and 3).  With it, the 8 keys that one lane
// of a 32x32x16 MFMA operand needs are 8 consecutive slots.
__host__ __device__ constexpr int perm16(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}
__host__ __device__ constexpr int perm64(int x) { return (x & ~15) | perm16(x & 15); }

// |x| of packed bf16 / fp32 values as float bit patterns (monotone in |x|;
// >= kInfBits means inf or NaN).
__device__ __forceinline__ uint32_t absbits_bf16x2(uint32_t w) {
    uint32_t lo = (w & 0x7FFFu) << 16, hi = (w & 0x7FFF0000u);
    return lo > hi ? lo : hi;
}
__device__ __forceinline__ uint32_t absbits_u4_bf16(uint4 v) {
    uint32_t a = max(absbits_bf16x2(v.x), absbits_bf16x2(v.y));
    uint32_t b = max(absbits_bf16x2(v.z), absbits_bf16x2(v.w));
    return max(a, b);
}
__device__ __forceinline__ uint32_t absbits_f4(float4 v) {
    uint32_t a = max(__float_as_uint(v.x) & 0x7FFFFFFFu, __float_as_uint(v.y) & 0x7FFFFFFFu);
    uint32_t b = max(__float_as_uint(v.z) & 0x7FFFFFFFu, __float_as_uint(v.w) & 0x7FFFFFFFu);
    return max(a, b);
}

// --------------------------------------------------------------------------
// Status and counter clear (fp32 path; the bf16 path clears them in vt_kernel).
__global__ void clear_status_kernel(int32_t *status, uint32_t *counters) {
    if (threadIdx.x == 0) status[0] = 0;
    if (threadIdx.x < 2) counters[threadIdx.x] = 0;
}

// --------------------------------------------------------------------------
// v [BH][n][D] (bf16 or fp32) -> v^T [BH][D][n_pad] bf16, keys stored in
// perm16 order inside each group of 16 and zero past n.  Block 0 also clears
// the status word and the counters (this kernel runs first on the bf16 path).
template <int D, bool VF32>
__global__ __launch_bounds__(256) void vt_kernel(const void *__restrict__ v,
                                                  uint16_t *__restrict__ vt, int64_t n,
                                                  int64_t n_pad, int n_kt,
                                                  int32_t *__restrict__ status,
                                                  uint32_t *__restrict__ counters) {
    __shared__ __align__(16) uint16_t tile[D][BK + 8];
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0) status[0] = 0;
    if (blockIdx.x == 0 && tid < 2) counters[tid] = 0;
    const int64_t bh = blockIdx.x / n_kt;
    const int64_t kt = blockIdx.x % n_kt;
    for (int c = tid; c < BK * D / 8; c += 256) {
        const int key = c / (D / 8), c8 = c % (D / 8);
        const int64_t p = kt * BK + key;
        uint16_t vals[8];
        if (p < n) {
            if constexpr (VF32) {
                const float *src = static_cast<const float *>(v) + (bh * n + p) * D + 8 * c8;
                const float4 f0 = *reinterpret_cast<const float4 *>(src);
                const float4 f1 = *reinterpret_cast<const float4 *>(src + 4);
                const float fs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 b = (__bf16)fs[e];
                    vals[e] = __builtin_bit_cast(uint16_t, b);
                }
            } else {
                const uint16_t *src = static_cast<const uint16_t *>(v) + (bh * n + p) * D + 8 * c8;
                const uint4 raw = *reinterpret_cast<const uint4 *>(src);
                const uint32_t ws[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vals[2 * e] = uint16_t(ws[e] & 0xFFFFu);
                    vals[2 * e + 1] = uint16_t(ws[e] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[e] = 0;
        }
        const int slot = perm64(key);
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[8 * c8 + e][slot] = vals[e];
    }
    __syncthreads();
    for (int c = tid; c < D * BK / 8; c += 256) {
        const int d = c / (BK / 8), c8 = c % (BK / 8);
        const uint4 val = *reinterpret_cast<const uint4 *>(&tile[d][8 * c8]);
        *reinterpret_cast<uint4 *>(vt + (bh * D + d) * n_pad + kt * BK + 8 * c8) = val;
    }
}

// --------------------------------------------------------------------------
// Gates: blend and gate in f64 (section "Object"; lerp(1,u,g) = (1-g)*1 + g*u
// without a fused multiply-add, exact at g = 0 and g = 1), the inclusive
// prefix product inside each query tile, the exclusive suffix product inside
// each key tile and the product of each key tile, with modulus twins.  One
// wave per query tile, PPL consecutive positions per lane.  Refuses a
// non-finite u or theta and an overflowing g*theta (section "Evaluation and
// refusals").
struct GatesArgs {
    const float *u, *theta;
    double g;
    int64_t n, n_pad;
    int n_qt, n_kt;
    float *a_re, *a_im, *a_m, *s_re, *s_im, *s_m, *p_re, *p_im, *p_m;
    double *t_re, *t_im, *t_m;
    int32_t *status;
};

__device__ __forceinline__ void cmul_d(double xr, double xi, double yr, double yi, double &r,
                                       double &i) {
    r = xr * yr - xi * yi;
    i = xr * yi + xi * yr;
}

__global__ __launch_bounds__(64) void gates_kernel(GatesArgs A) {
#pragma clang fp contract(off)
    constexpr int PPL = BQ / 64;
    constexpr int SEG = BK / PPL;  // lanes per key tile
    const int lane = threadIdx.x;
    const int64_t bh = blockIdx.x / A.n_qt;
    const int64_t qt = blockIdx.x % A.n_qt;
    const int64_t p0 = qt * BQ + PPL * lane;
    double ar[PPL], ai[PPL], am[PPL];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        const int64_t p = p0 + e;
        if (p < A.n) {
            const float uu = A.u[bh * A.n + p], tt = A.theta[bh * A.n + p];
            if (!isfinite(uu) || !isfinite(tt)) bad = true;
            double l = (1.0 - A.g) * 1.0 + A.g * (double)uu;
            l = l < 0.0 ? 0.0 : (l > 1.0 ? 1.0 : l);
            const double tp = A.g * (double)tt;
            if (!isfinite(tp)) bad = true;
            ar[e] = l * cos(tp);
            ai[e] = l * sin(tp);
            am[e] = l;
        } else {
            ar[e] = 1.0;
            ai[e] = 0.0;
            am[e] = 1.0;
        }
    }
    if (bad) A.status[0] = kNonFinite;

    // inclusive prefix inside the query tile
    double lr[PPL], li[PPL], lm[PPL];
    double cr = 1.0, ci = 0.0, cm = 1.0;
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        cmul_d(cr, ci, ar[e], ai[e], cr, ci);
        cm = cm * am[e];
        lr[e] = cr;
        li[e] = ci;
        lm[e] = cm;
    }
    double xr = cr, xi = ci, xm = cm;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double yr = __shfl_up(xr, off), yi = __shfl_up(xi, off), ym = __shfl_up(xm, off);
        if (lane >= off) {
            cmul_d(yr, yi, xr, xi, xr, xi);
            xm = ym * xm;
        }
    }
    double er = __shfl_up(xr, 1), ei = __shfl_up(xi, 1), em = __shfl_up(xm, 1);
    if (lane == 0) {
        er = 1.0;
        ei = 0.0;
        em = 1.0;
    }
    const int64_t base = bh * A.n_pad;
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        double r, i;
        cmul_d(er, ei, lr[e], li[e], r, i);
        A.p_re[base + p0 + e] = (float)r;
        A.p_im[base + p0 + e] = (float)i;
        A.p_m[base + p0 + e] = (float)(em * lm[e]);
        A.a_re[base + p0 + e] = (float)ar[e];
        A.a_im[base + p0 + e] = (float)ai[e];
        A.a_m[base + p0 + e] = (float)am[e];
    }

    // exclusive suffix inside each key tile, and the key-tile products
    double sr[PPL], si[PPL], sm[PPL];
    double tr = 1.0, ti = 0.0, tm = 1.0;
#pragma unroll
    for (int e = PPL - 1; e >= 0; --e) {
        sr[e] = tr;
        si[e] = ti;
        sm[e] = tm;
        cmul_d(ar[e], ai[e], tr, ti, tr, ti);
        tm = am[e] * tm;
    }
    xr = tr;
    xi = ti;
    xm = tm;
    const int seg_lane = lane % SEG;
#pragma unroll
    for (int off = 1; off < SEG; off <<= 1) {
        const double yr = __shfl_down(xr, off), yi = __shfl_down(xi, off),
                     ym = __shfl_down(xm, off);
        if (seg_lane + off < SEG) {
            cmul_d(xr, xi, yr, yi, xr, xi);
            xm = xm * ym;
        }
    }
    er = __shfl_down(xr, 1);
    ei = __shfl_down(xi, 1);
    em = __shfl_down(xm, 1);
    if (seg_lane == SEG - 1) {
        er = 1.0;
        ei = 0.0;
        em = 1.0;
    }
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        double r, i;
        cmul_d(sr[e], si[e], er, ei, r, i);
        A.s_re[base + p0 + e] = (float)r;
        A.s_im[base + p0 + e] = (float)i;
        A.s_m[base + p0 + e] = (float)(sm[e] * em);
    }
    if (seg_lane == 0) {
        const int64_t kt = (qt * BQ + PPL * lane) / BK;
        A.t_re[bh * A.n_kt + kt] = xr;
        A.t_im[bh * A.n_kt + kt] = xi;
        A.t_m[bh * A.n_kt + kt] = xm;
    }
}

// --------------------------------------------------------------------------
// Fused forward.
struct FwdArgs {
    const void *q, *k, *v;
    const uint16_t *vt;
    const float *a_re, *a_im, *a_m, *s_re, *s_im, *s_m, *p_re, *p_im, *p_m;
    const double *t_re, *t_im, *t_m;
    float *o_re, *o_im;
    uint32_t *qstat, *kstat, *counters;
    int32_t *status;
    int64_t n, n_pad;
    int n_qt, n_kt, BH;
    float c, beta, one_minus_beta;
    int beta_mode, qk_zero;
};

// Shared-memory plan: two buffers, each holding one key tile K [BK][D], its
// values (bf16 path: v^T [D][BK] in perm16 key order; fp32 path: V [BK][D]),
// and per-key side data (the carried gate factor T_j = C*S_j with its modulus
// for tiles before the query tile; the gates a_{j+1} for the query tile's
// own keys).  Tiles are stored 16-byte-chunk-major: chunk c of row r sits at
// (c * rows + r) * 16.  One direct global->LDS wave instruction then copies
// one chunk of 64 consecutive rows (lane L -> row L), and each half-wave of
// an MFMA operand read touches 512 contiguous bytes (no bank conflicts), at
// an immediate offset from one per-lane base address.
template <bool F32, int D>
struct Smem {
    static constexpr int ESZ = F32 ? 4 : 2;
    static constexpr int KCH = D * ESZ / 16;    // 16-byte chunks per K (and fp32 V) row
    static constexpr int VCH = BK * 2 / 16;     // chunks per v^T row (bf16 path)
    static constexpr size_t k_bytes = size_t(KCH) * BK * 16;
    static constexpr size_t v_bytes = F32 ? size_t(KCH) * BK * 16 : size_t(VCH) * D * 16;
    static constexpr size_t side_off = k_bytes + v_bytes;
    // side data: 3 x BK floats, then 2 flag words (32-key block b of the
    // staged tile holds a dead column)
    static constexpr size_t flag_off = side_off + 3 * BK * sizeof(float);
    static constexpr size_t buf_bytes = flag_off + 16;
    static constexpr size_t misc_off = 2 * buf_bytes;
    static constexpr size_t bytes = misc_off + 8 * sizeof(uint32_t);
    static_assert(KCH % NWAVES == 0 && (VCH * D / 64) % NWAVES == 0, "whole wave copies");
};

template <bool F32, int D>
struct Frag {
    using type = typename std::conditional<F32, float, bf16x8>::type;
    static constexpr int count = F32 ? D / 2 : D / 16;
};

typedef __attribute__((address_space(3))) void lds_void;

// A wave-uniform double kept in scalar registers.
__device__ __forceinline__ double uniform_f64(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(b >> 32));
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ void g2lds16(const void *g, unsigned char *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(lds), 16, 0, 0);
}

// Query fragment (B operand of S^T = K Q^T) for the lane's row; returns the
// largest |q| as float bits.
template <bool F32, int D>
__device__ __forceinline__ uint32_t load_q(const FwdArgs &A, int64_t bh, int64_t row, bool row_ok,
                                           int h, typename Frag<F32, D>::type (&qf)[Frag<F32, D>::count]) {
    uint32_t bits = 0;
    if constexpr (!F32) {
        const uint16_t *qp = static_cast<const uint16_t *>(A.q) + (bh * A.n + row) * D + 8 * h;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (row_ok) raw = *reinterpret_cast<const uint4 *>(qp + 16 * s);
            bits = max(bits, absbits_u4_bf16(raw));
            qf[s] = __builtin_bit_cast(bf16x8, raw);
        }
    } else {
        const float *qp = static_cast<const float *>(A.q) + (bh * A.n + row) * D + (D / 2) * h;
#pragma unroll
        for (int t = 0; t < D / 8; ++t) {
            float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row_ok) f = *reinterpret_cast<const float4 *>(qp + 4 * t);
            bits = max(bits, absbits_f4(f));
            qf[4 * t + 0] = f.x;
            qf[4 * t + 1] = f.y;
            qf[4 * t + 2] = f.z;
            qf[4 * t + 3] = f.w;
        }
    }
    return bits;
}

// Start the asynchronous copy of key tile t (K, and the values unless
// k_only) into buffer buf.  Wave w copies chunks w, w+NWAVES, ...: lane L
// fetches 16 bytes of row L.  Keys past n repeat key n-1 (their entries are
// masked); the v^T copy is zero there.
template <bool F32, int D>
__device__ __forceinline__ void stage_async(const FwdArgs &A, unsigned char *buf, int64_t bh,
                                            int64_t t, bool k_only) {
    using SM = Smem<F32, D>;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int64_t ROWB = D * SM::ESZ;  // bytes per q/k/v row in memory
    // head base (uniform) + 32-bit offset of row `lane` of the tile (clamped)
    const int64_t hbase = bh * A.n * ROWB;
    const uint32_t koff = uint32_t(tile_row_src(bh, A.n, t, lane, ROWB, 0) - hbase);
    const unsigned char *kh = static_cast<const unsigned char *>(A.k) + hbase;
#pragma unroll
    for (int i = 0; i < SM::KCH / NWAVES; ++i) {
        const int c = w + NWAVES * i;
        g2lds16(kh + (koff + uint32_t(c * 16)), buf + c * 1024);
    }
    if (k_only) return;
    if constexpr (!F32) {
        // v^T rows d = lane + 64 grp, chunks of 8 keys
        const int64_t vbase = bh * D * A.n_pad * 2;
        const uint32_t voff = uint32_t(vt_src(bh, D, A.n_pad, t, lane, 0) - vbase);
        const uint32_t row64 = uint32_t(64 * A.n_pad * 2);
        const unsigned char *vh = reinterpret_cast<const unsigned char *>(A.vt) + vbase;
        constexpr int NI = SM::VCH * D / 64 / NWAVES;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int idx = w + NWAVES * i;  // (chunk, 64-row group)
            const int c = idx % SM::VCH, grp = idx / SM::VCH;
            g2lds16(vh + (voff + uint32_t(grp) * row64 + uint32_t(c * 16)),
                    buf + SM::k_bytes + (c * D + 64 * grp) * 16);
        }
    } else {
        const unsigned char *vh = static_cast<const unsigned char *>(A.v) + hbase;
#pragma unroll
        for (int i = 0; i < SM::KCH / NWAVES; ++i) {
            const int c = w + NWAVES * i;
            g2lds16(vh + (koff + uint32_t(c * 16)), buf + SM::k_bytes + c * 1024);
        }
    }
}

// Largest |k| over the staged key tile, keys below n only (float bits).
template <bool F32, int D>
__device__ __forceinline__ uint32_t tile_kbits(const FwdArgs &A, const unsigned char *buf,
                                               int64_t t) {
    using SM = Smem<F32, D>;
    uint32_t bits = 0;
    for (int u = threadIdx.x; u < SM::KCH * BK; u += NTHREADS) {
        if (t * BK + (u % BK) >= A.n) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(buf + u * 16);
        if constexpr (F32)
            bits = max(bits, absbits_f4(__builtin_bit_cast(float4, v)));
        else
            bits = max(bits, absbits_u4_bf16(v));
    }
    return bits;
}

// S^T for keys kb..kb+31 of the staged tile against the wave's 32 queries.
// Lane (qi, h), register r holds key kb + 8(r/4) + 4h + r%4 of query qi.
template <bool F32, int D>
__device__ __forceinline__ f32x16 s_block(const unsigned char *buf, int kb, int qi, int h,
                                          const typename Frag<F32, D>::type (&qf)[Frag<F32, D>::count]) {
    using SM = Smem<F32, D>;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    if constexpr (!F32) {
        const unsigned char *kp = buf + (h * BK + kb + qi) * 16;  // chunk 2s+h of row kb+qi
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kp + 2 * s * BK * 16);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], acc, 0, 0, 0);
        }
    } else {
        const unsigned char *kp = buf + (h * (D / 8) * BK + kb + qi) * 16;
#pragma unroll
        for (int t = 0; t < D / 8; ++t) {
            const float4 a = *reinterpret_cast<const float4 *>(kp + t * BK * 16);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qf[4 * t + 0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qf[4 * t + 1], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qf[4 * t + 2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qf[4 * t + 3], acc, 0, 0, 0);
        }
    }
    return acc;
}

// O^T += V^T W~^T for the 16 keys of chunk kc (registers 8kc..8kc+7 of the
// S^T block at kb): two accumulators, one for Re W~ and one for Im W~, that
// share the V operand.
template <bool F32, int D>
__device__ __forceinline__ void pv_chunk(const unsigned char *buf, int kb, int kc, int qi, int h,
                                         const float (&wre)[8], const float (&wim)[8],
                                         f32x16 (&ore)[D / 32], f32x16 (&oim)[D / 32]) {
    using SM = Smem<F32, D>;
    const unsigned char *vb = buf + SM::k_bytes;
    if constexpr (!F32) {
        bf16x8 bre, bim;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bre[e] = (__bf16)wre[e];
            bim[e] = (__bf16)wim[e];
        }
        // chunk (kb/8 + 2kc + h) of v^T row 32db + qi
        const unsigned char *vp = vb + (((kb >> 3) + 2 * kc + h) * D + qi) * 16;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vp + 32 * db * 16);
            ore[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bre, ore[db], 0, 0, 0);
            oim[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bim, oim[db], 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = 8 * kc + e;
            const int key = kb + 8 * (s / 4) + 4 * h + (s % 4);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int d = 32 * db + qi;
                const float a = *reinterpret_cast<const float *>(
                    vb + ((d >> 2) * BK + key) * 16 + (d & 3) * 4);
                ore[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, wre[e], ore[db], 0, 0, 0);
                oim[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, wim[e], oim[db], 0, 0, 0);
            }
        }
    }
}

// Lazy rescaling: the shift M only moves when a logit exceeds it by more than
// this many binary orders (weights stay <= 2^8 in between; the epilogue uses
// whatever shift was last applied, so the result is the same).
constexpr float kLazy = 8.0f;

template <bool F32, int D, bool QKZ>
__global__ __launch_bounds__(NTHREADS, F32 ? 1 : 2) void fwd_kernel(
    FwdArgs A, const double *__restrict__ tre, const double *__restrict__ tim,
    const double *__restrict__ tmm) {
    // (the key-tile products come as separate read-only arguments so that
    // their wave-uniform loads go through the scalar cache)
    using SM = Smem<F32, D>;
    using FR = Frag<F32, D>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *misc = reinterpret_cast<uint32_t *>(smem + SM::misc_off);
    // misc[2]: largest |q|; misc[3]: largest |k|

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, qi = lane & 31;
    // Work item of this workgroup.  Workgroups go round-robin to the 8 XCDs
    // (L mod 8); when the heads split evenly, XCD x takes heads x, x+8, ...
    // one at a time (its L2 then holds one head's keys and values), each
    // head's query tiles heaviest first.
    const int L = blockIdx.x;
    int64_t qt, bh;
    if ((A.BH & 7) == 0) {
        const int x = L & 7, j = L >> 3;
        bh = x + 8 * (j / A.n_qt);
        qt = A.n_qt - 1 - (j % A.n_qt);
    } else {
        qt = A.n_qt - 1 - L / A.BH;
        bh = L % A.BH;
    }
    const int64_t i0 = qt * BQ;
    const int64_t row = i0 + 32 * w + qi;
    const bool row_ok = row < A.n;
    const int64_t gbase = bh * A.n_pad;
    const int64_t t_diag0 = i0 / BK;            // first key tile of the query tile
    constexpr int NDIAG = BQ / BK;

    if (tid == 0) {
        misc[2] = 0;
        misc[3] = 0;
    }

    // ---- the tile schedule: off-diagonal tiles last to first while the
    // carried modulus is non-zero in float32, then the query tile's own tiles
    int64_t t_cur = t_diag0 > 0 ? t_diag0 - 1 : t_diag0 + NDIAG - 1;
    bool off_cur = t_diag0 > 0;
    double Cre = 1.0, Cim = 0.0, Cm = 1.0;  // carried gates: end of t_cur .. i0-1

    // side data of a tile, written by wave 0 into a buffer: T_j = C S_j
    // (off-diagonal) or the gates a_{j+1} (the query tile's own keys)
    auto write_side = [&](unsigned char *buf, int64_t t, bool off, double cr, double ci,
                          double cm, float g0, float g1, float g2) {
        float *sd = reinterpret_cast<float *>(buf + SM::side_off);
        if (off) {
            const int slot = perm64(tid);
            sd[slot] = (float)(cr * (double)g0 - ci * (double)g1);
            sd[BK + slot] = (float)(cr * (double)g1 + ci * (double)g0);
            const float rt = (float)(cm * (double)g2);
            sd[2 * BK + slot] = rt;
            const uint64_t dead = __ballot(rt == 0.0f);
            uint32_t *fl = reinterpret_cast<uint32_t *>(buf + SM::flag_off);
            if (tid == 0) {
                fl[0] = (uint32_t)(dead & 0xFFFFFFFFull) != 0u;
                fl[1] = (uint32_t)(dead >> 32) != 0u;
            }
        } else {
            sd[tid] = g0;
            sd[BK + tid] = g1;
            sd[2 * BK + tid] = g2;
        }
    };
    // gate data wave 0 needs for a tile's side data (one key per lane)
    auto load_side = [&](int64_t t, bool off, float &g0, float &g1, float &g2) {
        if (off) {
            const int64_t pos = gbase + t * BK + tid;
            g0 = A.s_re[pos];
            g1 = A.s_im[pos];
            g2 = A.s_m[pos];
        } else {
            const int64_t pos = t * BK + 1 + tid;  // a_{j+1} for key j = t*BK + tid
            const bool ok = pos < A.n;
            g0 = ok ? A.a_re[gbase + pos] : 1.0f;
            g1 = ok ? A.a_im[gbase + pos] : 0.0f;
            g2 = ok ? A.a_m[gbase + pos] : 1.0f;
        }
    };

    int cur = 0;
    stage_async<F32, D>(A, smem, bh, t_cur, false);
    if (tid < BK) {
        float g0, g1, g2;
        load_side(t_cur, off_cur, g0, g1, g2);
        write_side(smem, t_cur, off_cur, Cre, Cim, Cm, g0, g1, g2);
    }
    typename FR::type qf[FR::count];
    const uint32_t qbits = load_q<F32, D>(A, bh, row, row_ok, h, qf);

    // the modulus of the query tile's prefix product for this row: a row whose
    // prefix holds a closed gate sees no key before the query tile
    const bool row_live = !(A.p_m[gbase + row] == 0.0f);
    const bool wave_dead_rows = __any(!row_live);
    bool row_live_cur = row_live;  // rows gate the off-diagonal tiles only

    f32x16 ore[D / 32], oim[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ore[db][r] = 0.f;
            oim[db][r] = 0.f;
        }
    // shift of the live logits (log2 units), same in both halves; with qk = 0
    // every live logit is 0 and the shift is 0 throughout
    float M = QKZ ? 0.0f : -INFINITY;
    float z = 0.f;        // this lane's share of the normaliser
    uint32_t tiles_done = 0;

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    atomicMax(&misc[2], qbits);

    // Raw scores S of one S^T block (QKZ: qk = 0 never forms the product).
    // Logits are c*S in log2 units; c = qk log2(e)/sqrt(d) may be negative.
    const bool cpos = A.c > 0.0f;
    const float dead_s = cpos ? -INFINITY : INFINITY;  // a score whose logit is -inf
    auto scores = [&](const unsigned char *buf, int kb, float (&x)[16]) {
        if constexpr (!QKZ) {
            const f32x16 sc = s_block<F32, D>(buf, kb, qi, h, qf);
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = sc[r];
        }
    };
    // online max of the block's live logits, with lazy rescaling of O and z;
    // returns the shift to subtract (0 while a row has no live entry yet)
    auto update_max = [&](const float (&x)[16]) -> float {
        if constexpr (QKZ) {
            return 0.0f;  // every live logit is 0: the shift stays 0
        } else {
            float ts;
            if (cpos) {
                ts = x[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) ts = fmaxf(ts, x[r]);
                ts = fmaxf(ts, __shfl_xor(ts, 32));
            } else {
                ts = x[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) ts = fminf(ts, x[r]);
                ts = fminf(ts, __shfl_xor(ts, 32));
            }
            float t;
            {
#pragma clang fp contract(off)
                t = ts * A.c;  // the block's largest logit (-inf if none is live)
            }
            const bool grow = t > M + kLazy || (M == -INFINITY && t > M);
            if (__any(grow && M != -INFINITY)) {
                const float alpha =
                    (grow && M != -INFINITY) ? __builtin_amdgcn_exp2f(M - t) : 1.0f;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        ore[db][r] *= alpha;
                        oim[db][r] *= alpha;
                    }
                z *= alpha;
            }
            M = grow ? t : M;
            return (M == -INFINITY) ? 0.0f : M;
        }
    };
    // exponentials e = 2^(c S - M), normaliser and the two W~ V products of
    // one 16-key chunk; `live` (QKZ only) marks the entries that are not masked
    auto chunk = [&](const unsigned char *buf, int kb, int kc, const float (&x)[16], float msub,
                     const float (&fre)[8], const float (&fim)[8], const float (&fm)[8],
                     bool all_live) {
        float wre[8], wim[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float ex;
            if constexpr (QKZ)
                ex = (all_live || (fm[e] > 0.0f && row_live_cur)) ? 1.0f : 0.0f;
            else
                ex = __builtin_amdgcn_exp2f(fmaf(x[8 * kc + e], A.c, -msub));
            z += ex * fm[e];
            wre[e] = ex * fre[e];
            wim[e] = ex * fim[e];
        }
        pv_chunk<F32, D>(buf, kb, kc, qi, h, wre, wim, ore, oim);
    };

    // ---- key tiles wholly before the query tile: G = S_j C_t P_i ----------
    while (off_cur) {
        unsigned char *buf = smem + cur * SM::buf_bytes;
        unsigned char *nbuf = smem + (cur ^ 1) * SM::buf_bytes;
        const float *side = reinterpret_cast<const float *>(buf + SM::side_off);
        // the next tile, and its asynchronous copy
        const int64_t tp = bh * A.n_kt + t_cur;
        const double are = tre[tp], aim = tim[tp], am = tmm[tp];
        const double nCre = uniform_f64(are * Cre - aim * Cim);
        const double nCim = uniform_f64(are * Cim + aim * Cre);
        const double nCm = uniform_f64(am * Cm);
        // every earlier key is dead once the carried modulus is 0 in float32
        const bool off_nxt = t_cur > 0 && (float)nCm != 0.0f;
        const int64_t t_nxt = off_nxt ? t_cur - 1 : t_diag0 + NDIAG - 1;
        stage_async<F32, D>(A, nbuf, bh, t_nxt, false);
        float g0 = 0.f, g1 = 0.f, g2 = 0.f;
        if (tid < BK) load_side(t_nxt, off_nxt, g0, g1, g2);

        ++tiles_done;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int kb = 32 * blk;
            float x[16];
            scores(buf, kb, x);
            const bool masked = wave_dead_rows ||
                                reinterpret_cast<const uint32_t *>(buf + SM::flag_off)[blk] != 0u;
            if (!QKZ && masked) {
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const float4 m0 =
                        *reinterpret_cast<const float4 *>(side + 2 * BK + kb + 16 * kc + 8 * h);
                    const float4 m1 =
                        *reinterpret_cast<const float4 *>(side + 2 * BK + kb + 16 * kc + 8 * h + 4);
                    const float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        x[8 * kc + e] = (mm[e] > 0.0f && row_live) ? x[8 * kc + e] : dead_s;
                }
            }
            const float msub = update_max(x);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                float fre[8], fim[8], fm[8];
                const int s0 = kb + 16 * kc + 8 * h;
#pragma unroll
                for (int e = 0; e < 8; e += 4) {
                    const float4 a = *reinterpret_cast<const float4 *>(side + s0 + e);
                    const float4 b = *reinterpret_cast<const float4 *>(side + BK + s0 + e);
                    const float4 c = *reinterpret_cast<const float4 *>(side + 2 * BK + s0 + e);
                    fre[e] = a.x; fre[e + 1] = a.y; fre[e + 2] = a.z; fre[e + 3] = a.w;
                    fim[e] = b.x; fim[e + 1] = b.y; fim[e + 2] = b.z; fim[e + 3] = b.w;
                    fm[e] = c.x; fm[e + 1] = c.y; fm[e + 2] = c.z; fm[e + 3] = c.w;
                }
                chunk(buf, kb, kc, x, msub, fre, fim, fm, !masked);
            }
        }

        if (tid < BK) write_side(nbuf, t_nxt, off_nxt, nCre, nCim, nCm, g0, g1, g2);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        Cre = nCre;
        Cim = nCim;
        Cm = nCm;
        t_cur = t_nxt;
        off_cur = off_nxt;
        cur ^= 1;
        if (!off_cur) {
            // leaving the off-diagonal tiles: rotate by the prefix product P_i
            const float Pre = A.p_re[gbase + row], Pim = A.p_im[gbase + row];
            const float Pm = A.p_m[gbase + row];
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float xr = ore[db][r], xi = oim[db][r];
                    ore[db][r] = Pre * xr - Pim * xi;
                    oim[db][r] = Pre * xi + Pim * xr;
                }
            z *= Pm;
        }
    }

    // ---- the query tile's own keys: explicit G_ij, last key first ---------
    row_live_cur = true;
    float gre = 0.f, gim = 0.f, gm = 0.f;  // running G_{row,j}, R_{row,j}
    uint32_t kbits = 0;
    while (true) {
        unsigned char *buf = smem + cur * SM::buf_bytes;
        unsigned char *nbuf = smem + (cur ^ 1) * SM::buf_bytes;
        const float *side = reinterpret_cast<const float *>(buf + SM::side_off);
        const bool more = t_cur > t_diag0;
        float g0 = 0.f, g1 = 0.f, g2 = 0.f;
        if (more) {
            stage_async<F32, D>(A, nbuf, bh, t_cur - 1, false);
            if (tid < BK) load_side(t_cur - 1, false, g0, g1, g2);
        }
        kbits = max(kbits, tile_kbits<F32, D>(A, buf, t_cur));
#pragma unroll
        for (int blk = 1; blk >= 0; --blk) {
            const int cidx = int((t_cur - t_diag0) * (BK / 32)) + blk;
            if (cidx > w) continue;  // wholly above this wave's rows
            const int kb = 32 * blk;
            const int dpos = int(row - (t_cur * BK + kb));  // 0..31 on the block's diagonal
            // pass 1: modulus R_{row,j} of the 16 keys this lane holds
            float Gm[16];
            const float gre0 = gre, gim0 = gim;
#pragma unroll
            for (int jj = 31; jj >= 0; --jj) {
                const float nm = gm * side[2 * BK + kb + jj];
                gm = (jj == dpos) ? 1.0f : nm;
                if (h == ((jj >> 2) & 1)) Gm[4 * (jj >> 3) + (jj & 3)] = gm;
            }
            float x[16];
            scores(buf, kb, x);
            if constexpr (!QKZ) {
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = (Gm[r] > 0.0f) ? x[r] : dead_s;
            }
            const float msub = update_max(x);
            // pass 2: G_{row,j} chunk by chunk, keys 31..16 then 15..0
            gre = gre0;
            gim = gim0;
#pragma unroll
            for (int kc = 1; kc >= 0; --kc) {
                float fre[8], fim[8], fm[8];
#pragma unroll
                for (int jj = 16 * kc + 15; jj >= 16 * kc; --jj) {
                    const float dr = side[kb + jj], di = side[BK + kb + jj];
                    const float nr = gre * dr - gim * di;
                    const float ni = gre * di + gim * dr;
                    const bool diag = (jj == dpos);
                    gre = diag ? 1.0f : nr;
                    gim = diag ? 0.0f : ni;
                    if (h == ((jj >> 2) & 1)) {
                        const int e = 4 * ((jj - 16 * kc) >> 3) + (jj & 3);
                        fre[e] = gre;
                        fim[e] = gim;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) fm[e] = Gm[8 * kc + e];
                chunk(buf, kb, kc, x, msub, fre, fim, fm, false);
            }
        }
        if (!more) break;
        if (tid < BK) write_side(nbuf, t_cur - 1, false, 0.0, 0.0, 0.0, g0, g1, g2);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        t_cur -= 1;
        cur ^= 1;
    }
    atomicMax(&misc[3], kbits);

    // ---- epilogue: O *= exp2((1-beta) M) z^-beta -------------------------
    const float zt = z + __shfl_xor(z, 32);
    float f;
    if (A.beta_mode == 1)
        f = 1.0f / zt;
    else if (A.beta_mode == 0)
        f = exp2f(M);
    else
        f = exp2f(A.one_minus_beta * M - A.beta * log2f(zt));
    if (row_ok) {
        float *orp = A.o_re + (bh * A.n + row) * D;
        float *oip = A.o_im + (bh * A.n + row) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * db + 8 * g4 + 4 * h;
                float4 vr, vi;
                vr.x = ore[db][4 * g4 + 0] * f;
                vr.y = ore[db][4 * g4 + 1] * f;
                vr.z = ore[db][4 * g4 + 2] * f;
                vr.w = ore[db][4 * g4 + 3] * f;
                vi.x = oim[db][4 * g4 + 0] * f;
                vi.y = oim[db][4 * g4 + 1] * f;
                vi.z = oim[db][4 * g4 + 2] * f;
                vi.w = oim[db][4 * g4 + 3] * f;
                *reinterpret_cast<float4 *>(orp + d0) = vr;
                *reinterpret_cast<float4 *>(oip + d0) = vi;
            }
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t qb = misc[2], kb = misc[3];
        A.qstat[bh * A.n_qt + qt] = qb;
        A.kstat[bh * A.n_qt + qt] = kb;
        if (qb >= kInfBits || kb >= kInfBits) A.status[0] = kNonFinite;
        atomicAdd(&A.counters[0], tiles_done);
    }
}

// --------------------------------------------------------------------------
// Refusal of an overflowing logit (section "Evaluation and refusals").  The
// extrema of |q| and |k| that fwd_kernel recorded bound every logit by
// |c| d max|q| max|k|; only a head where that bound reaches the float32 range
// recomputes its logits (with the same MFMA code and scale as fwd_kernel) and
// checks every j <= i.
template <bool F32, int D>
__global__ __launch_bounds__(NTHREADS) void logit_check_kernel(FwdArgs A) {
    using FR = Frag<F32, D>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int go;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, qi = lane & 31;
    const int L = blockIdx.x;
    const int64_t qt = A.n_qt - 1 - L / A.BH;
    const int64_t bh = L % A.BH;
    if (tid == 0) {
        uint32_t qm = 0, km = 0;
        for (int t = 0; t < A.n_qt; ++t) {
            qm = max(qm, A.qstat[bh * A.n_qt + t]);
            km = max(km, A.kstat[bh * A.n_qt + t]);
        }
        const double bound = fabs((double)A.c) * (double)D * (double)__uint_as_float(qm) *
                             (double)__uint_as_float(km) * 1.01;
        go = !(bound < 3.0e38);
    }
    __syncthreads();
    if (!go) return;
    const int64_t i0 = qt * BQ;
    const int64_t row = i0 + 32 * w + qi;
    const bool row_ok = row < A.n;
    typename FR::type qf[FR::count];
    load_q<F32, D>(A, bh, row, row_ok, h, qf);
    bool bad = false;
    for (int64_t t = 0; t < (i0 + BQ) / BK; ++t) {
        __syncthreads();
        stage_async<F32, D>(A, smem, bh, t, true);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const f32x16 s = s_block<F32, D>(smem, 32 * blk, qi, h, qf);
            {
#pragma clang fp contract(off)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t j = t * BK + 32 * blk + 8 * (r / 4) + 4 * h + (r % 4);
                    const float x = s[r] * A.c;
                    if (row_ok && j <= row && j < A.n && !isfinite(x)) bad = true;
                }
            }
        }
    }
    if (__any(bad) && lane == 0) A.status[0] = kNonFinite;
}

template <bool F32, int D>
int launch_typed(const Problem &P, hipStream_t st, hipEvent_t const *marks) {
    using SM = Smem<F32, D>;
    const Layout &L = P.L;
    unsigned char *ws = P.ws;
    uint32_t *counters = reinterpret_cast<uint32_t *>(ws + L.counters);
    if (marks) (void)hipEventRecord(marks[0], st);
    auto fptr = [&](int i) { return reinterpret_cast<float *>(ws + L.gate[i]); };
    auto dptr = [&](int i) { return reinterpret_cast<double *>(ws + L.tile[i]); };
    const int BH = (int)L.BH;

    if constexpr (!F32) {
        uint16_t *vt = reinterpret_cast<uint16_t *>(ws + L.vt);
        if (P.v_f32)
            hipLaunchKernelGGL((vt_kernel<D, true>), dim3(BH * L.n_kt), dim3(256), 0, st, P.v, vt,
                               L.n, L.n_pad, (int)L.n_kt, P.status, counters);
        else
            hipLaunchKernelGGL((vt_kernel<D, false>), dim3(BH * L.n_kt), dim3(256), 0, st, P.v, vt,
                               L.n, L.n_pad, (int)L.n_kt, P.status, counters);
    } else {
        hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, st, P.status, counters);
    }

    GatesArgs G;
    G.u = P.u;
    G.theta = P.theta;
    G.g = P.g;
    G.n = L.n;
    G.n_pad = L.n_pad;
    G.n_qt = (int)L.n_qt;
    G.n_kt = (int)L.n_kt;
    G.a_re = fptr(0);
    G.a_im = fptr(1);
    G.a_m = fptr(2);
    G.s_re = fptr(3);
    G.s_im = fptr(4);
    G.s_m = fptr(5);
    G.p_re = fptr(6);
    G.p_im = fptr(7);
    G.p_m = fptr(8);
    G.t_re = dptr(0);
    G.t_im = dptr(1);
    G.t_m = dptr(2);
    G.status = P.status;
    hipLaunchKernelGGL(gates_kernel, dim3(BH * L.n_qt), dim3(64), 0, st, G);

    FwdArgs F;
    F.q = P.q;
    F.k = P.k;
    F.v = P.v;
    F.vt = reinterpret_cast<const uint16_t *>(ws + L.vt);
    F.a_re = G.a_re;
    F.a_im = G.a_im;
    F.a_m = G.a_m;
    F.s_re = G.s_re;
    F.s_im = G.s_im;
    F.s_m = G.s_m;
    F.p_re = G.p_re;
    F.p_im = G.p_im;
    F.p_m = G.p_m;
    F.t_re = G.t_re;
    F.t_im = G.t_im;
    F.t_m = G.t_m;
    F.o_re = P.o_re;
    F.o_im = P.o_im;
    F.qstat = reinterpret_cast<uint32_t *>(ws + L.qstat);
    F.kstat = reinterpret_cast<uint32_t *>(ws + L.kstat);
    F.counters = counters;
    F.status = P.status;
    F.n = L.n;
    F.n_pad = L.n_pad;
    F.n_qt = (int)L.n_qt;
    F.n_kt = (int)L.n_kt;
    F.BH = BH;
    F.c = P.c;
    F.beta = P.beta;
    F.one_minus_beta = 1.0f - P.beta;
    F.beta_mode = P.beta_mode;
    F.qk_zero = P.qk_zero ? 1 : 0;
    const size_t shm = SM::bytes;
    if (shm > 65536) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_kernel<F32, D, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_kernel<F32, D, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&logit_check_kernel<F32, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    }
    if (marks) (void)hipEventRecord(marks[1], st);
    if (P.qk_zero)
        hipLaunchKernelGGL((fwd_kernel<F32, D, true>), dim3(BH * L.n_qt), dim3(NTHREADS), shm, st,
                           F, G.t_re, G.t_im, G.t_m);
    else
        hipLaunchKernelGGL((fwd_kernel<F32, D, false>), dim3(BH * L.n_qt), dim3(NTHREADS), shm,
                           st, F, G.t_re, G.t_im, G.t_m);
    if (marks) (void)hipEventRecord(marks[2], st);
    if (!P.qk_zero)
        hipLaunchKernelGGL((logit_check_kernel<F32, D>), dim3(BH * L.n_qt), dim3(NTHREADS), shm,
                           st, F);
    if (marks) (void)hipEventRecord(marks[3], st);
    return (int)hipGetLastError();
}

}  // namespace

int launch_forward(const Problem &P, void *stream, void *const *marks) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t const *ev = reinterpret_cast<hipEvent_t const *>(marks);
    const bool f32 = !P.L.bf16_path;
    if (P.L.d == 64)
        return f32 ? launch_typed<true, 64>(P, st, ev) : launch_typed<false, 64>(P, st, ev);
    return f32 ? launch_typed<true, 128>(P, st, ev) : launch_typed<false, 128>(P, st, ev);
}

}  // namespace resolvent
