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
// the product of every gate between the end of tile t and i0 (the product of
// the whole-tile products, accumulated in f64 as the key tiles are visited
// backwards from the diagonal), and P_i the inclusive prefix product inside
// the query tile.  P_i is applied once to the accumulators when the loop
// reaches the query tile's own keys; those keys use G_ij formed explicitly
// by a running product per row, multiplying a_i, a_{i-1}, ..., a_{j+1} in the
// order the page's "Rust API" section fixes.
//
// Kernels, in launch order on the caller's stream:
//   prep_kernel                      status := OK; blend + gate in f64 and the
//                                    in-tile scans; fp32 values on the bf16
//                                    path rounded to bf16
//   schedule_kernel                  key tiles each query tile visits
//   fwd_pad_kernel / fwd_kernel      the fused forward (bf16 / fp32 MFMA); the
//                                    carried products C_t are formed in it
//   logit_check_(pad_)kernel         exact logit-overflow refusal, only for
//                                    heads whose |q|,|k| extrema allow one
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
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
// Waves 0 .. NCOPY-1 issue the tile copies (all of them: each wave's share
// of a tile is small enough to fit the slack after its matrix step).
constexpr int NCOPY = NWAVES;

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
// x f for the epilogue's scale: an exactly zero accumulator stays (signed)
// zero when f overflows to inf (a zero lane of G stays 0, never NaN).
__device__ __forceinline__ float scale_keep_zero(float x, float f) { return x == 0.0f ? x : x * f; }

// Largest value over the wave, returned uniform: four DPP steps give every
// row of 16 lanes its maximum, four lane reads combine the rows.  (An LDS
// atomic of a per-lane value otherwise becomes a 64-step scalar loop.)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0xB1, 0xF, 0xF, false)));
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x4E, 0xF, 0xF, false)));
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x124, 0xF, 0xF, false)));
    v = max(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x128, 0xF, 0xF, false)));
    const uint32_t a = max(uint32_t(__builtin_amdgcn_readlane(int(v), 0)),
                           uint32_t(__builtin_amdgcn_readlane(int(v), 16)));
    const uint32_t b = max(uint32_t(__builtin_amdgcn_readlane(int(v), 32)),
                           uint32_t(__builtin_amdgcn_readlane(int(v), 48)));
    return max(a, b);
}

__device__ __forceinline__ uint32_t absbits_f4(float4 v) {
    uint32_t a = max(__float_as_uint(v.x) & 0x7FFFFFFFu, __float_as_uint(v.y) & 0x7FFFFFFFu);
    uint32_t b = max(__float_as_uint(v.z) & 0x7FFFFFFFu, __float_as_uint(v.w) & 0x7FFFFFFFu);
    return max(a, b);
}

// --------------------------------------------------------------------------
// Status and counter clear (before the gates alone, which the chain-corner
// scan runs).
__global__ void clear_status_kernel(int32_t *status, uint32_t *counters) {
    if (threadIdx.x == 0) status[0] = 0;
    if (threadIdx.x < 2) counters[threadIdx.x] = 0;
}

// fp32 values on the bf16 path: v rounded to bf16 once, row-major as v
// ([k/v head][key][channel]), eight values a thread (index i of count8).
__device__ __forceinline__ void v16_convert(const float *__restrict__ v, uint16_t *__restrict__ v16,
                                            int64_t count8, int64_t i) {
    if (i >= count8) return;
    const float4 f0 = *reinterpret_cast<const float4 *>(v + 8 * i);
    const float4 f1 = *reinterpret_cast<const float4 *>(v + 8 * i + 4);
    const float fs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)fs[2 * e]);
        const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)fs[2 * e + 1]);
        o[e] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4 *>(v16 + 8 * i) = make_uint4(o[0], o[1], o[2], o[3]);
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
    int64_t ldu;  // positions between heads in u, theta (>= n)
    int n_qt, n_kt;
    int64_t BH;
    float *a_re, *a_im, *a_m, *s_re, *s_im, *s_m, *p_re, *p_im, *p_m;
    double *t_re, *t_im, *t_m;
    double *t4;  // (A_re, A_im, A_m, 0) per key tile
    int32_t *status;
};

__device__ __forceinline__ void cmul_d(double xr, double xi, double yr, double yi, double &r,
                                       double &i) {
    r = xr * yr - xi * yi;
    i = xr * yi + xi * yr;
}

// One query tile qt of head bh on one wave (lane 0..63); returns whether this
// lane saw a refused input.
__device__ __forceinline__ bool gates_tile(const GatesArgs &A, int64_t bh, int64_t qt, int lane) {
#pragma clang fp contract(off)
    constexpr int PPL = BQ / 64;
    constexpr int SEG = BK / PPL;  // lanes per key tile
    const int64_t p0 = qt * BQ + PPL * lane;
    double ar[PPL], ai[PPL], am[PPL];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < PPL; ++e) {
        const int64_t p = p0 + e;
        if (p < A.n) {
            const float uu = A.u[bh * A.ldu + p], tt = A.theta[bh * A.ldu + p];
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
        double *t4 = A.t4 + 4 * (bh * A.n_kt + kt);
        t4[0] = xr;
        t4[1] = xi;
        t4[2] = xm;
        t4[3] = 0.0;
    }
    return bad;
}

// One wave per query tile.
__global__ __launch_bounds__(64) void gates_kernel(GatesArgs A) {
    if (gates_tile(A, blockIdx.x / A.n_qt, blockIdx.x % A.n_qt, threadIdx.x))
        A.status[0] = kNonFinite;
}

// The forward pass's first launch: clears the status word and the counters
// (block 0), runs the gates of four query tiles per block in blocks
// [0, ngb) -- a refusal is noted in gbad[query tile], always written, which
// schedule_kernel folds into the status word -- and (bf16 path, fp32 values)
// rounds v to bf16 in the blocks after them, 2048 values a block.
template <bool VCONV>
__global__ __launch_bounds__(256) void prep_kernel(GatesArgs G, int ngb, int32_t *__restrict__ gbad,
                                                   const float *__restrict__ v,
                                                   uint16_t *__restrict__ v16, int64_t count8,
                                                   uint32_t *__restrict__ counters) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0) G.status[0] = 0;
    if (blockIdx.x == 0 && tid < 16) counters[tid] = 0;
    if ((int)blockIdx.x < ngb) {
        const int64_t tq = 4 * int64_t(blockIdx.x) + (tid >> 6);  // query tile, all heads
        if (tq < G.BH * G.n_qt) {
            const bool bad = gates_tile(G, tq / G.n_qt, tq % G.n_qt, tid & 63);
            const bool any_bad = __any(bad);
            if ((tid & 63) == 0) gbad[tq] = any_bad ? 1 : 0;
        }
    } else if constexpr (VCONV) {
        v16_convert(v, v16, count8, 256 * (int64_t(blockIdx.x) - ngb) + tid);
    }
}

// --------------------------------------------------------------------------
// Fused forward.
struct FwdArgs {
    const void *q, *k, *v;
    const uint16_t *v16;  // bf16 path: the values in bf16, row-major as v
    const float *a_re, *a_im, *a_m, *s_re, *s_im, *s_m, *p_re, *p_im, *p_m;
    const double *t_re, *t_im, *t_m;
    const double *t4;     // (A_re, A_im, A_m, 0) per key tile [BH][n_kt]
    const float *gates;   // gate plane 0; plane k starts `plane` floats later
    int64_t plane;
    float *o_re, *o_im;
    uint32_t *qstat, *kstat, *counters;
    uint32_t *queues;  // bf16 path: the work queues' counters (cleared by prep_kernel)
    int nq, order;     // number of queues (1 or 8), item order inside a queue (queue_item)
    int q0;            // order 2: the light query tiles, qt < q0
    const int32_t *noff;
    int32_t *status;
    int64_t n, n_pad;
    int n_qt, n_kt, BH;
    int H, group;  // query heads per batch entry; query heads per k/v head
    float c, beta, one_minus_beta;
    int beta_mode, qk_zero;
};

// The k/v head that query head bh (= b H + h) reads: b H/group + h/group.
// (Args: FwdArgs, or FwdArgs read in place from the argument segment.)
template <typename Args>
__device__ __forceinline__ int64_t kv_head(const Args &A, int64_t bh) {
    return (bh / A.H) * (A.H / A.group) + (bh % A.H) / A.group;
}

// Shared-memory plan of the fp32 path: NBUF buffers, each holding one key
// tile K [BK][D] and its values V [BK][DV], per-key side data (the carried
// gate factor T_j = C*S_j with its modulus for tiles before the query tile;
// the gates a_{j+1} for the query tile's own keys) and the raw in-tile suffix
// products S_j it is formed from.  Tiles are 16-byte-chunk-major: chunk c of
// row r sits at (c * BK + r) * 16 (one wave instruction copies one chunk of
// the 64 rows).  Buffers start on 256-byte boundaries.
template <int D, int DV = D>
struct Smem {
    static constexpr int KCH = D * 4 / 16;    // 16-byte chunks per K row
    static constexpr int VINS = DV * 4 / 16;  // chunks per V row = V copy instructions per tile
    static constexpr size_t k_bytes = size_t(KCH) * BK * 16;
    static constexpr size_t v_bytes = size_t(VINS) * BK * 16;
    static constexpr size_t side_off = k_bytes + v_bytes;
    // side data: 3 x BK floats; raw: S_j as 3 x BK floats and the product of
    // the tile's gates (A_re, A_im, A_m, 0) as doubles; then 2 flag words
    // (32-key block b of the staged tile holds a dead column)
    static constexpr size_t raw_off = side_off + 3 * BK * sizeof(float);
    static constexpr size_t tprod_off = raw_off + 3 * BK * sizeof(float);
    static constexpr size_t flag_off = tprod_off + 4 * sizeof(double);
    static constexpr size_t buf_bytes = (flag_off + 16 + 255) / 256 * 256;
    // four buffers keep two tiles in flight while two are read, when they
    // fit into the 160 KB of LDS (d = dv = 128 takes two)
    static constexpr int NBUF = 4 * buf_bytes + 64 <= 160 * 1024 ? 4 : 2;
    static constexpr size_t misc_off = NBUF * buf_bytes;
    // the running carried product of the landings (3 doubles)
    static constexpr size_t carry_off = misc_off + 8 * sizeof(uint32_t);
    static constexpr size_t bytes = carry_off + 4 * sizeof(double);
    static_assert(KCH % NCOPY == 0 && VINS % NCOPY == 0, "whole wave copies");
};

template <bool F32, int D>
struct Frag {
    using type = typename std::conditional<F32, float, bf16x8>::type;
    static constexpr int count = F32 ? D / 2 : D / 16;
};

typedef __attribute__((address_space(3))) void lds_void;

// A wave-uniform pointer kept in scalar registers (also keeps the compiler
// from folding a per-lane offset into it and hoisting 64-bit lane addresses).
template <typename T>
__device__ __forceinline__ const T *uniform_ptr(const T *p) {
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(b >> 32));
    return reinterpret_cast<const T *>((uint64_t(hi) << 32) | lo);
}

// The lane index, computed where it is used: the compiler can neither hoist
// nor merge the asm statement, so per-lane copy offsets derived from it are
// recomputed inside the loop instead of held in registers across it.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// LDS byte address of a pointer into the workgroup's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p) {
    return (uint32_t)(uintptr_t)(lds_void *)(p);
}

// Direct global->LDS copy of 16 bytes per lane: lane L reads base + off and
// writes LDS address lds + 16 L; base and lds (a byte address) are
// wave-uniform.  Written as
// inline assembly so that the compiler does not track it as an LDS store: its
// aliasing rules would otherwise hold every later LDS read of any buffer until
// the copy lands.  Readers wait for the copy explicitly (wait_vmcnt() and a
// barrier).  m0 carries the LDS address and is restored afterwards.
__device__ __forceinline__ void g2lds16(const unsigned char *base_, uint32_t off, uint32_t lds) {
    const unsigned char *base = uniform_ptr(base_);
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(la)
        : "memory");
}

// The same for 4 bytes per lane (lane L writes lds + 4 L).
__device__ __forceinline__ void g2lds4(const unsigned char *base_, uint32_t off, uint32_t lds) {
    const unsigned char *base = uniform_ptr(base_);
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(la)
        : "memory");
}

// 16 bytes in each of lanes 0 and 1 (lane L reads base + off and writes
// lds + 16 L; the other lanes are masked off for the one instruction and
// restored).
__device__ __forceinline__ void g2lds16x2(const unsigned char *base_, uint32_t off, uint32_t lds) {
    const unsigned char *base = uniform_ptr(base_);
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds);
    uint32_t saved;
    uint64_t ex;
    asm volatile(
        "s_mov_b64 %1, exec\n\t"
        "s_mov_b64 exec, 3\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_mov_b64 exec, %1"
        : "=&s"(saved), "=&s"(ex)
        : "v"(off), "s"(base), "s"(la)
        : "memory");
}

// s_waitcnt vmcnt(N) for a compile-time N (gfx9 encoding: low bits 3:0,
// high bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// Workgroup barrier that waits for the wave's own LDS operations only, not
// for its copies in flight (the __syncthreads() of HIP also waits on vmcnt).
// Keeps the computation of v before this point: the empty asm statement reads
// it, and volatile asm statements keep their order.  (lds_barrier orders
// memory operations only; arithmetic whose result is first used after a
// barrier may otherwise be sunk past it, into the next phase.)
template <typename T>
__device__ __forceinline__ void settle(const T &v) {
    asm volatile("" ::"v"(v));
}

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Query fragment (B operand of S^T = K Q^T) for the lane's row; returns the
// largest |q| as float bits.
template <bool F32, int D, typename Args>
__device__ __forceinline__ uint32_t load_q(const Args &A, int64_t bh, int64_t row, bool row_ok,
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
// k_only) into buffer buf (an LDS byte address), fp32 path.  Wave w < NCOPY
// copies chunks w, w+NCOPY, ...: lane L fetches 16 bytes of row L; other
// waves copy nothing.  Keys past n repeat key n-1 (their entries are masked).
// kh, vh: this head's rows of k and of v, wave-uniform.
template <int D, int DV>
__device__ __forceinline__ void stage_async(const FwdArgs &A, uint32_t buf,
                                            const unsigned char *kh, const unsigned char *vh,
                                            int t, bool k_only, int w) {
    using SM = Smem<D, DV>;
    const int lane = fresh_lane();
    if (w >= NCOPY) return;
    const uint32_t koff = tile_row_off(A.n, t, lane, D * 4);
#pragma unroll
    for (int i = 0; i < SM::KCH / NCOPY; ++i) {
        const int c = w + NCOPY * i;
        g2lds16(kh, koff + uint32_t(c * 16), buf + uint32_t(c * 1024));
    }
    if (k_only) return;
    const uint32_t voff = tile_row_off(A.n, t, lane, DV * 4);
#pragma unroll
    for (int i = 0; i < SM::VINS / NCOPY; ++i) {
        const int c = w + NCOPY * i;
        g2lds16(vh, voff + uint32_t(c * 16), buf + uint32_t(SM::k_bytes + c * 1024));
    }
}

// Bases of the tile copies for k/v head kvh (wave-uniform): its rows of k,
// and of the bf16 values (bf16 path) or v (fp32 path).
template <bool F32, int D, int DV, typename Args>
__device__ __forceinline__ void head_bases(const Args &A, int64_t kvh,
                                           const unsigned char *&kh, const unsigned char *&vh) {
    constexpr int64_t ROWB = D * (F32 ? 4 : 2);
    kh = uniform_ptr(static_cast<const unsigned char *>(A.k) + kvh * A.n * ROWB);
    if constexpr (!F32)
        vh = uniform_ptr(reinterpret_cast<const unsigned char *>(A.v16) + kvh * A.n * (DV * 2));
    else
        vh = uniform_ptr(static_cast<const unsigned char *>(A.v) + kvh * A.n * (DV * 4));
}

// Largest |k| (float bits) over the K bytes of key tile t that wave w copied
// itself (stage_async: its copy instructions j = w, w+NCOPY, ... wrote LDS
// offset 1024 j + 16 lane).  A row past the sequence end holds a copy of key
// n-1.  Valid once the wave's own copies have landed.
template <int D>
__device__ __forceinline__ uint32_t own_kbits(const unsigned char *buf, int w) {
    using SM = Smem<D>;
    uint32_t bits = 0;
    if (w < NCOPY) {
#pragma unroll
        for (int i = 0; i < SM::KCH / NCOPY; ++i) {
            const int j = w + NCOPY * i;
            const uint4 v = *reinterpret_cast<const uint4 *>(buf + (j * 64 + fresh_lane()) * 16);
            bits = max(bits, absbits_f4(__builtin_bit_cast(float4, v)));
        }
    }
    return bits;
}

// S^T for keys kb..kb+31 of the staged tile against the wave's 32 queries
// (fp32 path).  Lane (qi, h), register r holds key kb + 8(r/4) + 4h + r%4 of
// query qi.
template <int D>
__device__ __forceinline__ f32x16 s_block(const unsigned char *buf, int kb, int qi, int h,
                                          const float (&qf)[D / 2]) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const unsigned char *kp = buf + (h * (D / 8) * BK + kb + qi) * 16;
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
        const float4 a = *reinterpret_cast<const float4 *>(kp + t * BK * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qf[4 * t + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qf[4 * t + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qf[4 * t + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qf[4 * t + 3], acc, 0, 0, 0);
    }
    return acc;
}

// O^T += V^T W~^T for the 16 keys of chunk kc of the 32-key block at kb
// (fp32 path), W~ as 8 floats per lane.
template <int D, int DV>
__device__ __forceinline__ void pv_chunk_f32(const unsigned char *buf, int kb, int kc, int qi,
                                             int h, const float (&wre)[8], const float (&wim)[8],
                                             f32x16 (&ore)[DV / 32], f32x16 (&oim)[DV / 32]) {
    const unsigned char *vb = buf + Smem<D>::k_bytes;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int s = 8 * kc + e;
        const int key = kb + 8 * (s / 4) + 4 * h + (s % 4);
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) {
            const int d = 32 * db + qi;
            const float a =
                *reinterpret_cast<const float *>(vb + ((d >> 2) * BK + key) * 16 + (d & 3) * 4);
            ore[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, wre[e], ore[db], 0, 0, 0);
            oim[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, wim[e], oim[db], 0, 0, 0);
        }
    }
}

// Lazy rescaling: the shift M only moves when a logit exceeds it by more than
// this many binary orders (weights stay <= 2^8 in between; the epilogue uses
// whatever shift was last applied, so the result is the same).
constexpr float kLazy = 8.0f;

// --------------------------------------------------------------------------
// Visit count per query tile.  The key tiles before query tile qt are
// visited last to first; visit s carries
//     C_s = A_{t0-1} A_{t0-2} ... A_{t0-s}   (C_0 = 1; A_t the whole-tile
// product of key tile t, t0 the query tile's first key tile), the gate
// product from the end of the visited tile up to the query tile.  C is
// accumulated in f64 in visiting order (fwd_kernel repeats this recurrence
// as it lands the tiles); the visits stop after the tile whose product makes
// the modulus of C zero in float32: every key before it sits behind a closed
// gate (section "Object") and is exactly dead.  One wave per query tile: the
// lanes fetch 64 tile products at a time and the product is accumulated in
// order.
__global__ __launch_bounds__(64) void schedule_kernel(const double *__restrict__ tre,
                                                      const double *__restrict__ tim,
                                                      const double *__restrict__ tmm, int n_kt,
                                                      int n_qt, int32_t *__restrict__ noff,
                                                      uint32_t *__restrict__ qstat,
                                                      uint32_t *__restrict__ kstat,
                                                      const int32_t *__restrict__ gbad,
                                                      int32_t *__restrict__ status) {
#pragma clang fp contract(off)
    const int L = blockIdx.x;
    if (threadIdx.x == 0 && gbad[L] != 0) status[0] = kNonFinite;  // the query tile's gates
    const int64_t bh = L / n_qt;
    const int qt = L % n_qt;
    const int lane = threadIdx.x;
    const int t0 = qt * (BQ / BK);  // first key tile of the query tile
    const double *pr = tre + bh * n_kt, *pi = tim + bh * n_kt, *pm = tmm + bh * n_kt;
    double cr = 1.0, ci = 0.0, cm = 1.0;
    int result = t0;  // every tile before the query tile
    auto lane_f64 = [](double x, int s) {
        const uint64_t bits = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(bits), s);
        const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(bits >> 32), s);
        return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
    };
    for (int base = 0; base < t0; base += 64) {
        const bool valid = base + lane < t0;
        const int t = t0 - 1 - (base + lane);
        const double ar = valid ? pr[t] : 1.0, ai = valid ? pi[t] : 0.0,
                     am = valid ? pm[t] : 1.0;
        const int cnt = min(64, t0 - base);
        int found = -1;
        for (int s = 0; s < cnt; ++s) {
            const double xr = lane_f64(ar, s), xi = lane_f64(ai, s), xm = lane_f64(am, s);
            const double nr = xr * cr - xi * ci;
            const double ni = xr * ci + xi * cr;
            cm = xm * cm;
            cr = nr;
            ci = ni;
            if (base + s == t0 - 1 || (float)cm == 0.0f) {
                found = base + s + 1;
                break;
            }
        }
        if (found >= 0) {
            result = found;
            break;
        }
    }
    if (lane == 0) noff[L] = result;
    if (qt == 0 && lane == 0) {  // the head's |q|, |k| extrema, folded in by fwd_kernel
        qstat[bh] = 0u;
        kstat[bh] = 0u;
    }
}

// Fused forward, fp32 path (fp32 q, k, v; the bf16 path runs
// fwd_pad_kernel).  A workgroup owns the BQ queries [i0, i0+BQ) of one head;
// wave w owns rows i0+32w .. i0+32w+31.  Keys go in 32-key blocks, tile by
// tile: the n_off key tiles before the query tile that the visit count
// allows, last to first, then the query tile's own NDIAG tiles, last to first.
//
// Each block k passes through two steps of a wave:
//   M(k)  matrix step: S(k) = K(k) Q^T;
//   V(k)  vector step: masks, shift, exponentials and gate factors of block
//         k, giving W~(k), and O += W~(k) V(k).
// The workgroup advances in phases separated by LDS-only barriers.  Waves
// 0..3 run step p in phase p and waves 4..7 one phase later, so the two
// waves that share a SIMD (w and w+4) alternate between matrix and vector
// work.  Key tiles, and the gate data of their side data, are copied
// asynchronously into NBUF rotating LDS buffers phases ahead of use; what is
// copied and landed in a phase is a function of the phase number alone, and
// every vector-memory operation in the phase loops is such a copy, waited
// for with exact counts.
template <int D, int DV, bool QKZ>
__global__ __launch_bounds__(NTHREADS, 1) void fwd_kernel(FwdArgs A) {
    using SM = Smem<D, DV>;
    using FR = Frag<true, D>;
    constexpr int NBUF = SM::NBUF;
    constexpr int NDIAG = BQ / BK;    // key tiles inside the query tile
    constexpr int NDB = 2 * NDIAG;    // 32-key blocks inside the query tile
    // copies a leading wave issues per tile: its K and V chunks (wave 0 also
    // the three gate planes of the side data and the tile's product)
    constexpr int VM_TILE = SM::KCH / NCOPY + SM::VINS / NCOPY;
    static_assert(VM_TILE + 4 < 64, "vmcnt range");
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *misc = reinterpret_cast<uint32_t *>(smem + SM::misc_off);
    // misc[2]: largest |q|; misc[3]: largest |k|

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, qi = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lag = w / (NWAVES / 2);  // 0: leading waves, 1: trailing waves
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
    const int t_diag0 = int(i0 / BK);  // first key tile of the query tile
    const int n_off = __builtin_amdgcn_readfirstlane(A.noff[bh * A.n_qt + qt]);
    const int n_tiles = n_off + NDIAG;
    const unsigned char *kh, *vh;
    head_bases<true, D, DV>(A, kv_head(A, bh), kh, vh);

    if (tid == 0) {
        misc[2] = 0;
        misc[3] = 0;
    }

    // key tile visited at schedule position sg, and its buffer
    auto tile_of = [&](int sg) __attribute__((always_inline)) {
        return sg < n_off ? t_diag0 - 1 - sg : t_diag0 + NDIAG - 1 - (sg - n_off);
    };
    auto tile_buf = [&](int sg) __attribute__((always_inline)) {
        return smem + (sg % NBUF) * SM::buf_bytes;
    };

    // ---- copies.  issue(sg) starts the copy of tile sg: K and V, and (wave
    // 0) three gate planes of its 64 keys -- S_j (re, im, modulus) into the
    // raw area for a tile before the query tile, a_{j+1} straight into the
    // side area for an own tile (the gate planes hold the identity gate past
    // n, and a_{j+1} past the head's last position is only ever multiplied
    // into an entry above the diagonal) -- and the tile's product.
    const uint32_t smem_lds = lds_addr(smem);
    // this head's S_j planes, a_{j+1} planes and tile products
    const double *t4 = uniform_ptr(A.t4 + 4 * bh * A.n_kt);
    const float *gS = uniform_ptr(A.gates + 3 * A.plane + bh * A.n_pad);
    const float *gA = uniform_ptr(A.gates + bh * A.n_pad + 1);
    auto issue = [&](int sg) __attribute__((always_inline)) {
        if (sg >= n_tiles) return;
        const int t = tile_of(sg);
        const uint32_t buf = smem_lds + uint32_t((sg % NBUF) * SM::buf_bytes);
        stage_async<D, DV>(A, buf, kh, vh, t, false, w);
        if (w == 0) {
            const bool off = sg < n_off;
            const uint32_t lo = uint32_t(fresh_lane() * 4);
            // (gate_src(bh, n_pad, t, lane, !off) of plane 3 or 0)
            const float *g = (off ? gS : gA) + t * BK;
            const uint32_t dst = buf + uint32_t(off ? SM::raw_off : SM::side_off);
            g2lds4(reinterpret_cast<const unsigned char *>(g), lo, dst);
            g2lds4(reinterpret_cast<const unsigned char *>(g + A.plane), lo, dst + BK * 4);
            g2lds4(reinterpret_cast<const unsigned char *>(g + 2 * A.plane), lo, dst + 2 * BK * 4);
            // the product of the tile's gates (32 bytes, lanes 0 and 1; an own
            // tile copies its own too, unused, so that every tile costs wave
            // 0 the same copies)
            g2lds16x2(reinterpret_cast<const unsigned char *>(t4 + 4 * t),
                      uint32_t(fresh_lane() * 16), buf + uint32_t(SM::tprod_off));
        }
    };
    uint32_t kbits = 0;
    // Landing of tile sg, once this wave's copies of it are in.  Wave 0 forms
    // T_j = C S_j of its 64 keys (C the visit's carried product, rounded to
    // float; one float rounding per product, far below the bf16 rounding of
    // the weights) with the dead flags.  C_s of visit s is accumulated by
    // wave 0 in f64 with the recurrence and rounding of the visit-count scan
    // (schedule_kernel): C_0 = 1, C_{s+1} = A_t C_s, A_t the product of the
    // gates of visit s's key tile t (copied with the tile); the running value
    // lives in LDS.  For an own tile every copying wave takes the largest |k|
    // of the K bytes it copied.
    double *cst = reinterpret_cast<double *>(smem + SM::carry_off);
    auto land = [&](int sg) __attribute__((always_inline)) {
        if (sg >= n_tiles) return;
        unsigned char *buf = tile_buf(sg);
        if (sg < n_off) {
            if (w == 0) {
                const int ln = fresh_lane();
                double c_re = 1.0, c_im = 0.0, c_m = 1.0;
                if (sg > 0) {
                    c_re = cst[0];
                    c_im = cst[1];
                    c_m = cst[2];
                }
                {
#pragma clang fp contract(off)
                    const double *at = reinterpret_cast<const double *>(buf + SM::tprod_off);
                    const double ar = at[0], ai = at[1], am = at[2];
                    const double nr = ar * c_re - ai * c_im;
                    const double ni = ar * c_im + ai * c_re;
                    const double nm = am * c_m;
                    if (ln == 0) {
                        cst[0] = nr;
                        cst[1] = ni;
                        cst[2] = nm;
                    }
                }
                const float ccx = (float)c_re, ccy = (float)c_im, ccz = (float)c_m;
                const float *raw = reinterpret_cast<const float *>(buf + SM::raw_off);
                float *sd = reinterpret_cast<float *>(buf + SM::side_off);
                const float g0 = raw[ln], g1 = raw[BK + ln], g2 = raw[2 * BK + ln];
                const float rt = ccz * g2;
                const int slot = perm64(ln);
                sd[slot] = ccx * g0 - ccy * g1;
                sd[BK + slot] = ccx * g1 + ccy * g0;
                sd[2 * BK + slot] = rt;
                const uint64_t dead = __ballot(rt == 0.0f);
                if (ln == 0) {
                    uint32_t *fl = reinterpret_cast<uint32_t *>(buf + SM::flag_off);
                    fl[0] = (uint32_t)(dead & 0xFFFFFFFFull) != 0u;
                    fl[1] = (uint32_t)(dead >> 32) != 0u;
                }
            }
        } else {
            kbits = max(kbits, own_kbits<D>(buf, w));
        }
    };
    // wait until this wave's copies of the tile landing now are in, leaving
    // those of the one tile after it (if started) in flight
    auto wait_landing = [&](bool newer_in_flight) __attribute__((always_inline)) {
        if (!newer_in_flight)
            wait_vmcnt<0>();
        else if (w == 0)
            wait_vmcnt<VM_TILE + 4>();
        else
            wait_vmcnt<VM_TILE>();
    };
    // Copies, around the steps of block k (tile m = k/2; the matrix step of
    // block k runs in phase 2k + lag, its vector step in phase 2k + 1 + lag).
    // Four buffers: every wave starts its share of tile m+2 right after its
    // matrix step of block 2m (phase 4m for the leading waves, 4m+1 for the
    // trailing ones; the buffer is tile m-2's, last read in phase 4m-3), and
    // waits for its share of tile m+1 in phase 4m+2 -- the leading waves
    // after their matrix step of block 2m+1, where wave 0 also lands the tile,
    // the trailing ones after their vector step of block 2m -- so that the
    // barrier closing phase 4m+2 publishes tile m+1.  A matrix step ends a
    // little before its partner's vector step: the copy work fills that
    // slack.  Two buffers (fp32 d = 128): tile m+1 is started in phase 4m+2
    // (the buffer of tile m-1, last read in phase 4m+1) and landed in phase
    // 4m+3.
    auto land_wait = [&](int m) __attribute__((always_inline)) {
        wait_landing(m + 2 < n_tiles);
        land(m + 1);
    };
    auto after_m = [&](int k) __attribute__((always_inline)) {
        const int m = k >> 1;
        if constexpr (NBUF == 4) {
            if ((k & 1) == 0)
                issue(m + 2);
            else if (!lag)
                land_wait(m);
        } else {
            static_assert(NBUF == 2, "two or four buffers");
            if (k & 1) {
                if (!lag) {
                    issue(m + 1);
                } else {
                    wait_vmcnt<0>();
                    land(m + 1);
                }
            }
        }
    };
    auto after_v = [&](int k) __attribute__((always_inline)) {
        const int m = k >> 1;
        if constexpr (NBUF == 4) {
            if (lag && (k & 1) == 0) land_wait(m);
        } else {
            if (!lag && (k & 1)) {
                wait_vmcnt<0>();
                land(m + 1);
            } else if (lag && (k & 1) == 0) {
                issue(m + 1);
            }
        }
    };

    // ---- prologue: the first tiles, Q, the row's prefix product (the copies
    // first, so that their latency and that of the loads overlap)
#pragma unroll
    for (int sg = 0; sg < NBUF / 2; ++sg) issue(sg);
    typename FR::type qf[FR::count];
    const uint32_t qbits = load_q<true, D>(A, bh, row, row_ok, h, qf);
    // a row whose prefix inside the query tile holds a closed gate sees no
    // key before the query tile
    const float prow_re = A.p_re[gbase + row], prow_im = A.p_im[gbase + row];
    const float prow_m = A.p_m[gbase + row];
    const bool row_live = !(prow_m == 0.0f);
    const bool wave_dead_rows = __any(!row_live);
    wait_vmcnt<0>();
    land(0);
    lds_barrier();
    atomicMax(&misc[2], wave_max_u32(qbits));

    f32x16 ore[DV / 32], oim[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ore[db][r] = 0.f;
            oim[db][r] = 0.f;
        }
    // shift of the live logits (log2 units), same in both halves; with qk = 0
    // every live logit is 0 and the shift is 0 throughout
    float M = QKZ ? 0.0f : -INFINITY;
    float z = 0.f;                         // this lane's share of the normaliser
    float gre = 0.f, gim = 0.f, gm = 0.f;  // running G_{row,j}, R_{row,j} (own tiles)
    f32x16 x;                              // scores of the block between M and V
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = 0.f;
    // Logits are c*S in log2 units; c = qk log2(e)/sqrt(d) may be negative.
    const bool cpos = A.c > 0.0f;
    const float dead_s = cpos ? -INFINITY : INFINITY;  // a score whose logit is -inf

    // New shift of block k from its (masked) scores, with the lazy rescale
    // of O and z (O then holds every block before k); returns the shift the
    // block's exponentials use (0 while a row has no live entry yet).
    // (the row's two halves meet through v_permlane32_swap of ts with itself:
    // its first result carries the lower half's values into both halves, its
    // second the upper half's)
    auto block_shift = [&]() __attribute__((always_inline)) -> float {
        if constexpr (QKZ) {
            return 0.0f;  // every live logit is 0: the shift stays 0
        } else {
            float ts = x[0];
            if (cpos) {
#pragma unroll
                for (int r = 1; r < 16; ++r) ts = fmaxf(ts, x[r]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ts),
                                                                 __float_as_uint(ts), false, false);
                ts = fmaxf(ts, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
            } else {
#pragma unroll
                for (int r = 1; r < 16; ++r) ts = fminf(ts, x[r]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ts),
                                                                 __float_as_uint(ts), false, false);
                ts = fminf(ts, fminf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
            }
            float t;
            {
#pragma clang fp contract(off)
                t = ts * A.c;  // the block's largest logit (-inf if none is live)
            }
            const bool grow = (t > M + kLazy) | ((M == -INFINITY) & (t > M));
            const bool resc = grow & (M != -INFINITY);
            if (__any(resc)) {
                const float alpha = resc ? __builtin_amdgcn_exp2f(M - t) : 1.0f;
#pragma unroll
                for (int db = 0; db < DV / 32; ++db)
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
    // exponentials e = 2^(c S - M) of one 16-key chunk, the normaliser, and
    // W~ = e * gate factor, multiplied into O right away.  QKZ: e is 1 on live entries
    // (all_live, or a non-zero modulus on a live row), else 0.
    // own: the exponent is formed as the rounded logit c*S minus the shift,
    // the shift being the rounded logit of the row's maximum when it was set,
    // so a row whose maximum sets the shift weighs that entry exactly 1 (the
    // query tile's own keys: every row's diagonal entry is live there).
    auto weights = [&](const unsigned char *buf, int kb, int kc, float msub, const float (&fre)[8],
                       const float (&fim)[8], const float (&fm)[8], bool all_live,
                       bool rlive, bool own) __attribute__((always_inline)) {
        float wre[8], wim[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float ex;
            if constexpr (QKZ) {
                ex = (all_live || (fm[e] > 0.0f && rlive)) ? 1.0f : 0.0f;
            } else if (own) {
#pragma clang fp contract(off)
                const float lg = x[8 * kc + e] * A.c;
                ex = __builtin_amdgcn_exp2f(lg - msub);
            } else {
                ex = __builtin_amdgcn_exp2f(fmaf(x[8 * kc + e], A.c, -msub));
            }
            z += ex * fm[e];
            wre[e] = ex * fre[e];
            wim[e] = ex * fim[e];
        }
        pv_chunk_f32<D, DV>(buf, kb, kc, qi, h, wre, wim, ore, oim);
    };
    // vector step of a block of a tile before the query tile: G = S_j C_t P_i
    // (P_i applied to O once, when the query tile's own keys begin); masked:
    // the block holds a dead column or the wave a dead row
    auto vstep_off = [&](const unsigned char *buf, int kb, bool masked) __attribute__((always_inline)) {
        const float *side = reinterpret_cast<const float *>(buf + SM::side_off);
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
        const float msub = block_shift();
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
            weights(buf, kb, kc, msub, fre, fim, fm, !masked, row_live, false);
            __builtin_amdgcn_sched_barrier(0);  // one chunk's side data at a time
        }
    };
    // vector step of a block of the query tile's own keys: explicit G_ij by a
    // running product per row, a_i a_{i-1} ... a_{j+1}, last key first; the
    // product restarts at 1 on the diagonal and is 0 above it
    auto vstep_own = [&](const unsigned char *buf, int kb, int dpos) __attribute__((always_inline)) {
        // The block's gates a_{j+1} are the same for every lane: lane L holds
        // those of key L mod 32 (one LDS read per plane), and each step of the
        // chains takes its key's value from that lane into a scalar register,
        // so the chains never wait on LDS.
        const float *side = reinterpret_cast<const float *>(buf + SM::side_off);
        const int kl = kb + (lane & 31);
        const float vre = side[kl], vim = side[BK + kl], vm = side[2 * BK + kl];
        auto key_gate = [](float v, int j) __attribute__((always_inline)) {
            return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
        };
        // pass 1: modulus R_{row,j} of the 16 keys this lane holds
        float Gm[16];
        const float gre0 = gre, gim0 = gim;
#pragma unroll
        for (int jj = 31; jj >= 0; --jj) {
            const float nm = gm * key_gate(vm, jj);
            gm = (jj == dpos) ? 1.0f : nm;
            if (h == ((jj >> 2) & 1)) Gm[4 * (jj >> 3) + (jj & 3)] = gm;
        }
        if constexpr (!QKZ) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (Gm[r] > 0.0f) ? x[r] : dead_s;
        }
        const float msub = block_shift();
        // pass 2: G_{row,j} chunk by chunk, keys 31..16 then 15..0
        gre = gre0;
        gim = gim0;
#pragma unroll
        for (int kc = 1; kc >= 0; --kc) {
            float fre[8], fim[8], fm[8];
#pragma unroll
            for (int jj = 16 * kc + 15; jj >= 16 * kc; --jj) {
                const float dr = key_gate(vre, jj), di = key_gate(vim, jj);
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
            weights(buf, kb, kc, msub, fre, fim, fm, false, true, true);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto block_buf = [&](int k) __attribute__((always_inline)) { return tile_buf(k >> 1); };
    // key offset of block k inside its tile: ascending in the tiles before
    // the query tile, descending in its own tiles
    auto block_kb = [&](int k, bool off) __attribute__((always_inline)) {
        return off ? 32 * (k & 1) : 32 * (1 - (k & 1));
    };
    // an own-tile block wholly above this wave's rows is skipped
    auto block_active = [&](int k, bool off) __attribute__((always_inline)) {
        return off || k - 2 * n_off >= NDB - 1 - w;
    };
    // dead-column flag of block k (read during its matrix step, where the LDS
    // latency hides behind the matrix instructions)
    uint32_t kflag = 0;
    // matrix step of block k when blocks k-1 and k both lie before the query
    // tile
    auto m_step_off = [&](int k) __attribute__((always_inline)) {
        kflag = reinterpret_cast<const uint32_t *>(block_buf(k) + SM::flag_off)[k & 1];
        if constexpr (!QKZ) x = s_block<D>(block_buf(k), block_kb(k, true), qi, h, qf);
    };
    auto m_step = [&](int k) __attribute__((always_inline)) {
        if constexpr (!QKZ) {
            if ((k >> 1) < n_tiles) {
                const bool off = (k >> 1) < n_off;
                if (block_active(k, off)) x = s_block<D>(block_buf(k), block_kb(k, off), qi, h, qf);
            }
        }
    };
    // the vector step's results stay in its own phase
    auto settle_weights = [&]() __attribute__((always_inline)) { settle(z); };
    // vector step of block k of a tile before the query tile
    auto v_step_off = [&](int k) __attribute__((always_inline)) {
        vstep_off(block_buf(k), block_kb(k, true),
                  wave_dead_rows || __builtin_amdgcn_readfirstlane(kflag) != 0u);
        settle_weights();
    };
    // vector step of block k of the query tile's own tiles
    auto v_step_own = [&](int k) __attribute__((always_inline)) {
        if (n_off > 0 && k == 2 * n_off) {
            // the last block before the query tile is in O: rotate by P_i
#pragma unroll
            for (int db = 0; db < DV / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float xr = ore[db][r], xi = oim[db][r];
                    ore[db][r] = prow_re * xr - prow_im * xi;
                    oim[db][r] = prow_re * xi + prow_im * xr;
                }
            z *= prow_m;
        }
        if (!block_active(k, false)) return;
        const int kb = block_kb(k, false);
        const int tl = NDIAG - 1 - ((k >> 1) - n_off);  // key tile, counted from t_diag0
        vstep_own(block_buf(k), kb, 32 * w + qi - (tl * BK + kb));  // 0..31 on the block's diagonal
        settle_weights();
    };

    // ---- the phases.  Block k has its matrix step in phase 2k + lag and its
    // vector step in phase 2k + 1 + lag; a barrier ends every phase, and the
    // trailing waves pass one extra barrier first, the leading ones one last.
    // The copies of a phase (leading waves only) run around its step.
    if (lag) lds_barrier();
    int k = 0;
    for (; k < 2 * n_off; ++k) {
        m_step_off(k);
        after_m(k);
        lds_barrier();
        v_step_off(k);
        after_v(k);
        lds_barrier();
    }
    for (; k < 2 * n_tiles; ++k) {
        m_step(k);
        after_m(k);
        lds_barrier();
        v_step_own(k);
        after_v(k);
        lds_barrier();
    }
    m_step(k);  // (no block left: keeps the phase count)
    after_m(k);
    lds_barrier();
    if (!lag) lds_barrier();
    atomicMax(&misc[3], wave_max_u32(kbits));

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
        float *orp = A.o_re + (bh * A.n + row) * DV;
        float *oip = A.o_im + (bh * A.n + row) * DV;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * db + 8 * g4 + 4 * h;
                float4 vr, vi;
                vr.x = scale_keep_zero(ore[db][4 * g4 + 0], f);
                vr.y = scale_keep_zero(ore[db][4 * g4 + 1], f);
                vr.z = scale_keep_zero(ore[db][4 * g4 + 2], f);
                vr.w = scale_keep_zero(ore[db][4 * g4 + 3], f);
                vi.x = scale_keep_zero(oim[db][4 * g4 + 0], f);
                vi.y = scale_keep_zero(oim[db][4 * g4 + 1], f);
                vi.z = scale_keep_zero(oim[db][4 * g4 + 2], f);
                vi.w = scale_keep_zero(oim[db][4 * g4 + 3], f);
                *reinterpret_cast<float4 *>(orp + d0) = vr;
                *reinterpret_cast<float4 *>(oip + d0) = vi;
            }
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t qb = misc[2], kb = misc[3];
        atomicMax(&A.qstat[bh], qb);
        atomicMax(&A.kstat[bh], kb);
        if (qb >= kInfBits || kb >= kInfBits) A.status[0] = kNonFinite;
        atomicAdd(&A.counters[0], uint32_t(n_off));
    }
}

// --------------------------------------------------------------------------
// Refusal of an overflowing logit (section "Evaluation and refusals").  The
// per-head extrema of |q| and |k| that the fused forward folded in bound every
// logit by |c| d max|q| max|k|; only a head where that bound reaches the
// float32 range recomputes its logits (with the same MFMA code and scale as
// the fused forward) and checks every j <= i.  fp32 path; the bf16 path runs
// logit_check_pad_kernel.
template <int D>
__global__ __launch_bounds__(NTHREADS) void logit_check_kernel(FwdArgs A) {
    using FR = Frag<true, D>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int go;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, qi = lane & 31;
    const int L = blockIdx.x;
    const int64_t qt = A.n_qt - 1 - L / A.BH;
    const int64_t bh = L % A.BH;
    if (tid == 0) {
        const uint32_t qm = A.qstat[bh], km = A.kstat[bh];
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
    load_q<true, D>(A, bh, row, row_ok, h, qf);
    const unsigned char *kh, *vh;
    head_bases<true, D, D>(A, kv_head(A, bh), kh, vh);
    bool bad = false;
    for (int64_t t = 0; t < (i0 + BQ) / BK; ++t) {
        __syncthreads();
        stage_async<D, D>(A, lds_addr(smem), kh, vh, int(t), true,
                            __builtin_amdgcn_readfirstlane(w));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const f32x16 s = s_block<D>(smem, 32 * blk, qi, h, qf);
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

// --------------------------------------------------------------------------
// Fused forward, bf16 path: padded tiles (row strides of an odd number of
// 16-byte slots, so every matrix-operand read is a per-lane base plus an
// immediate offset and a half-wave's rows fall into distinct bank groups),
// and a loop unrolled per key tile, so that the step of each block is fixed
// at compile time, with one workgroup barrier per key tile.  Waves 1..7 copy
// the K and value tiles; wave 0 copies the gate planes and the tile products
// and lands the tiles.
template <int D, int DV>
struct PSmem {
    static constexpr int KSL = pad_kslots<D>();
    static constexpr int KROW = 16 * KSL;          // bytes per K row
    static constexpr int VSTR = 16 * pad_vslots<DV>();  // bytes per value row
    static constexpr int NKC = pad_kcopies<D>();   // copy instructions of a K tile
    static constexpr int NVC = pad_vcopies<DV>();  // of a value tile
    static constexpr int NC = NKC + NVC;
    static constexpr int CPW = pad_copies_per_wave<D, DV>();  // per copying wave and tile
    static constexpr size_t k_bytes = size_t(1024) * NKC;
    static constexpr size_t v_bytes = size_t(1024) * NVC;
    static constexpr size_t side_off = k_bytes + v_bytes;
    static constexpr size_t raw_off = side_off + 3 * BK * sizeof(float);
    static constexpr size_t tprod_off = raw_off + 3 * BK * sizeof(float);
    static constexpr size_t flag_off = tprod_off + 4 * sizeof(double);
    static constexpr size_t buf_bytes = (flag_off + 16 + 255) / 256 * 256;
    static constexpr int NBUF = 4;
    static constexpr size_t misc_off = NBUF * buf_bytes;
    static constexpr size_t carry_off = misc_off + 8 * sizeof(uint32_t);
    // per-lane source offsets of each copying wave's copies, [NWAVES-1][CPW][64]
    static constexpr size_t coff_off = carry_off + 4 * sizeof(double);
    static constexpr size_t bytes = coff_off + size_t(NWAVES - 1) * CPW * 64 * sizeof(uint32_t);
    // every copying wave issues CPW distinct copies, instruction j = w - 1 + 7 i:
    // the first NKHI (waves 1..WSPLIT) or NKHI - 1 (the others) are K copies
    static constexpr bool EXACT = (NWAVES - 1) * CPW == NC;
    static constexpr int NKHI = (NKC + NWAVES - 2) / (NWAVES - 1);
    static constexpr int WSPLIT = NKC - (NWAVES - 1) * (NKHI - 1);
    static_assert(bytes <= 160 * 1024, "LDS");
    static_assert(size_t(BK) * KROW == k_bytes && size_t(BK) * VSTR == v_bytes, "whole copies");
    static_assert(CPW <= 5, "copy batch");
};

// The copies of one wave for one tile when every copying wave issues CPW = 5
// distinct ones (j = w - 1 + 7 i): the first NK read K rows (base kb), the
// others value rows (base vb); copy i writes at LDS address l0 + 7168 i.  m0 is
// saved once, set before each direct global->LDS load (lane L reads base +
// o[i], writes 16 bytes at m0 + 16 L) and restored at the end.
#define RESOLVENT_G2LS(v, s, imm) \
    "s_add_u32 m0, %8, " #imm "\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %" #v ", %" #s "\n\t"
template <int NK>
__device__ __forceinline__ void g2l_split5(const uint32_t (&o)[5], const unsigned char *kb,
                                           const unsigned char *vb, uint32_t l0) {
    static_assert(NK == 2 || NK == 3, "split");
    uint32_t sv;
    if constexpr (NK == 3)
        asm volatile("s_mov_b32 %0, m0\n\t" RESOLVENT_G2LS(1, 6, 0) RESOLVENT_G2LS(2, 6, 7168)
                     RESOLVENT_G2LS(3, 6, 14336) RESOLVENT_G2LS(4, 7, 21504)
                     RESOLVENT_G2LS(5, 7, 28672) "s_mov_b32 m0, %0"
                     : "=&s"(sv)
                     : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "s"(kb), "s"(vb), "s"(l0)
                     : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\t" RESOLVENT_G2LS(1, 6, 0) RESOLVENT_G2LS(2, 6, 7168)
                     RESOLVENT_G2LS(3, 7, 14336) RESOLVENT_G2LS(4, 7, 21504)
                     RESOLVENT_G2LS(5, 7, 28672) "s_mov_b32 m0, %0"
                     : "=&s"(sv)
                     : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "s"(kb), "s"(vb), "s"(l0)
                     : "memory");
}
#undef RESOLVENT_G2LS

// The copies of one wave for one tile, as one instruction group: m0 is saved
// once, set to each copy's LDS address (wave-uniform) before its direct
// global->LDS load (lane L reads base + off and writes 16 bytes at
// m0 + 16 L), and restored at the end.
#define RESOLVENT_G2L(v, s, l) \
    "s_mov_b32 m0, %" #l "\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %" #v ", %" #s "\n\t"
template <int N>
struct G2LBatch;
template <>
struct G2LBatch<1> {
    __device__ __forceinline__ static void go(const uint32_t (&o)[1], const unsigned char *const (&b)[1],
                                              const uint32_t (&l)[1]) {
        uint32_t sv;
        asm volatile("s_mov_b32 %0, m0\n\t" RESOLVENT_G2L(1, 2, 3) "s_mov_b32 m0, %0"
                     : "=&s"(sv) : "v"(o[0]), "s"(b[0]), "s"(l[0]) : "memory");
    }
};
template <>
struct G2LBatch<2> {
    __device__ __forceinline__ static void go(const uint32_t (&o)[2], const unsigned char *const (&b)[2],
                                              const uint32_t (&l)[2]) {
        uint32_t sv;
        asm volatile("s_mov_b32 %0, m0\n\t" RESOLVENT_G2L(1, 3, 5) RESOLVENT_G2L(2, 4, 6)
                     "s_mov_b32 m0, %0"
                     : "=&s"(sv) : "v"(o[0]), "v"(o[1]), "s"(b[0]), "s"(b[1]), "s"(l[0]), "s"(l[1])
                     : "memory");
    }
};
template <>
struct G2LBatch<3> {
    __device__ __forceinline__ static void go(const uint32_t (&o)[3], const unsigned char *const (&b)[3],
                                              const uint32_t (&l)[3]) {
        uint32_t sv;
        asm volatile("s_mov_b32 %0, m0\n\t" RESOLVENT_G2L(1, 4, 7) RESOLVENT_G2L(2, 5, 8)
                     RESOLVENT_G2L(3, 6, 9) "s_mov_b32 m0, %0"
                     : "=&s"(sv)
                     : "v"(o[0]), "v"(o[1]), "v"(o[2]), "s"(b[0]), "s"(b[1]), "s"(b[2]), "s"(l[0]),
                       "s"(l[1]), "s"(l[2])
                     : "memory");
    }
};
template <>
struct G2LBatch<4> {
    __device__ __forceinline__ static void go(const uint32_t (&o)[4], const unsigned char *const (&b)[4],
                                              const uint32_t (&l)[4]) {
        uint32_t sv;
        asm volatile("s_mov_b32 %0, m0\n\t" RESOLVENT_G2L(1, 5, 9) RESOLVENT_G2L(2, 6, 10)
                     RESOLVENT_G2L(3, 7, 11) RESOLVENT_G2L(4, 8, 12) "s_mov_b32 m0, %0"
                     : "=&s"(sv)
                     : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "s"(b[0]), "s"(b[1]), "s"(b[2]),
                       "s"(b[3]), "s"(l[0]), "s"(l[1]), "s"(l[2]), "s"(l[3])
                     : "memory");
    }
};
template <>
struct G2LBatch<5> {
    __device__ __forceinline__ static void go(const uint32_t (&o)[5], const unsigned char *const (&b)[5],
                                              const uint32_t (&l)[5]) {
        uint32_t sv;
        asm volatile("s_mov_b32 %0, m0\n\t" RESOLVENT_G2L(1, 6, 11) RESOLVENT_G2L(2, 7, 12)
                     RESOLVENT_G2L(3, 8, 13) RESOLVENT_G2L(4, 9, 14) RESOLVENT_G2L(5, 10, 15)
                     "s_mov_b32 m0, %0"
                     : "=&s"(sv)
                     : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "s"(b[0]), "s"(b[1]),
                       "s"(b[2]), "s"(b[3]), "s"(b[4]), "s"(l[0]), "s"(l[1]), "s"(l[2]), "s"(l[3]),
                       "s"(l[4])
                     : "memory");
    }
};
#undef RESOLVENT_G2L

// The A operand of O^T += V^T W~^T for one (16-key chunk, 32-channel group)
// from the value rows: two transposing 8-byte reads at the lane's address p
// and eight rows further on (keys +8).
template <int DV>
__device__ __forceinline__ bf16x8 vread_tr(const unsigned char *p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(lds_void *)(p));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s *)(lds_void *)(p + 8 * 16 * pad_vslots<DV>()));
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s ab = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return __builtin_bit_cast(bf16x8, ab);
}

// Operand fragments of a matrix step stream through four-deep pipelines (LDS
// latency under load is a few hundred cycles).
constexpr int MDEPTH = 4;
struct MPrefetch {
    bf16x8 vf[MDEPTH], kf[MDEPTH];
};
// Weights W~ of one 32-key block as the B operand of O^T += V^T W~^T, per
// 16-key chunk kc, packed bf16.
struct BlockW {
    bf16x8 r[2], i[2];
};

// Matrix step on padded tiles: O^T += V^T W~^T for the block whose value rows
// start at vb (lane part included) at key offset KBV (PV), and S^T = K Q^T for
// the block at K offset KBS of the K tile at kb (lane part included) (S).
// Operand fragments stream four deep through pf; NPRE of each kind were
// requested before (pstep_prefetch).
template <int D, int DV, int KBV, int KBS, bool PV, bool S, int I0, int I1>
__device__ __forceinline__ void pstep_prefetch(const unsigned char *vb, const unsigned char *kb,
                                               MPrefetch &pf) {
    constexpr int NV = PV ? 2 * (DV / 32) : 0;
    constexpr int NK = S ? D / 16 : 0;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        if (i < NV) {
            const int kc = i / (DV / 32), db = i % (DV / 32);
            pf.vf[i] = vread_tr<DV>(vb + (KBV + 16 * kc) * (16 * pad_vslots<DV>()) + 64 * db);
        }
        if (i < NK)
            pf.kf[i] = *reinterpret_cast<const bf16x8 *>(kb + KBS * 16 * pad_kslots<D>() + 32 * i);
    }
}
template <int D, int DV, int KBV, int KBS, bool PV, bool S, int NPRE>
__device__ __forceinline__ void pstep(const unsigned char *vb, const unsigned char *kb,
                                      MPrefetch &pf, const bf16x8 (&wr)[2], const bf16x8 (&wi)[2],
                                      const bf16x8 (&qf)[D / 16], f32x16 (&ore)[DV / 32],
                                      f32x16 (&oim)[DV / 32], f32x16 &sacc) {
    constexpr int NDB = DV / 32;
    constexpr int NV = PV ? 2 * NDB : 0;
    constexpr int NK = S ? D / 16 : 0;
    constexpr int NSTEP = NV > NK ? NV : NK;
    pstep_prefetch<D, DV, KBV, KBS, PV, S, NPRE, MDEPTH>(vb, kb, pf);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i < NV) {
            const int kc = i / NDB, db = i % NDB;
            const bf16x8 a = pf.vf[i % MDEPTH];
            ore[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wr[kc], ore[db], 0, 0, 0);
            oim[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wi[kc], oim[db], 0, 0, 0);
            if (i + MDEPTH < NV) {
                const int kc2 = (i + MDEPTH) / NDB, db2 = (i + MDEPTH) % NDB;
                pf.vf[i % MDEPTH] =
                    vread_tr<DV>(vb + (KBV + 16 * kc2) * (16 * pad_vslots<DV>()) + 64 * db2);
            }
        }
        if (i < NK) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf.kf[i % MDEPTH], qf[i],
                                                            i == 0 ? f32x16{} : sacc, 0, 0, 0);
            if (i + MDEPTH < NK)
                pf.kf[i % MDEPTH] = *reinterpret_cast<const bf16x8 *>(
                    kb + KBS * 16 * pad_kslots<D>() + 32 * (i + MDEPTH));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// The next work item of a workgroup whose home queue is `home` (the query
// tile bh * n_qt + qt, queue_item), or -1 when every queue is empty: a
// workgroup takes items from its home queue and, once that is empty, from the
// others in turn.  Called by every lane of one wave, with
// no divergent branch: lane 0 adds 1 to the queue's counter and the other
// lanes 0, and every lane takes lane 0's result.  (A branch on the thread
// index here, inside the workgroup's loop, let the compiler run the lanes of
// the fetching wave through different loop paths with different barrier
// sequences.)
template <typename Args>
__device__ __forceinline__ int next_item(const Args &A, int home) {
    const int lane = threadIdx.x & 63;
    const uint32_t inc = lane == 0 ? 1u : 0u;
    const uint32_t count = uint32_t(A.BH / A.nq) * uint32_t(A.n_qt);  // items per queue
    // every queue's counter at once (lane x reads queue x): a counter only
    // grows, so one at or past the end proves its queue empty without an
    // atomic (a workgroup's last fetch would otherwise take nq atomics in turn)
    const uint32_t seen = lane < A.nq ? __atomic_load_n(&A.queues[lane], __ATOMIC_RELAXED) : count;
    for (int i = 0; i < A.nq; ++i) {
        const int x = home + i < A.nq ? home + i : home + i - A.nq;
        if (uint32_t(__builtin_amdgcn_readlane(int(seen), x)) >= count) continue;
        const uint32_t k = __builtin_amdgcn_readfirstlane(atomicAdd(&A.queues[x], inc));
        const int64_t it = queue_item(x, k, A.nq, A.BH, A.n_qt, A.order, A.q0);
        if (it >= 0) return int(it);
    }
    return -1;
}

template <int D, int DV, bool QKZ, typename Args>
__device__ __forceinline__ void fwd_pad_item(const Args &A, int64_t bh, int64_t qt, int home) {
    using SM = PSmem<D, DV>;
    constexpr int NBUF = SM::NBUF;
    constexpr int NDIAG = BQ / BK;  // key tiles inside the query tile
    constexpr int NDB = 2 * NDIAG;  // 32-key blocks inside the query tile
    constexpr int CPW = SM::CPW;
    constexpr int KROW = SM::KROW, VSTR = SM::VSTR;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *misc = reinterpret_cast<uint32_t *>(smem + SM::misc_off);
    // misc[2]: largest |q|; misc[3]: largest |k|; misc[4]: the first work
    // item, misc[5]: the next one

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, qi = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lag = w / (NWAVES / 2);  // 0: leading waves, 1: trailing waves
    const int64_t i0 = qt * BQ;
    const int64_t row = i0 + 32 * w + qi;
    const bool row_ok = row < A.n;
    const int64_t gbase = bh * A.n_pad;
    const int t_diag0 = int(i0 / BK);
    const int n_off = __builtin_amdgcn_readfirstlane(A.noff[bh * A.n_qt + qt]);
    const int n_tiles = n_off + NDIAG;
    const unsigned char *kh, *vh;
    head_bases<false, D, DV>(A, kv_head(A, bh), kh, vh);
    if (w == 0) {  // whole wave: no divergent branch in the workgroup's loop
        misc[2] = 0;
        misc[3] = 0;
    }
    auto tile_of = [&](int sg) __attribute__((always_inline)) {
        return sg < n_off ? t_diag0 - 1 - sg : t_diag0 + NDIAG - 1 - (sg - n_off);
    };
    auto tile_buf = [&](int sg) __attribute__((always_inline)) {
        return smem + (sg & (NBUF - 1)) * SM::buf_bytes;
    };
    const uint32_t smem_lds = lds_addr(smem);
    const int n32 = int(A.n);  // n <= 2^22 (checked on the host)

    // ---- copies: waves 1..7 copy K and V, CPW instructions each per tile,
    // with per-lane source offsets computed once; wave 0 copies the three gate
    // planes of the tile's 64 keys (S_j into the raw area for a tile before
    // the query tile, a_{j+1} into the side area for an own tile) and the tile
    // product.
    uint32_t *coffs = reinterpret_cast<uint32_t *>(smem + SM::coff_off);
    if (w > 0) {
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            coffs[((w - 1) * CPW + i) * 64 + lane] =
                pad_copy_src<D, DV>(pad_copy_j<D, DV>(w, i), lane);
    }
    const double *t4 = uniform_ptr(A.t4 + 4 * bh * A.n_kt);
    const float *gS = uniform_ptr(A.gates + 3 * A.plane + bh * A.n_pad);
    const float *gA = uniform_ptr(A.gates + bh * A.n_pad + 1);
    auto issue = [&](int sg) __attribute__((always_inline)) {
        if (sg >= n_tiles) return;
        const int t = tile_of(sg);
        const uint32_t buf = smem_lds + uint32_t((sg & (NBUF - 1)) * SM::buf_bytes);
        if (w > 0) {
            // a tile reaching past key n-1 takes K rows clamped to it, with
            // offsets relative to the head's rows
            const bool ragged = (t + 1) * BK > n32;
            const unsigned char *kt =
                uniform_ptr(ragged ? kh : kh + int64_t(t) * (BK * D * 2));
            const unsigned char *vt =
                uniform_ptr(ragged ? vh : vh + int64_t(t) * (BK * DV * 2));
            const uint32_t *co = coffs + (w - 1) * CPW * 64 + fresh_lane();
            uint32_t o[CPW];
#pragma unroll
            for (int i = 0; i < CPW; ++i) o[i] = co[64 * i];
            if (ragged) {
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    const int j = pad_copy_j<D, DV>(w, i);
                    o[i] = j < SM::NKC
                               ? pad_kcopy_src_ragged<D>(j, fresh_lane(), A.n, t)
                               : pad_vcopy_src_ragged<DV>(j - SM::NKC, fresh_lane(), A.n, t);
                }
            }
            if constexpr (SM::EXACT && CPW == 5) {
                const uint32_t l0 = __builtin_amdgcn_readfirstlane(buf + uint32_t(1024 * (w - 1)));
                if (w <= SM::WSPLIT)
                    g2l_split5<SM::NKHI>(o, kt, vt, l0);
                else
                    g2l_split5<SM::NKHI - 1>(o, kt, vt, l0);
            } else {
                uint32_t l[CPW];
                const unsigned char *b[CPW];
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    const int j = pad_copy_j<D, DV>(w, i);
                    b[i] = j < SM::NKC ? kt : vt;
                    l[i] = __builtin_amdgcn_readfirstlane(buf + uint32_t(1024 * j));
                }
                G2LBatch<CPW>::go(o, b, l);
            }
        } else {
            const bool off = sg < n_off;
            const uint32_t lo = uint32_t(fresh_lane() * 4);
            const float *g = uniform_ptr((off ? gS : gA) + t * BK);
            const uint32_t dst = buf + uint32_t(off ? SM::raw_off : SM::side_off);
            g2lds4(reinterpret_cast<const unsigned char *>(g), lo, dst);
            g2lds4(reinterpret_cast<const unsigned char *>(g + A.plane), lo, dst + BK * 4);
            g2lds4(reinterpret_cast<const unsigned char *>(g + 2 * A.plane), lo, dst + 2 * BK * 4);
            g2lds16x2(reinterpret_cast<const unsigned char *>(uniform_ptr(t4 + 4 * t)),
                      uint32_t(fresh_lane() * 16), buf + uint32_t(SM::tprod_off));
        }
    };
    // Landing of tile sg once the wave's copies of it are in (as fwd_kernel):
    // wave 0 forms T_j = C S_j of the 64 keys of a tile before the query tile
    // (C the visit's carried product, accumulated in f64 in LDS with the
    // recurrence and rounding of the visit-count scan) and its dead-column
    // flags; for an own tile each copying wave takes the largest |k| of the K
    // slots it copied.
    uint32_t kbits = 0;
    double *cst = reinterpret_cast<double *>(smem + SM::carry_off);
    auto land = [&](int sg) __attribute__((always_inline)) {
        if (sg >= n_tiles) return;
        unsigned char *buf = tile_buf(sg);
        if (sg < n_off) {
            if (w == 0) {
                // every LDS read first, so that they share one round trip:
                // the tile's gate factors (one key per lane), the tile's
                // product and the carried product before the tile
                const int ln = fresh_lane();
                const float *raw = reinterpret_cast<const float *>(buf + SM::raw_off);
                const float g0 = raw[ln], g1 = raw[BK + ln], g2 = raw[2 * BK + ln];
                const double *at = reinterpret_cast<const double *>(buf + SM::tprod_off);
                const double ar = at[0], ai = at[1], am = at[2];
                double c_re = 1.0, c_im = 0.0, c_m = 1.0;
                if (sg > 0) {
                    c_re = cst[0];
                    c_im = cst[1];
                    c_m = cst[2];
                }
                settle(ar);
                settle(ai);
                settle(am);
                const float ccx = (float)c_re, ccy = (float)c_im, ccz = (float)c_m;
                float *sd = reinterpret_cast<float *>(buf + SM::side_off);
                const float rt = ccz * g2;
                const int slot = perm64(ln);
                // explicit fused forms: the rounding does not depend on
                // which product the compiler would contract
                sd[slot] = fmaf(ccx, g0, -(ccy * g1));
                sd[BK + slot] = fmaf(ccx, g1, ccy * g0);
                sd[2 * BK + slot] = rt;
                // the carried product of the next tile (the visit-count
                // recurrence and rounding), and the dead keys of this one as
                // a 64-bit mask: a word is nonzero when its 32-key block holds
                // a dead key
                const uint64_t dead = __ballot(rt == 0.0f);
                double nr, ni, nm;
                {
#pragma clang fp contract(off)
                    nr = ar * c_re - ai * c_im;
                    ni = ar * c_im + ai * c_re;
                    nm = am * c_m;
                }
                // (every lane holds the same values and writes them: no
                // divergent branch in the workgroup's loop)
                cst[0] = nr;
                cst[1] = ni;
                cst[2] = nm;
                *reinterpret_cast<uint64_t *>(buf + SM::flag_off) = dead;
            }
        } else if (w == 0) {
            // an own tile: the inclusive suffix products of its gate factors
            // inside each group of 8 keys, S8_l = c_l c_{l+1} ... c_{8g+7}
            // (c_l = a_{t0+l+1}, g = l / 8), into the raw area
            const int ln = fresh_lane();
            const float *sd = reinterpret_cast<const float *>(buf + SM::side_off);
            float sr = sd[ln], si = sd[BK + ln], sm = sd[2 * BK + ln];
#pragma unroll
            for (int k = 1; k < 8; k <<= 1) {
                const float orr = __shfl_down(sr, k), oi = __shfl_down(si, k), om = __shfl_down(sm, k);
                if ((ln & 7) + k < 8) {
                    const float nr = fmaf(sr, orr, -(si * oi));
                    const float ni = fmaf(sr, oi, si * orr);
                    sr = nr;
                    si = ni;
                    sm = sm * om;
                }
            }
            float *s8 = reinterpret_cast<float *>(buf + SM::raw_off);
            s8[ln] = sr;
            s8[BK + ln] = si;
            s8[2 * BK + ln] = sm;
        } else {
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int j = pad_copy_j<D, DV>(w, i);
                if (j < SM::NKC) {
                    const uint4 v =
                        *reinterpret_cast<const uint4 *>(buf + 1024 * j + 16 * fresh_lane());
                    kbits = max(kbits, absbits_u4_bf16(v));
                }
            }
        }
    };
    // wait for this wave's copies of the tile landing now, leaving those of
    // the tile after it (if started) in flight, then land it
    auto land_wait = [&](int m) __attribute__((always_inline)) {
        if (m + 2 >= n_tiles)
            wait_vmcnt<0>();
        else if (w == 0)
            wait_vmcnt<4>();
        else
            wait_vmcnt<CPW>();
        land(m + 1);
    };

    // ---- prologue: the first two tiles, Q (negated when c < 0, so that the
    // largest logit is the largest score), the row's prefix product
    issue(0);
    issue(1);
    bf16x8 qf[D / 16];
    const uint32_t qbits = load_q<false, D>(A, bh, row, row_ok, h, qf);
    const float c = fabsf(A.c);  // logits are c S in log2 units
    if (A.c < 0.0f) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            uint4 u = __builtin_bit_cast(uint4, qf[s]);
            u.x ^= 0x80008000u;
            u.y ^= 0x80008000u;
            u.z ^= 0x80008000u;
            u.w ^= 0x80008000u;
            qf[s] = __builtin_bit_cast(bf16x8, u);
        }
    }
    const float prow_re = A.p_re[gbase + row], prow_im = A.p_im[gbase + row];
    const float prow_m = A.p_m[gbase + row];
    const bool row_live = !(prow_m == 0.0f);
    const bool wave_dead_rows = __any(!row_live);
    wait_vmcnt<0>();
    land(0);
    lds_barrier();
    atomicMax(&misc[2], wave_max_u32(qbits));

    f32x16 ore[DV / 32], oim[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            ore[db][r] = 0.f;
            oim[db][r] = 0.f;
        }
    float M = QKZ ? 0.0f : -INFINITY;
    float z = 0.f;
    float gre = 0.f, gim = 0.f, gm = 0.f;
    f32x16 x;
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = 0.f;
    BlockW wk;
    constexpr float dead_s = -INFINITY;

    // per-lane parts of the operand and side-data reads
    const int klane = qi * KROW + 16 * h;
    const int vlane = pad_vread_tr<D, DV>(0, 0, 0, 0, lane);
    const int slane = int(SM::side_off) + 32 * h;

    auto block_shift = [&]() __attribute__((always_inline)) -> float {
        if constexpr (QKZ) {
            return 0.0f;
        } else {
            // a tree of depth 3 (the maximum is the same in any order)
            const float m0 = fmaxf(fmaxf(x[0], x[1]), x[2]), m1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
            const float m2 = fmaxf(fmaxf(x[6], x[7]), x[8]), m3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
            const float m4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
            float ts = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), x[15]));
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ts),
                                                             __float_as_uint(ts), false, false);
            ts = fmaxf(ts, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
            float t;
            {
#pragma clang fp contract(off)
                t = ts * c;
            }
            const bool grow = (t > M + kLazy) | ((M == -INFINITY) & (t > M));
            const bool resc = grow & (M != -INFINITY);
            if (__any(resc)) {
                const float alpha = resc ? __builtin_amdgcn_exp2f(M - t) : 1.0f;
#pragma unroll
                for (int db = 0; db < DV / 32; ++db)
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
    // exponentials, normaliser and packed weights of one 16-key chunk (own:
    // the exponent is the rounded logit minus the shift, as in fwd_kernel)
    auto weights = [&](int kc, float msub, const float (&fre)[8], const float (&fim)[8],
                       const float (&fm)[8], bool all_live, bool rlive,
                       bool own) __attribute__((always_inline)) {
        float wre[8], wim[8], ex[8];
        if constexpr (QKZ) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ex[e] = (all_live || (fm[e] > 0.0f && rlive)) ? 1.0f : 0.0f;
        } else {
            // the exponents first, then the exponentials, then their uses
            float t[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (own) {
#pragma clang fp contract(off)
                    const float lg = x[8 * kc + e] * c;
                    t[e] = lg - msub;
                } else {
                    t[e] = fmaf(x[8 * kc + e], c, -msub);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 8; ++e) ex[e] = __builtin_amdgcn_exp2f(t[e]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            z += ex[e] * fm[e];
            wre[e] = ex[e] * fre[e];
            wim[e] = ex[e] * fim[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            wk.r[kc][e] = (__bf16)wre[e];
            wk.i[kc][e] = (__bf16)wim[e];
        }
    };
    // vector step of the block at KB of a tile before the query tile (side
    // data at sb, lane part included): G = S_j C_t P_i (P_i applied to O once,
    // when the query tile's own keys begin); masked: a dead column or row
    typedef float v4f __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const v4f lds_v4f;
    auto unpack = [](const v4f &a, const v4f &b, float (&o)[8]) __attribute__((always_inline)) {
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    };
    auto vstep_off = [&](const unsigned char *sb, int kb, bool masked) __attribute__((always_inline)) {
        lds_v4f *sv = (lds_v4f *)(lds_void *)(sb + 4 * kb);
#define RD128(r, off) r = __builtin_nontemporal_load(sv + (off) / 16)
        v4f a0, a1, b0, b1, c0, c1;
        __builtin_amdgcn_sched_barrier(0);
        RD128(a0, 0); RD128(a1, 16); RD128(b0, 4 * BK); RD128(b1, 4 * BK + 16); RD128(c0, 8 * BK); RD128(c1, 8 * BK + 16);
        __builtin_amdgcn_sched_barrier(0);
        if (!QKZ && masked) {
            v4f m0, m1;
            RD128(m0, 8 * BK + 64); RD128(m1, 8 * BK + 80);
            float fm0[8], fm1[8];
            unpack(c0, c1, fm0);
            unpack(m0, m1, fm1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = (fm0[e] > 0.0f && row_live) ? x[e] : dead_s;
                x[8 + e] = (fm1[e] > 0.0f && row_live) ? x[8 + e] : dead_s;
            }
        }
        const float msub = block_shift();
        __builtin_amdgcn_sched_barrier(0);
        float fre[8], fim[8], fm[8];
        unpack(a0, a1, fre);
        unpack(b0, b1, fim);
        unpack(c0, c1, fm);
        float ex[8];
        if constexpr (QKZ) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ex[e] = (!masked || (fm[e] > 0.0f && row_live)) ? 1.0f : 0.0f;
        } else {
            float t[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = fmaf(x[e], c, -msub);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 8; ++e) ex[e] = __builtin_amdgcn_exp2f(t[e]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) z += ex[e] * fm[e];
        __builtin_amdgcn_sched_barrier(0);
        RD128(a0, 64); RD128(a1, 80); RD128(b0, 4 * BK + 64); RD128(b1, 4 * BK + 80);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            wk.r[0][e] = (__bf16)(ex[e] * fre[e]);
            wk.i[0][e] = (__bf16)(ex[e] * fim[e]);
        }
        __builtin_amdgcn_sched_barrier(0);
        RD128(c0, 8 * BK + 64); RD128(c1, 8 * BK + 80);
        __builtin_amdgcn_sched_barrier(0);
        unpack(a0, a1, fre);
        unpack(b0, b1, fim);
        unpack(c0, c1, fm);
        weights(1, msub, fre, fim, fm, !masked, row_live, false);
        __builtin_amdgcn_sched_barrier(0);
#undef RD128
    };
    // vector step of a block of the query tile's own keys: explicit G_ij by a
    // running product per row, a_i a_{i-1} ... a_{j+1}, last key first (as
    // fwd_kernel)
    // vector step of a block of the query tile's own keys.  The block's
    // keys fall in four groups of 8; for key j of group g and row i,
    // G_ij = a_i a_{i-1} ... a_{j+1} is S8_j (the suffix product inside the
    // group, formed when the tile landed) times R_i(g+1), the row's product
    // from the top of group g down to the row, when group g lies below the
    // row's own group; inside the row's own group it is the row's running
    // product taken key by key (restarting at the row's own key); above the
    // row it is 0.  R steps down a group at a time, R_i(g) = S8_{8g} R_i(g+1),
    // and starts at the row's own group, or, for a block wholly below the
    // wave's rows (diag false), at the row's running product carried from
    // the blocks above; R_i(0) is carried to the next block.
    auto vstep_own = [&](const unsigned char *buf, int kb, bool diag) __attribute__((always_inline)) {
        const float *side = reinterpret_cast<const float *>(buf + SM::side_off);
        const float *s8 = reinterpret_cast<const float *>(buf + SM::raw_off);
        lds_v4f *sv = (lds_v4f *)(lds_void *)(s8 + kb + 4 * h);
        lds_v4f *cv = (lds_v4f *)(lds_void *)(side + kb + 8 * (qi >> 3));
        const int gi = diag ? (qi >> 3) : 4;  // the row's own group (4: above the block)
        const int pi = qi & 7;                // the row's key inside its group
        // moduli
        float Gm[16];
        float rm_next;
        {
            float own[4] = {0.f, 0.f, 0.f, 0.f}, pre = 0.f;
            if (diag) {
                const v4f c0 = cv[(2 * BK) / 4], c1 = cv[(2 * BK) / 4 + 1];
                const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                float v[8];
                float g = 0.f;
#pragma unroll
                for (int t = 7; t >= 0; --t) {
                    g = (t == pi) ? 1.0f : g * c[t];
                    v[t] = g;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) own[e] = h ? v[4 + e] : v[e];
                pre = v[0];
            }
            float rm = diag ? 0.f : gm;
#pragma unroll
            for (int g = 3; g >= 0; --g) {
                const v4f q = sv[(2 * BK + 8 * g) / 4];
                const float qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) Gm[4 * g + e] = (g == gi) ? own[e] : qv[e] * rm;
                rm = (g == gi) ? pre : s8[2 * BK + kb + 8 * g] * rm;
            }
            rm_next = rm;
        }
        if constexpr (!QKZ) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (Gm[r] > 0.0f) ? x[r] : dead_s;
        }
        const float msub = block_shift();
        // complex values, a chunk of two groups at a time
        float own_r[4] = {0.f, 0.f, 0.f, 0.f}, own_i[4] = {0.f, 0.f, 0.f, 0.f};
        float pre_r = 0.f, pre_i = 0.f;
        if (diag) {
            const v4f r0 = cv[0], r1 = cv[1], i0 = cv[BK / 4], i1 = cv[BK / 4 + 1];
            const float cr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
            const float ci[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
            float vr[8], vi[8];
            float gr_ = 0.f, gi_ = 0.f;
#pragma unroll
            for (int t = 7; t >= 0; --t) {
                const float nr = fmaf(gr_, cr[t], -(gi_ * ci[t]));
                const float ni = fmaf(gr_, ci[t], gi_ * cr[t]);
                gr_ = (t == pi) ? 1.0f : nr;
                gi_ = (t == pi) ? 0.0f : ni;
                vr[t] = gr_;
                vi[t] = gi_;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                own_r[e] = h ? vr[4 + e] : vr[e];
                own_i[e] = h ? vi[4 + e] : vi[e];
            }
            pre_r = vr[0];
            pre_i = vi[0];
        }
        float rr = diag ? 0.f : gre, ri = diag ? 0.f : gim;
#pragma unroll
        for (int kc = 1; kc >= 0; --kc) {
            float fre[8], fim[8], fm[8];
#pragma unroll
            for (int g = 2 * kc + 1; g >= 2 * kc; --g) {
                const v4f qr = sv[(8 * g) / 4], qi4 = sv[(BK + 8 * g) / 4];
                const float tr[4] = {qr.x, qr.y, qr.z, qr.w};
                const float ti[4] = {qi4.x, qi4.y, qi4.z, qi4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = 4 * (g - 2 * kc) + e;
                    fre[k] = (g == gi) ? own_r[e] : fmaf(tr[e], rr, -(ti[e] * ri));
                    fim[k] = (g == gi) ? own_i[e] : fmaf(tr[e], ri, ti[e] * rr);
                }
                const float fr8 = s8[kb + 8 * g], fi8 = s8[BK + kb + 8 * g];
                const float nr = fmaf(fr8, rr, -(fi8 * ri));
                const float ni = fmaf(fr8, ri, fi8 * rr);
                rr = (g == gi) ? pre_r : nr;
                ri = (g == gi) ? pre_i : ni;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) fm[e] = Gm[8 * kc + e];
            weights(kc, msub, fre, fim, fm, false, true, true);
            __builtin_amdgcn_sched_barrier(0);
        }
        gre = rr;
        gim = ri;
        gm = rm_next;
    };
    auto settle_weights = [&]() __attribute__((always_inline)) {
        settle(wk.r[0]);
        settle(wk.r[1]);
        settle(wk.i[0]);
        settle(wk.i[1]);
        settle(z);
    };
    // an own-tile block (visit index kk = 0..7, highest keys first) is
    // skipped by the waves whose rows all lie above it
    auto own_active = [&](int kk) __attribute__((always_inline)) { return kk >= NDB - 1 - w; };
    auto flag_of = [&](const unsigned char *buf, int blk) __attribute__((always_inline)) {
        return reinterpret_cast<const uint32_t *>(buf + SM::flag_off)[blk];
    };

    MPrefetch pf;
    constexpr int NPRE = 2;  // fragments of each kind requested at the end of a vector step
    auto zero_w = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wk.r[kc][e] = (__bf16)0.0f;
                wk.i[kc][e] = (__bf16)0.0f;
            }
    };
    // ---- the key tiles before the query tile.  Tile m holds blocks 2m and
    // 2m+1.  Every wave runs its steps back to back, with one barrier per
    // tile: the leading waves (0..3) run M(2m) V(2m) M(2m+1) V(2m+1) before
    // it, the trailing ones (4..7) run V(2m+1) after it, so that the two
    // waves of a SIMD stay one step apart and alternate between matrix and
    // vector work.  Every wave issues its copies of tile m+2 after its matrix
    // step of block 2m (into the buffer of tile m-2, which every wave has
    // finished before the barrier closing tile m-1) and waits for its copies
    // of tile m+1 after its matrix step of block 2m+1, where wave 0 also lands
    // tile m+1; the barrier closing tile m publishes it.  The K fragments of
    // tile m+1 are therefore requested after that barrier (the leading waves
    // at the start of the next tile), the value fragments of the block before
    // at the end of the vector step.  Every matrix step runs the W~ V of the
    // block before it (W~ = 0 before the first block and after a block a wave
    // skips, so that it adds exact zeros) and the scores of its own block
    // (ignored by a wave that skips the block), one instruction sequence for
    // every block: vprev points at the value rows of the previous block.
    zero_w();
    const unsigned char *vprev = tile_buf(0) + vlane;
    if (n_off > 0)
        pstep_prefetch<D, DV, 0, 0, true, !QKZ, 0, NPRE>(vprev, tile_buf(0) + klane, pf);
    int m = 0;
    for (; m < n_off; ++m) {
        const unsigned char *bufm = tile_buf(m);
        const unsigned char *kb_ = bufm + klane;
        const unsigned char *vb_ = bufm + vlane;
        if (m > 0 && !lag) pstep_prefetch<D, DV, 0, 0, false, !QKZ, 0, NPRE>(vprev, kb_, pf);
        // block 2m (keys 0..31 of tile m)
        const uint32_t kflag0 = flag_of(bufm, 0);
        pstep<D, DV, 0, 0, true, !QKZ, NPRE>(vprev, kb_, pf, wk.r, wk.i, qf, ore, oim, x);
        issue(m + 2);
        vstep_off(bufm + slane, 0, wave_dead_rows || __builtin_amdgcn_readfirstlane(kflag0) != 0u);
        settle_weights();
        pstep_prefetch<D, DV, 0, 32, true, !QKZ, 0, NPRE>(vb_, kb_, pf);
        // block 2m+1 (keys 32..63)
        const uint32_t kflag1 = flag_of(bufm, 1);
        pstep<D, DV, 0, 32, true, !QKZ, NPRE>(vb_, kb_, pf, wk.r, wk.i, qf, ore, oim, x);
        vprev = vb_ + 32 * VSTR;
        land_wait(m);
        if (lag) lds_barrier();
        vstep_off(bufm + slane, 32, wave_dead_rows || __builtin_amdgcn_readfirstlane(kflag1) != 0u);
        settle_weights();
        if (lag && m + 1 < n_off)
            pstep_prefetch<D, DV, 0, 0, true, !QKZ, 0, NPRE>(vprev, tile_buf(m + 1) + klane, pf);
        else
            pstep_prefetch<D, DV, 0, 0, true, false, 0, NPRE>(vprev, vprev, pf);
        if (!lag) lds_barrier();
    }
    // ---- the query tile's own tiles: blocks visited highest keys first
    // (keys 32..63 of a tile, then 0..31); the block of visit index kk of the
    // NDB is active for wave w when kk >= NDB-1-w.  Every wave runs its active
    // blocks back to back: no buffer is written while a tile's blocks run
    // (the copies of the tile two ahead go to a buffer every wave has
    // finished), and one barrier per own tile publishes the next one, landed
    // by the copy waits before it.
    if (n_off > 0) {
        // the W~ V of the last block before the query tile; then the blocks
        // before the query tile are in O: rotate by P_i
        pstep<D, DV, 0, 0, true, false, NPRE>(vprev, vprev, pf, wk.r, wk.i, qf, ore, oim, x);
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float xr = ore[db][r], xi = oim[db][r];
                ore[db][r] = prow_re * xr - prow_im * xi;
                oim[db][r] = prow_re * xi + prow_im * xr;
            }
        z *= prow_m;
    }
    // until a wave's first active block its W~ is zero and the W~ V of the
    // step before that block reads the first own tile's values (never rewritten)
    zero_w();
    vprev = tile_buf(m) + vlane;
    for (int mm = 0; mm < NDIAG; ++mm, ++m) {
        const unsigned char *bufm = tile_buf(m);
        const unsigned char *kb_ = bufm + klane;
        const unsigned char *vb_ = bufm + vlane;
        const int tl = NDIAG - 1 - mm;  // key tile, counted from t_diag0
        issue(m + 2);
        if (own_active(2 * mm)) {  // keys 32..63 of the tile
            pstep_prefetch<D, DV, 0, 32, true, !QKZ, 0, NPRE>(vprev, kb_, pf);
            pstep<D, DV, 0, 32, true, !QKZ, NPRE>(vprev, kb_, pf, wk.r, wk.i, qf, ore, oim, x);
            vstep_own(bufm, 32, __builtin_amdgcn_readfirstlane(32 * w - (tl * BK + 32)) < 32);
            vprev = vb_ + 32 * VSTR;
        }
        if (own_active(2 * mm + 1)) {  // keys 0..31 of the tile
            pstep_prefetch<D, DV, 0, 0, true, !QKZ, 0, NPRE>(vprev, kb_, pf);
            pstep<D, DV, 0, 0, true, !QKZ, NPRE>(vprev, kb_, pf, wk.r, wk.i, qf, ore, oim, x);
            vstep_own(bufm, 0, __builtin_amdgcn_readfirstlane(32 * w - tl * BK) < 32);
            vprev = vb_;
        }
        land_wait(m);
        // wave 0 (whose rows see only the last own block) fetches the
        // workgroup's next item here, where its copies are in and it has
        // nothing else to do; the barrier publishes it
        if (mm == 0 && w == 0) misc[5] = uint32_t(next_item(A, home));
        lds_barrier();
    }
    // the last block's W~ V (keys 0..31 of the lowest own tile: every wave)
    pstep_prefetch<D, DV, 0, 0, true, false, 0, NPRE>(vprev, vprev, pf);
    pstep<D, DV, 0, 0, true, false, NPRE>(vprev, vprev, pf, wk.r, wk.i, qf, ore, oim, x);
    atomicMax(&misc[3], wave_max_u32(kbits));

    // ---- epilogue: O *= exp2((1-beta) M) z^-beta -------------------------
    const float zt = z + __shfl_xor(z, 32);
    float f;
    if (A.beta_mode == 1)
        f = 1.0f / zt;
    else if (A.beta_mode == 0)
        f = exp2f(M);
    else
        f = exp2f(A.one_minus_beta * M - A.beta * log2f(zt));
    // Stored through LDS: a lane holds 4-channel groups of its row, so stores
    // straight from the accumulators write 32 bytes in each of 32 rows per
    // instruction.  Once every wave has finished reading the tiles, each wave
    // stages its 32 rows, 64 channels at a time (rows of SROW floats, padded so
    // that the writes spread over the banks), and stores 16 lanes per row:
    // four rows of 256 contiguous bytes per instruction.
    lds_barrier();
    constexpr int SROW = 64 + 8;
    static_assert(size_t(NWAVES) * 32 * SROW * sizeof(float) <= SM::misc_off,
                  "staging fits the tile buffers");
    float *stg = reinterpret_cast<float *>(smem) + w * (32 * SROW);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
        float *op = part ? A.o_im : A.o_re;
#pragma unroll
        for (int half = 0; half < DV / 64; ++half) {
#pragma unroll
            for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    // channels 64 half + 32 dd + 8 g4 + 4 h .. +3 of row qi
                    const f32x16 &acc = part ? oim[2 * half + dd] : ore[2 * half + dd];
                    float4 v;
                    v.x = scale_keep_zero(acc[4 * g4 + 0], f);
                    v.y = scale_keep_zero(acc[4 * g4 + 1], f);
                    v.z = scale_keep_zero(acc[4 * g4 + 2], f);
                    v.w = scale_keep_zero(acc[4 * g4 + 3], f);
                    *reinterpret_cast<float4 *>(stg + qi * SROW + 32 * dd + 8 * g4 + 4 * h) = v;
                }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + (lane >> 4);  // row of the wave
                const float4 v =
                    *reinterpret_cast<const float4 *>(stg + r * SROW + 4 * (lane & 15));
                const int64_t grow = i0 + 32 * w + r;
                if (grow < A.n)
                    *reinterpret_cast<float4 *>(op + (bh * A.n + grow) * DV + 64 * half +
                                                4 * (lane & 15)) = v;
            }
        }
    }
    // (every wave's staged rows are read before the next item's copies
    // overwrite the buffers)
    __syncthreads();
    if (w == 0) {  // whole wave (the maxima are idempotent; lane 0 counts)
        const uint32_t qb = __builtin_amdgcn_readfirstlane(misc[2]);
        const uint32_t kb = __builtin_amdgcn_readfirstlane(misc[3]);
        atomicMax(&A.qstat[bh], qb);
        atomicMax(&A.kstat[bh], kb);
        if (qb >= kInfBits || kb >= kInfBits) A.status[0] = kNonFinite;
        atomicAdd(&A.counters[0], lane == 0 ? uint32_t(n_off) : 0u);
    }
}


// Fused forward, bf16 path: one workgroup per compute unit (the grid is at
// most the number of compute units), each taking query tiles from the work
// queues until they are empty.  Workgroup g starts on queue g mod nq: with
// nq = 8, the XCD that round-robin placement puts it on.
template <int D, int DV, bool QKZ>
__global__ __launch_bounds__(NTHREADS, 1) void fwd_pad_kernel(FwdArgs A) {
    using SM = PSmem<D, DV>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *misc = reinterpret_cast<uint32_t *>(smem + SM::misc_off);
    const int home = int(blockIdx.x) % A.nq;
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    typedef __attribute__((address_space(4))) const FwdArgs cfwd;
    // Every branch in this loop is uniform across each wave (wave 0 fetches
    // with all its lanes, and the item body's per-item bookkeeping runs in
    // whole waves too), so that every wave passes the same barriers.
    // the first item; each item's wave 0 fetches the next one during the
    // item (misc[5], published by the item's barriers)
    if (w == 0) misc[4] = uint32_t(next_item(A, home));  // every lane, one value
    __syncthreads();
    int it = __builtin_amdgcn_readfirstlane(int(misc[4]));
    while (it >= 0) {
        // the arguments are read afresh for every item, from the kernel's
        // argument segment (A is its only argument) through a pointer the
        // compiler cannot prove loop-invariant, instead of held in registers
        // across the loop
        cfwd *ap = (cfwd *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        fwd_pad_item<D, DV, QKZ>(*ap, it / A.n_qt, it % A.n_qt, home);
        it = __builtin_amdgcn_readfirstlane(int(misc[5]));
    }
}

// Refusal of an overflowing logit on the bf16 path (padded K tiles): as
// logit_check_kernel, staging each key tile with the padded copies.
template <int D>
__global__ __launch_bounds__(NTHREADS) void logit_check_pad_kernel(FwdArgs A) {
    constexpr int KSL = pad_kslots<D>();
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int go;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, qi = lane & 31;
    const int L = blockIdx.x;
    const int64_t qt = A.n_qt - 1 - L / A.BH;
    const int64_t bh = L % A.BH;
    if (tid == 0) {
        const uint32_t qm = A.qstat[bh], km = A.kstat[bh];
        const double bound = fabs((double)A.c) * (double)D * (double)__uint_as_float(qm) *
                             (double)__uint_as_float(km) * 1.01;
        go = !(bound < 3.0e38);
    }
    __syncthreads();
    if (!go) return;
    const int64_t i0 = qt * BQ;
    const int64_t row = i0 + 32 * w + qi;
    const bool row_ok = row < A.n;
    bf16x8 qf[D / 16];
    load_q<false, D>(A, bh, row, row_ok, h, qf);
    const unsigned char *kh, *vh;
    head_bases<false, D, D>(A, kv_head(A, bh), kh, vh);
    bool bad = false;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    for (int64_t t = 0; t < (i0 + BQ) / BK; ++t) {
        __syncthreads();
        for (int j = wu; j < KSL; j += NWAVES)
            g2lds16(kh, pad_kcopy_src_ragged<D>(j, lane, A.n, t), lds_addr(smem) + uint32_t(1024 * j));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const bf16x8 a =
                    *reinterpret_cast<const bf16x8 *>(smem + pad_kread<D>(32 * blk, st, qi, h));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s, 0, 0, 0);
            }
            {
#pragma clang fp contract(off)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t j = t * BK + 32 * blk + 8 * (r / 4) + 4 * h + (r % 4);
                    const float xx = s[r] * A.c;
                    if (row_ok && j <= row && j < A.n && !isfinite(xx)) bad = true;
                }
            }
        }
    }
    if (__any(bad) && lane == 0) A.status[0] = kNonFinite;
}

GatesArgs gates_args(const Layout &L, const float *u, const float *theta, double g,
                     unsigned char *ws, int32_t *status) {
    auto fptr = [&](int i) { return reinterpret_cast<float *>(ws + L.gate[i]); };
    auto dptr = [&](int i) { return reinterpret_cast<double *>(ws + L.tile[i]); };
    GatesArgs G;
    G.u = u;
    G.theta = theta;
    G.g = g;
    G.n = L.n;
    G.n_pad = L.n_pad;
    G.ldu = L.n;
    G.n_qt = (int)L.n_qt;
    G.n_kt = (int)L.n_kt;
    G.BH = L.BH;
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
    G.t4 = reinterpret_cast<double *>(ws + L.tile4);
    G.status = status;
    return G;
}

// Compute units of the current device, looked up once per device.
int compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <bool F32, int D, int DV>
int launch_typed(const Problem &P, hipStream_t st, hipEvent_t const *marks) {
    const Layout &L = P.L;
    unsigned char *ws = P.ws;
    uint32_t *counters = reinterpret_cast<uint32_t *>(ws + L.counters);
    if (marks) (void)hipEventRecord(marks[0], st);
    const int BH = (int)L.BH;

    // gates (four query tiles per block) and, on the bf16 path with fp32
    // values, their rounding to bf16 (2048 values per block) in one launch
    const GatesArgs G = gates_args(L, P.u, P.theta, P.g, ws, P.status);
    int32_t *gbad = reinterpret_cast<int32_t *>(ws + L.gbad);
    const int ngb = (int)((BH * L.n_qt + 3) / 4);
    uint16_t *v16 = reinterpret_cast<uint16_t *>(ws + L.v16);
    const int64_t count8 = L.BHkv * L.n * DV / 8;
    if (!F32 && P.v_f32) {
        const unsigned blocks = (unsigned)(ngb + (count8 + 255) / 256);
        hipLaunchKernelGGL(prep_kernel<true>, dim3(blocks), dim3(256), 0, st, G, ngb, gbad,
                           static_cast<const float *>(P.v), v16, count8, counters);
    } else {
        hipLaunchKernelGGL(prep_kernel<false>, dim3(ngb), dim3(256), 0, st, G, ngb, gbad,
                           static_cast<const float *>(P.v), v16, count8, counters);
    }
    int32_t *noff = reinterpret_cast<int32_t *>(ws + L.noff);
    hipLaunchKernelGGL(schedule_kernel, dim3(BH * L.n_qt), dim3(64), 0, st, G.t_re, G.t_im,
                       G.t_m, (int)L.n_kt, (int)L.n_qt, noff,
                       reinterpret_cast<uint32_t *>(ws + L.qstat),
                       reinterpret_cast<uint32_t *>(ws + L.kstat), gbad, P.status);

    FwdArgs F;
    F.q = P.q;
    F.k = P.k;
    F.v = P.v;
    F.v16 = P.v_f32 ? reinterpret_cast<const uint16_t *>(ws + L.v16)
                    : static_cast<const uint16_t *>(P.v);
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
    F.t4 = G.t4;
    F.gates = G.a_re;
    F.plane = int64_t(L.gate[1] - L.gate[0]) / int64_t(sizeof(float));
    F.o_re = P.o_re;
    F.o_im = P.o_im;
    F.qstat = reinterpret_cast<uint32_t *>(ws + L.qstat);
    F.kstat = reinterpret_cast<uint32_t *>(ws + L.kstat);
    F.counters = counters;
    F.queues = counters + 8;
    F.nq = (BH & 7) == 0 ? 8 : 1;
    // one head at a time per queue, so that the 32 compute units of an XCD
    // read one head's keys and values, which its L2 holds (heaviest query
    // tile first across the queue's heads balances the end better but reads
    // more from HBM: every item 5% slower at B=4 H=16 n=8192); the light
    // query tiles (the lowest sixth) of every head come last, heaviest first,
    // to fill the end (1.317 -> 1.292 ms there; a quarter or an eighth of the
    // query tiles does as well, a half does not)
    F.order = 2;
    F.q0 = (int)(L.n_qt / 6);
    F.noff = noff;
    F.status = P.status;
    F.n = L.n;
    F.n_pad = L.n_pad;
    F.n_qt = (int)L.n_qt;
    F.n_kt = (int)L.n_kt;
    F.BH = BH;
    F.H = (int)L.H;
    F.group = (int)(L.H / L.Hkv);
    F.c = P.c;
    F.beta = P.beta;
    F.one_minus_beta = 1.0f - P.beta;
    F.beta_mode = P.beta_mode;
    F.qk_zero = P.qk_zero ? 1 : 0;
    if constexpr (F32) {
        const size_t shm = Smem<D, DV>::bytes;
        if (shm > 65536) {
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_kernel<D, DV, false>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_kernel<D, DV, true>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&logit_check_kernel<D>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        }
        if (marks) (void)hipEventRecord(marks[1], st);
        if (P.qk_zero)
            hipLaunchKernelGGL((fwd_kernel<D, DV, true>), dim3(BH * L.n_qt), dim3(NTHREADS),
                               shm, st, F);
        else
            hipLaunchKernelGGL((fwd_kernel<D, DV, false>), dim3(BH * L.n_qt), dim3(NTHREADS),
                               shm, st, F);
        if (marks) (void)hipEventRecord(marks[2], st);
        if (!P.qk_zero)
            hipLaunchKernelGGL((logit_check_kernel<D>), dim3(BH * L.n_qt), dim3(NTHREADS),
                               shm, st, F);
    } else {
        const size_t shm = PSmem<D, DV>::bytes;
        if (shm > 65536) {
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_pad_kernel<D, DV, false>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_pad_kernel<D, DV, true>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&logit_check_pad_kernel<D>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        }
        if (marks) (void)hipEventRecord(marks[1], st);
        // one workgroup per compute unit (fewer when there are fewer query tiles)
        const int64_t items = int64_t(BH) * L.n_qt;
        const unsigned grid = (unsigned)std::min<int64_t>(items, compute_units());
        if (P.qk_zero)
            hipLaunchKernelGGL((fwd_pad_kernel<D, DV, true>), dim3(grid), dim3(NTHREADS), shm, st,
                               F);
        else
            hipLaunchKernelGGL((fwd_pad_kernel<D, DV, false>), dim3(grid), dim3(NTHREADS), shm,
                               st, F);
        if (marks) (void)hipEventRecord(marks[2], st);
        if (!P.qk_zero)
            hipLaunchKernelGGL((logit_check_pad_kernel<D>), dim3(BH * L.n_qt), dim3(NTHREADS),
                               shm, st, F);
    }
    if (marks) (void)hipEventRecord(marks[3], st);
    return (int)hipGetLastError();
}

}  // namespace

int launch_gates(const Layout &L, const float *u, const float *theta, double g,
                 unsigned char *ws, int32_t *status, void *stream, int64_t ldu) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t *counters = reinterpret_cast<uint32_t *>(ws + L.counters);
    hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, st, status, counters);
    GatesArgs G = gates_args(L, u, theta, g, ws, status);
    if (ldu > 0) G.ldu = ldu;
    hipLaunchKernelGGL(gates_kernel, dim3(L.BH * L.n_qt), dim3(64), 0, st, G);
    return (int)hipGetLastError();
}

int launch_forward(const Problem &P, void *stream, void *const *marks) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t const *ev = reinterpret_cast<hipEvent_t const *>(marks);
    const bool f32 = !P.L.bf16_path;
    const int64_t d = P.L.d, dv = P.L.dv;
    if (d == 64 && dv == 64)
        return f32 ? launch_typed<true, 64, 64>(P, st, ev) : launch_typed<false, 64, 64>(P, st, ev);
    if (d == 64 && dv == 128)
        return f32 ? launch_typed<true, 64, 128>(P, st, ev)
                   : launch_typed<false, 64, 128>(P, st, ev);
    if (d == 128 && dv == 64)
        return f32 ? launch_typed<true, 128, 64>(P, st, ev)
                   : launch_typed<false, 128, 64>(P, st, ev);
    return f32 ? launch_typed<true, 128, 128>(P, st, ev)
               : launch_typed<false, 128, 128>(P, st, ev);
}

}  // namespace resolvent
