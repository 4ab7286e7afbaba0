// decode_kernels.hip -- one decode step of the resolvent head (gfx950): the
// readout of the newest position, i = n-1, against the cached keys and values
// of positions 0..n-1 ("Resolvent Operator" page, section "Object", for the
// last row):
//     O_i = sum_{j<=i} G_ij e^{qk s_ij} V_j / Z_i^beta,   G_ij = a_{j+1} ... a_i.
// Positions are grouped in chunks of DEC_CT key tiles (256 positions).  For
// key j of chunk c, G_ij = C_c S_j: S_j the product of the gates after j up
// to the chunk's end, C_c = P_{c+1} ... P_{n_ch-1} the product of every gate
// after the chunk (P: the chunk products).  A chunk's partial sums are taken
// relative to its own end, so the chunks need nothing from one another; the
// carries C_c scale the partials in the merge.  Kernels, in stream order:
//   decode_part_kernel    one wave per chunk: its gates from u, theta in f64
//                         with suffix scans across lanes, the logits of every
//                         key (the refusal needs them all), the weights with an
//                         online shift and their V contraction -> partial
//                         (M, z, O) and the chunk product P_c; clears the
//                         status word (block 0)
//   decode_merge_kernel   one workgroup per head (decode_merge_small_kernel
//                         for heads of few chunks): the carries C_c by a suffix
//                         scan of the chunk products, then
//                         O = sum_c C_c 2^(M_c - M) O_c, z likewise with |C_c|,
//                         scaled by exp2((1-beta) M) z^-beta; sets the status
//                         word when a chunk refused its inputs
// Weights and sums are float32 (products of gates f64): the weights are not
// rounded to bf16 here.  Logits are in log2 units (c = qk log2(e) / sqrt(d)).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"
#include "layout.h"

namespace resolvent {
namespace {

using namespace dev;

constexpr int32_t kDecNonFinite = 1;

struct DecodeArgs {
    const void *q, *k, *v;           // q [BH][d]; k [BHkv][cap][d]; v [BHkv][cap][dv]
    const float *u, *theta;          // [BH][cap]
    double *p_re, *p_im, *p_m;       // chunk products [BH][n_ch]
    float4 *scale;                   // per chunk (re, im, modulus, 0) of C_c 2^(M_c - M)
    float *part;                     // [BH][n_ch][4 + 2 dv]: M, z, refused, 0, O_re[dv], O_im[dv]
    float *o_re, *o_im;              // [BH][dv]
    int32_t *status;
    double g;
    int64_t n, cap;                  // cap: positions per head in k, v, u, theta (>= n)
    int n_ch, H, group;              // group = query heads per k/v head
    float c, beta, one_minus_beta;
    int beta_mode, qk_zero;
};

// One wave per (head, chunk): blockIdx.x = bh n_ch + chunk.  The chunk's
// tiles are taken last to first, so that the product from each to the
// chunk's end is the one after it times that tile's product.  Key rows are
// read KL lanes to a row (16 bytes a lane: one instruction covers KR whole
// rows) and their dot products reduced across those lanes; value rows the same
// way, VL lanes to a row, each lane accumulating VE channels of VR interleaved
// row groups that are summed at the end.
template <bool QF32, bool VF32, int D, int DV>
__global__ __launch_bounds__(64) void decode_part_kernel(DecodeArgs A) {
    constexpr int KE = QF32 ? 4 : 8, KL = D / KE, KR = 64 / KL, KI = BK / KR;
    constexpr int VE = VF32 ? 4 : 8, VL = DV / VE, VR = 64 / VL, VI = BK / VR;
    constexpr int KB = QF32 ? 4 : 2, VB = VF32 ? 4 : 2;  // element bytes
    constexpr int64_t PF = dec_part_floats(DV);
    static_assert(KL <= 64 && VL <= 64 && BK % KR == 0 && BK % VR == 0, "row split");
    __shared__ float dots[BK], wr_s[BK], wi_s[BK];
    const int lane = threadIdx.x;
    const int64_t bh = blockIdx.x / A.n_ch;
    const int ch = int(blockIdx.x % A.n_ch);
    const int64_t kvh = (bh / A.H) * (A.H / A.group) + (bh % A.H) / A.group;
    const int64_t i = A.n - 1;
    const int kc = (lane % KL) * KE, kr = lane / KL;
    const int vc = (lane % VL) * VE, vr = lane / VL;
    const uint32_t koff = uint32_t(kc * KB), voff = uint32_t(vc * VB);
    const char *kbase = static_cast<const char *>(A.k) + kvh * A.cap * (D * KB);
    const char *vbase = static_cast<const char *>(A.v) + kvh * A.cap * (DV * VB);
    const float *ub = A.u + bh * A.cap, *tb = A.theta + bh * A.cap;
    if (blockIdx.x == 0 && lane == 0) A.status[0] = 0;  // set again by the merge
    bool bad = false;
    float qv[KE];
    unpack16<QF32>(load16<QF32>(A.q, bh * D + kc), qv);
#pragma unroll
    for (int e = 0; e < KE; ++e)
        if (!isfinite(qv[e])) bad = true;
    Cg carry = cg_one();  // the gates from the current tile's end to the chunk's end
    float M = -INFINITY;  // shift (log2 units) of this chunk's live logits
    float z = 0.f;        // this lane's share of the normaliser
    float ore[VE], oim[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        ore[e] = 0.f;
        oim[e] = 0.f;
    }
    // The chunk's last tile holding keys (the tiles after it lie past i).  Rows
    // past the last key re-read the last key's row (their weight is 0);
    // per-tile bases are uniform, the lanes' offsets 32-bit.
    const int last = (i - int64_t(ch) * DEC_CHUNK) / BK < DEC_CT - 1
                         ? int((i - int64_t(ch) * DEC_CHUNK) / BK)
                         : DEC_CT - 1;
    uint4 kw[KI];
    auto load_k = [&](int tt) {
        const int64_t t0 = int64_t(ch) * DEC_CHUNK + tt * BK;
        const int cnt = i - t0 + 1 < BK ? int(i - t0 + 1) : BK;
        const char *kt = kbase + t0 * (D * KB);
#pragma unroll
        for (int x = 0; x < KI; ++x) {
            const int row = x * KR + kr < cnt ? x * KR + kr : cnt - 1;
            kw[x] = *reinterpret_cast<const uint4 *>(kt + (uint32_t(row) * (D * KB) + koff));
        }
    };
    // Phase 1, the chunk's gates (every position is checked): per tile, from the
    // last to the first, the suffix products across lanes and this lane's
    // key's product to the chunk's end (float), the carry moving one tile back
    // each time.  A zero carry closes every key of the tile and of the tiles
    // before it.
    float gr[DEC_CT], gi[DEC_CT], gm[DEC_CT];
    bool open[DEC_CT];
#pragma unroll
    for (int tt = DEC_CT - 1; tt >= 0; --tt) {
        const int64_t t0 = int64_t(ch) * DEC_CHUNK + tt * BK;
        open[tt] = carry.m != 0.0;
        gr[tt] = gi[tt] = gm[tt] = 0.f;
        if (t0 > i) continue;  // past the newest position: identity gates
        const int64_t j = t0 + lane;
        Cg sfx = cg_one();
        if (j < A.n) sfx = gate_of(ub[j], tb[j], A.g, bad);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const Cg x = cg_down(sfx, o);
            if (lane + o < 64) sfx = cg_mul(sfx, x);
        }
        Cg after = cg_down(sfx, 1);  // the gates after this lane's key in the tile
        if (lane == 63) after = cg_one();
        const Cg G = cg_mul(carry, after);
        gr[tt] = float(G.re);
        gi[tt] = float(G.im);
        gm[tt] = float(G.m);
        carry = cg_mul(cg_lane(sfx, 0), carry);
    }
    // Phase 2, the rows, tile by tile: the key rows, the logits, the weights,
    // then the value rows and their contraction.  (Requesting the next tile's
    // keys early, or a tile's values with its keys, holds more registers and
    // measured slower.)
#pragma unroll
    for (int tt = DEC_CT - 1; tt >= 0; --tt) {
        if (tt > last) continue;  // past the newest position: no keys
        const int64_t t0 = int64_t(ch) * DEC_CHUNK + tt * BK;
        const int cnt = i - t0 + 1 < BK ? int(i - t0 + 1) : BK;  // keys in the tile
        const char *vt = vbase + t0 * (DV * VB);
        load_k(tt);
        uint4 vw[VI];
        auto load_v = [&]() {
#pragma unroll
            for (int x = 0; x < VI; ++x) {
                const int row = x * VR + vr < cnt ? x * VR + vr : cnt - 1;
                vw[x] = *reinterpret_cast<const uint4 *>(vt + (uint32_t(row) * (DV * VB) + voff));
            }
        };
        // the logit of every key (the refusal covers them all)
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
        const float rm = gm[tt];
        const bool live = open[tt] && key && rm > 0.0f;
        const float tmax = wave_max(live ? L : -INFINITY);
        if (tmax == -INFINITY) {  // no live key in the tile
            __syncthreads();
            continue;
        }
        if (tmax > M) {  // new shift: rescale what this chunk holds
            const float alpha = M == -INFINITY ? 0.f : exp2f(M - tmax);
            z *= alpha;
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                ore[e] *= alpha;
                oim[e] *= alpha;
            }
            M = tmax;
        }
        const float ex = live ? exp2f(L - M) : 0.f;
        z = fmaf(rm, ex, z);
        wr_s[lane] = gr[tt] * ex;
        wi_s[lane] = gi[tt] * ex;
        __syncthreads();
        // O += sum_j w_j V_j
        load_v();
#pragma unroll
        for (int x = 0; x < VI; ++x) {
            float vx[VE];
            unpack16<VF32>(vw[x], vx);
            const float a = wr_s[x * VR + vr], b = wi_s[x * VR + vr];
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                ore[e] = fmaf(a, vx[e], ore[e]);
                oim[e] = fmaf(b, vx[e], oim[e]);
            }
        }
        __syncthreads();
    }
    const bool refused = __any(bad);
    // sum the VR row groups: lanes 0..VL-1 end with the chunk's channel sums
#pragma unroll
    for (int o = VL; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            ore[e] += __shfl_xor(ore[e], o);
            oim[e] += __shfl_xor(oim[e], o);
        }
    const float zt = wave_sum(z);
    float *p = A.part + (bh * A.n_ch + ch) * PF;
    if (lane == 0) {
        *reinterpret_cast<float4 *>(p) = make_float4(M, zt, refused ? 1.f : 0.f, 0.f);
        const int64_t x = bh * A.n_ch + ch;
        A.p_re[x] = carry.re;
        A.p_im[x] = carry.im;
        A.p_m[x] = carry.m;
    }
    if (lane < VL) {
#pragma unroll
        for (int e = 0; e < VE; e += 4) {
            *reinterpret_cast<float4 *>(p + 4 + vc + e) =
                make_float4(ore[e], ore[e + 1], ore[e + 2], ore[e + 3]);
            *reinterpret_cast<float4 *>(p + 4 + DV + vc + e) =
                make_float4(oim[e], oim[e + 1], oim[e + 2], oim[e + 3]);
        }
    }
}

// One workgroup of MW waves per head.  Thread t owns a segment of
// consecutive chunks: it multiplies their products, an exclusive suffix scan
// across the threads (within each wave, then across the waves through LDS)
// gives the segment the product of everything after it, and walking the
// segment back to front gives each chunk its carry C_c.  The shift M is the
// largest M_c of the chunks with C_c != 0; a second walk stores each chunk's
// scale s_c = C_c 2^(M_c - M) (0 for a closed chunk) as (re, im, |s|, 0).  Then thread (r, ch) sums channel ch of s_c O_c over the
// chunks c = r mod (NT / DV) and the groups are added in LDS.
constexpr int MW = 4;
template <int DV>
__global__ __launch_bounds__(64 * MW) void decode_merge_kernel(DecodeArgs A) {
    constexpr int NT = 64 * MW, NG = NT / DV;  // threads, chunk groups
    constexpr int64_t PF = dec_part_floats(DV);
    __shared__ double wtot[3][MW];
    __shared__ float red[MW];
    __shared__ float ore_s[NG][DV], oim_s[NG][DV];
    __shared__ float zs[NG];
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
    const int64_t bh = blockIdx.x;
    const int n_ch = A.n_ch;
    const int64_t base = bh * n_ch;
    const float *p0 = A.part + base * PF;
    float4 *scale = A.scale + base;
    // ---- carries ----------------------------------------------------------
    const int seg = (n_ch + NT - 1) / NT;
    const int c0 = tid * seg < n_ch ? tid * seg : n_ch;
    const int c1 = c0 + seg < n_ch ? c0 + seg : n_ch;
    auto prod = [&](int c) { return Cg{A.p_re[base + c], A.p_im[base + c], A.p_m[base + c]}; };
    Cg q = cg_one();
    for (int c = c0; c < c1; ++c) q = cg_mul(q, prod(c));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {  // inclusive suffix inside the wave
        const Cg x = cg_down(q, o);
        if (lane + o < 64) q = cg_mul(q, x);
    }
    if (lane == 0) {
        wtot[0][w] = q.re;
        wtot[1][w] = q.im;
        wtot[2][w] = q.m;
    }
    __syncthreads();
    Cg after = cg_down(q, 1);  // the product of the later threads' segments
    if (lane == 63) after = cg_one();
    for (int v = w + 1; v < MW; ++v) after = cg_mul(after, Cg{wtot[0][v], wtot[1][v], wtot[2][v]});
    // ---- the shift, and refusals -------------------------------------------
    float Mh = -INFINITY;
    bool refused = false;
    {
        Cg x = after;
        for (int c = c1 - 1; c >= c0; --c) {
            const float4 hd = *reinterpret_cast<const float4 *>(p0 + c * PF);
            if (x.m > 0.0) Mh = fmaxf(Mh, hd.x);
            if (hd.z != 0.f) refused = true;
            x = cg_mul(prod(c), x);
        }
    }
    Mh = wave_max(Mh);
    if (lane == 0) red[w] = Mh;
    refused = __syncthreads_or(refused);
    Mh = red[0];
#pragma unroll
    for (int v = 1; v < MW; ++v) Mh = fmaxf(Mh, red[v]);
    if (refused) {
        if (tid == 0) A.status[0] = kDecNonFinite;
        return;  // the outputs are unspecified
    }
    {
        Cg x = after;
        for (int c = c1 - 1; c >= c0; --c) {
            const float mc = p0[c * PF];
            float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
            if (x.m > 0.0 && mc != -INFINITY) {
                const double e = (double)exp2f(mc - Mh);
                sc = make_float4(float(x.re * e), float(x.im * e), float(x.m * e), 0.f);
            }
            scale[c] = sc;
            x = cg_mul(prod(c), x);
        }
    }
    __syncthreads();  // the scales are read below by other threads
    // ---- O = sum_c s_c O_c, z = sum_c |s_c| z_c ------------------------------
    const int r = tid / DV, chn = tid % DV;
    float hre = 0.f, him = 0.f, zh = 0.f;
#pragma unroll 8
    for (int c = r; c < n_ch; c += NG) {
        const float *pc = p0 + c * PF;
        const float4 sc = scale[c];
        const float a = pc[4 + chn], b = pc[4 + DV + chn], zc = pc[1];
        hre = fmaf(sc.x, a, fmaf(-sc.y, b, hre));
        him = fmaf(sc.x, b, fmaf(sc.y, a, him));
        zh = fmaf(sc.z, zc, zh);
    }
    ore_s[r][chn] = hre;
    oim_s[r][chn] = him;
    if (chn == 0) zs[r] = zh;
    __syncthreads();
    if (tid < DV) {
        float sr = 0.f, si = 0.f, z = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            sr += ore_s[g][tid];
            si += oim_s[g][tid];
            z += zs[g];
        }
        float f;
        if (A.beta_mode == 1)
            f = 1.0f / z;
        else if (A.beta_mode == 0)
            f = exp2f(Mh);
        else
            f = exp2f(A.one_minus_beta * Mh - A.beta * log2f(z));
        A.o_re[bh * DV + tid] = scale_keep_zero(sr, f);
        A.o_im[bh * DV + tid] = scale_keep_zero(si, f);
    }
}

// The same merge for a head of at most NG NX chunks (NG = 256 / DV chunk
// groups): every load it needs -- the chunk products and headers (one chunk
// per thread) and this thread's channel of each of its NX chunks' partials --
// is issued first, so the merge takes one trip to memory; the carries come
// from a suffix scan across the threads (lanes, then waves through LDS), and
// the scales go through LDS.
template <int DV, int NX>
__global__ __launch_bounds__(64 * MW) void decode_merge_small_kernel(DecodeArgs A) {
    constexpr int NT = 64 * MW, NG = NT / DV;
    constexpr int64_t PF = dec_part_floats(DV);
    static_assert(NG * NX <= NT, "one chunk per thread");
    __shared__ double wtot[3][MW];
    __shared__ float red[MW];
    __shared__ float4 sc_s[NG * NX];
    __shared__ float ore_s[NG][DV], oim_s[NG][DV];
    __shared__ float zs[NG];
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
    const int64_t bh = blockIdx.x;
    const int n_ch = A.n_ch;
    const int64_t base = bh * n_ch;
    const float *p0 = A.part + base * PF;
    const int r = tid / DV, chn = tid % DV;
    // ---- every load, up front ---------------------------------------------
    const bool mine = tid < n_ch;  // thread tid owns chunk tid
    Cg q = cg_one();
    float4 hd = make_float4(-INFINITY, 0.f, 0.f, 0.f);
    if (mine) {
        q = Cg{A.p_re[base + tid], A.p_im[base + tid], A.p_m[base + tid]};
        hd = *reinterpret_cast<const float4 *>(p0 + tid * PF);
    }
    float ar[NX], ai[NX], zc[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int c = r + NG * x;
        const bool ok = c < n_ch;
        const float *pc = p0 + (ok ? c : 0) * PF;
        ar[x] = ok ? pc[4 + chn] : 0.f;
        ai[x] = ok ? pc[4 + DV + chn] : 0.f;
        zc[x] = ok ? pc[1] : 0.f;
    }
    // ---- carries: C_c = the product of the chunk products after c -----------
    Cg incl = q;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {  // inclusive suffix inside the wave
        const Cg x = cg_down(incl, o);
        if (lane + o < 64) incl = cg_mul(incl, x);
    }
    if (lane == 0) {
        wtot[0][w] = incl.re;
        wtot[1][w] = incl.im;
        wtot[2][w] = incl.m;
    }
    __syncthreads();
    Cg C = cg_down(incl, 1);
    if (lane == 63) C = cg_one();
    for (int v = w + 1; v < MW; ++v) C = cg_mul(C, Cg{wtot[0][v], wtot[1][v], wtot[2][v]});
    // ---- the shift over the chunks that reach position i, and refusals -------
    float Mh = (mine && C.m > 0.0) ? hd.x : -INFINITY;
    const bool refused_here = mine && hd.z != 0.f;
    Mh = wave_max(Mh);
    if (lane == 0) red[w] = Mh;
    const bool refused = __syncthreads_or(refused_here);
    Mh = red[0];
#pragma unroll
    for (int v = 1; v < MW; ++v) Mh = fmaxf(Mh, red[v]);
    if (refused) {
        if (tid == 0) A.status[0] = kDecNonFinite;
        return;  // the outputs are unspecified
    }
    if (mine) {
        float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (C.m > 0.0 && hd.x != -INFINITY) {
            const double e = (double)exp2f(hd.x - Mh);
            sc = make_float4(float(C.re * e), float(C.im * e), float(C.m * e), 0.f);
        }
        sc_s[tid] = sc;
    }
    __syncthreads();
    // ---- O = sum_c s_c O_c, z = sum_c |s_c| z_c ------------------------------
    float hre = 0.f, him = 0.f, zh = 0.f;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int c = r + NG * x;
        if (c < n_ch) {
            const float4 sc = sc_s[c];
            hre = fmaf(sc.x, ar[x], fmaf(-sc.y, ai[x], hre));
            him = fmaf(sc.x, ai[x], fmaf(sc.y, ar[x], him));
            zh = fmaf(sc.z, zc[x], zh);
        }
    }
    ore_s[r][chn] = hre;
    oim_s[r][chn] = him;
    if (chn == 0) zs[r] = zh;
    __syncthreads();
    if (tid < DV) {
        float sr = 0.f, si = 0.f, z = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            sr += ore_s[g][tid];
            si += oim_s[g][tid];
            z += zs[g];
        }
        float f;
        if (A.beta_mode == 1)
            f = 1.0f / z;
        else if (A.beta_mode == 0)
            f = exp2f(Mh);
        else
            f = exp2f(A.one_minus_beta * Mh - A.beta * log2f(z));
        A.o_re[bh * DV + tid] = scale_keep_zero(sr, f);
        A.o_im[bh * DV + tid] = scale_keep_zero(si, f);
    }
}

template <bool F32>
__device__ __forceinline__ float load_e(const void *p, int64_t i) {
    if constexpr (F32) {
        return static_cast<const float *>(p)[i];
    } else {
        const uint16_t b = static_cast<const uint16_t *>(p)[i];
        return __uint_as_float(uint32_t(b) << 16);
    }
}

// One chain step per (head, channel): y <- a y + v with a = gate(blend(u, theta, g)).
__global__ __launch_bounds__(64) void chain_step_kernel(float *y_re, float *y_im, const float *u,
                                                        const float *theta, const void *v,
                                                        bool v_f32, double g, int64_t BH,
                                                        int dv, int32_t *status) {
    const int64_t x = int64_t(blockIdx.x) * 64 + threadIdx.x;
    if (x >= BH * dv) return;
    const int64_t bh = x / dv;
    bool bad = false;
    const Cg a = gate_of(u[bh], theta[bh], g, bad);
    if (bad) {
        status[0] = kDecNonFinite;
        return;
    }
    const float ar = (float)a.re, ai = (float)a.im;
    const float vv = v_f32 ? static_cast<const float *>(v)[x] : load_e<false>(v, x);
    const float yr = y_re[x], yi = y_im[x];
    y_re[x] = ar * yr - ai * yi + vv;
    y_im[x] = ar * yi + ai * yr;
}

template <bool QF32, bool VF32, int D, int DV>
void launch_part(const DecodeArgs &A, hipStream_t st, int64_t BH) {
    hipLaunchKernelGGL((decode_part_kernel<QF32, VF32, D, DV>), dim3((unsigned)(BH * A.n_ch)),
                       dim3(64), 0, st, A);
}

}  // namespace

int launch_decode(const DecodeLayout &DL, const void *q, const void *k, const float *u,
                  const float *theta, const void *v, int64_t cap, bool qk_f32, bool v_f32,
                  double g, float c, float beta, int beta_mode, bool qk_zero, float *o_re,
                  float *o_im, unsigned char *ws, int32_t *status, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t per = sizeof(double) * size_t(DL.BH) * size_t(DL.n_ch);
    DecodeArgs A;
    A.q = q;
    A.k = k;
    A.v = v;
    A.u = u;
    A.theta = theta;
    A.p_re = reinterpret_cast<double *>(ws + DL.prod);
    A.p_im = reinterpret_cast<double *>(ws + DL.prod + per);
    A.p_m = reinterpret_cast<double *>(ws + DL.prod + 2 * per);
    A.scale = reinterpret_cast<float4 *>(ws + DL.scale);
    A.part = reinterpret_cast<float *>(ws + DL.part);
    A.o_re = o_re;
    A.o_im = o_im;
    A.status = status;
    A.g = g;
    A.n = DL.n;
    A.cap = cap;
    A.n_ch = (int)DL.n_ch;
    A.H = (int)DL.H;
    A.group = (int)(DL.H / DL.Hkv);
    A.c = c;
    A.beta = beta;
    A.one_minus_beta = 1.0f - beta;
    A.beta_mode = beta_mode;
    A.qk_zero = qk_zero ? 1 : 0;
    const int64_t BH = DL.BH;
    const int key = (qk_f32 ? 8 : 0) + (v_f32 ? 4 : 0) + (DL.d == 128 ? 2 : 0) +
                    (DL.dv == 128 ? 1 : 0);
    switch (key) {
        case 0: launch_part<false, false, 64, 64>(A, st, BH); break;
        case 1: launch_part<false, false, 64, 128>(A, st, BH); break;
        case 2: launch_part<false, false, 128, 64>(A, st, BH); break;
        case 3: launch_part<false, false, 128, 128>(A, st, BH); break;
        case 4: launch_part<false, true, 64, 64>(A, st, BH); break;
        case 5: launch_part<false, true, 64, 128>(A, st, BH); break;
        case 6: launch_part<false, true, 128, 64>(A, st, BH); break;
        case 7: launch_part<false, true, 128, 128>(A, st, BH); break;
        case 12: launch_part<true, true, 64, 64>(A, st, BH); break;
        case 13: launch_part<true, true, 64, 128>(A, st, BH); break;
        case 14: launch_part<true, true, 128, 64>(A, st, BH); break;
        case 15: launch_part<true, true, 128, 128>(A, st, BH); break;
        default: return (int)hipErrorInvalidValue;
    }
    // heads of few chunks (up to 16 per chunk group) take the one-trip merge
    if (DL.dv == 128 && DL.n_ch <= 2 * 16)
        hipLaunchKernelGGL((decode_merge_small_kernel<128, 16>), dim3((unsigned)BH), dim3(64 * MW),
                           0, st, A);
    else if (DL.dv == 64 && DL.n_ch <= 4 * 16)
        hipLaunchKernelGGL((decode_merge_small_kernel<64, 16>), dim3((unsigned)BH), dim3(64 * MW),
                           0, st, A);
    else if (DL.dv == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((unsigned)BH), dim3(64 * MW), 0, st, A);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((unsigned)BH), dim3(64 * MW), 0, st, A);
    return (int)hipGetLastError();
}

int launch_chain_step(float *y_re, float *y_im, const float *u, const float *theta,
                      const void *v, bool v_f32, double g, int64_t BH, int64_t dv,
                      int32_t *status, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t total = BH * dv;
    hipLaunchKernelGGL(chain_step_kernel, dim3((unsigned)((total + 63) / 64)), dim3(64), 0, st,
                       y_re, y_im, u, theta, v, v_f32, g, BH, (int)dv, status);
    return (int)hipGetLastError();
}

}  // namespace resolvent
