// layout.h -- tile sizes and the device-workspace layout of the resolvent
// forward pass (shared by the host entry points and the kernel launchers).
#pragma once

#include <cstddef>
#include <cstdint>

#if defined(__HIPCC__)
#define RESOLVENT_HD __host__ __device__
#else
#define RESOLVENT_HD
#endif

namespace resolvent {

// A workgroup owns BQ consecutive queries (NWAVES waves of 32 rows); keys are
// staged BK at a time.  Gate scans use the same tiling: an inclusive prefix
// inside each query tile and an exclusive suffix inside each key tile.
constexpr int NWAVES = 8;
constexpr int BQ = 32 * NWAVES;
constexpr int BK = 64;
static_assert(BQ % BK == 0, "a query tile must hold whole key tiles");

constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    int64_t BH = 0, n = 0, d = 0;
    int64_t H = 0, Hkv = 0, BHkv = 0, dv = 0;  // query heads per batch entry; k/v heads;
                                               // k/v heads in all; value channels
    int64_t n_pad = 0, n_qt = 0, n_kt = 0;
    bool bf16_path = true;
    // byte offsets into the workspace
    size_t gate[9] = {};  // a_re a_im a_m | s_re s_im s_m | p_re p_im p_m  (float [BH][n_pad])
    size_t tile[3] = {};  // A_re A_im A_m per key tile (double [BH][n_kt])
    size_t tile4 = 0;     // the same packed, (A_re, A_im, A_m, 0) per key tile (double4 [BH][n_kt])
    size_t qstat = 0, kstat = 0;  // per head max |q|, max |k| bits (uint32 [BH])
    size_t noff = 0;  // per query tile: key tiles before it that the forward visits (int32 [BH][n_qt])
    size_t gbad = 0;  // per query tile: 1 if its gates saw a refused input (int32 [BH][n_qt])
    size_t counters = 0;  // uint32 [16]: key tiles processed before the query tiles; spare;
                          // [8..15] the bf16 forward's work queues
    size_t v16 = 0;       // bf16 path, fp32 values only: v rounded to bf16 (bf16 [BHkv][n][dv])
    size_t total = 0;
};

// Hkv k/v heads (each shared by H/Hkv query heads) and dv value channels;
// 0 means Hkv = H and dv = d.  v_f32: the values come as fp32 (on the bf16
// path they are rounded to bf16 once, into the v16 region).
inline Layout make_layout(int64_t B, int64_t H, int64_t n, int64_t d, bool bf16_path,
                          int64_t Hkv = 0, int64_t dv = 0, bool v_f32 = false) {
    Layout L;
    L.BH = B * H;
    L.n = n;
    L.d = d;
    L.H = H;
    L.Hkv = Hkv > 0 ? Hkv : H;
    L.BHkv = B * L.Hkv;
    L.dv = dv > 0 ? dv : d;
    L.bf16_path = bf16_path;
    L.n_pad = (n + BQ - 1) / BQ * BQ;
    L.n_qt = L.n_pad / BQ;
    L.n_kt = L.n_pad / BK;
    size_t off = 0;
    const size_t per_pos = sizeof(float) * size_t(L.BH) * size_t(L.n_pad);
    for (int i = 0; i < 9; ++i) {
        L.gate[i] = off;
        off = align_up(off + per_pos, 256);
    }
    const size_t per_kt = sizeof(double) * size_t(L.BH) * size_t(L.n_kt);
    for (int i = 0; i < 3; ++i) {
        L.tile[i] = off;
        off = align_up(off + per_kt, 256);
    }
    L.tile4 = off;
    off = align_up(off + 4 * per_kt, 256);
    const size_t per_qt = sizeof(uint32_t) * size_t(L.BH) * size_t(L.n_qt);
    L.qstat = off;
    off = align_up(off + sizeof(uint32_t) * size_t(L.BH), 256);
    L.kstat = off;
    off = align_up(off + sizeof(uint32_t) * size_t(L.BH), 256);
    L.noff = off;
    off = align_up(off + per_qt, 256);
    L.gbad = off;
    off = align_up(off + per_qt, 256);
    L.counters = off;
    off = align_up(off + 16 * sizeof(uint32_t), 256);
    L.v16 = off;
    if (bf16_path && v_f32) off = align_up(off + 2 * size_t(L.BHkv) * size_t(L.n) * size_t(L.dv), 256);
    L.total = off;
    return L;
}

// Workspace of the chain-corner scan (resolvent_chain): the gate planes and
// tile products of make_layout, then per (head, 64-position tile, channel)
// the tile's own scan end with a zero carry-in (agg) and the carry into the
// tile (carry), both complex float (float2) [BH][n_kt][dv].
struct ChainLayout {
    Layout g;
    int64_t dv = 0;
    size_t agg = 0, carry = 0, total = 0;
};

inline ChainLayout make_chain_layout(int64_t B, int64_t H, int64_t n, int64_t dv) {
    ChainLayout C;
    C.g = make_layout(B, H, n, dv, false, 0, 0);
    C.dv = dv;
    const size_t per = 8 * size_t(C.g.BH) * size_t(C.g.n_kt) * size_t(dv);
    size_t off = C.g.total;
    C.agg = off;
    off = align_up(off + per, 256);
    C.carry = off;
    off = align_up(off + per, 256);
    C.total = off;
    return C;
}

// Workspace of a decode step (resolvent_decode).  Positions are grouped in
// chunks of DEC_CT key tiles (DEC_CT BK = 256 positions): per chunk its gate
// product P, f64 (double [3][BH][n_ch]: re, im, modulus), the merge's scale of
// the chunk, C 2^(M_c - M) with C the gates from the chunk's end to the newest
// position (float4 [BH][n_ch]: re, im, modulus, 0), and one partial
// (M, z, refused, 0, O_re[dv], O_im[dv]) relative to the chunk's end (float
// [BH][n_ch][4 + 2 dv]; the header is padded so that O starts on 16 bytes).
constexpr int DEC_CT = 4;
constexpr int64_t DEC_CHUNK = DEC_CT * BK;
constexpr int64_t dec_part_floats(int64_t dv) { return 4 + 2 * dv; }
struct DecodeLayout {
    int64_t BH = 0, H = 0, Hkv = 0, n = 0, d = 0, dv = 0, n_ch = 0;
    size_t prod = 0, scale = 0, part = 0, total = 0;
};

inline DecodeLayout make_decode_layout(int64_t B, int64_t H, int64_t Hkv, int64_t n, int64_t d,
                                       int64_t dv) {
    DecodeLayout D;
    D.BH = B * H;
    D.H = H;
    D.Hkv = Hkv;
    D.n = n;
    D.d = d;
    D.dv = dv;
    D.n_ch = (n + DEC_CHUNK - 1) / DEC_CHUNK;
    const size_t per = 3 * sizeof(double) * size_t(D.BH) * size_t(D.n_ch);
    size_t off = 0;
    D.prod = off;
    off = align_up(off + per, 256);
    D.scale = off;
    off = align_up(off + 16 * size_t(D.BH) * size_t(D.n_ch), 256);
    D.part = off;
    off = align_up(off + 4 * size_t(D.BH) * size_t(D.n_ch) * size_t(dec_part_floats(dv)), 256);
    D.total = off;
    return D;
}

// Workspace of the operator export (resolvent_operator), f64 planes
// (double [BH][n] each: re, im, modulus): the gate of every position, and
// the product of the gates after it up to the end of its 64-position tile
// plus one (a_{p+1} ... a_{t0+64}; gates past n count as 1).
struct OperatorLayout {
    int64_t BH = 0, n = 0, d = 0;
    size_t a_re = 0, a_im = 0, a_m = 0;  // the gates a_p
    size_t s_re = 0, s_im = 0, s_m = 0;  // a_{p+1} ... a_{t0+64} inside p's tile of 64
    size_t total = 0;
};

inline OperatorLayout make_operator_layout(int64_t B, int64_t H, int64_t n, int64_t d) {
    OperatorLayout O;
    O.BH = B * H;
    O.n = n;
    O.d = d;
    const size_t per = sizeof(double) * size_t(O.BH) * size_t(n);
    const size_t plane = align_up(per, 256);
    O.a_re = 0;
    O.a_im = plane;
    O.a_m = 2 * plane;
    O.s_re = 3 * plane;
    O.s_im = 4 * plane;
    O.s_m = 5 * plane;
    O.total = 6 * plane;
    return O;
}

// Source byte offsets of the direct global->LDS tile copies, relative to the
// start of the tensor (q, k or v).  Row `r`
// of key tile `t` is key t*BK + r, clamped into [0, n-1] so that a tile
// reaching past the sequence end still reads inside the tensor; `chunk` is a
// 16-byte chunk of that row.
RESOLVENT_HD inline int64_t tile_row_src(int64_t bh, int64_t n, int64_t t, int r,
                                         int64_t row_bytes, int chunk) {
    int64_t key = t * BK + r;
    key = key < n ? key : n - 1;
    return (bh * n + key) * row_bytes + int64_t(chunk) * 16;
}

// The same as 32-bit offsets inside one head (the kernels add them to a
// wave-uniform head base; every offset fits 32 bits for n <= 2^22, d <= 128).
RESOLVENT_HD inline uint32_t tile_row_off(int64_t n, int64_t t, int r, int64_t row_bytes) {
    int64_t key = t * BK + r;
    key = key < n ? key : n - 1;
    return uint32_t(key * row_bytes);
}

// Work queues of the bf16 forward: queue x (of nq, nq dividing BH) holds the
// query tiles of heads x, x + nq, x + 2 nq, ..., hx = BH / nq heads with n_qt
// query tiles each.  Entry k of the queue is the query tile bh * n_qt + qt
// (-1 past the queue's end).  order 0 takes the heaviest query tile (the
// last) of every head of the queue first, then the next ones; order 1 takes
// one head at a time, heaviest query tile first; order 2 takes the query
// tiles qt >= q0 of one head at a time, heaviest first, and then the light
// ones (qt < q0) of every head, heaviest first across the heads.
RESOLVENT_HD inline int64_t queue_item(int x, uint32_t k, int nq, int64_t BH, int64_t n_qt,
                                       int order, int64_t q0 = 0) {
    const int64_t hx = BH / nq;
    if (int64_t(k) >= hx * n_qt) return -1;
    int64_t hj, qt;
    if (order == 0) {
        hj = int64_t(k) % hx;
        qt = n_qt - 1 - int64_t(k) / hx;
    } else if (order == 1 || q0 <= 0 || q0 >= n_qt) {
        hj = int64_t(k) / n_qt;
        qt = n_qt - 1 - int64_t(k) % n_qt;
    } else {
        const int64_t heavy = n_qt - q0;  // per head
        if (int64_t(k) < hx * heavy) {
            hj = int64_t(k) / heavy;
            qt = n_qt - 1 - int64_t(k) % heavy;
        } else {
            const int64_t kk = int64_t(k) - hx * heavy;
            hj = kk % hx;
            qt = q0 - 1 - kk / hx;
        }
    }
    return (x + nq * hj) * n_qt + qt;
}

// Padded bf16 tiles of the fused forward (bf16 path).  A K row of d bf16
// values takes KSL = d/8 + 1 sixteen-byte slots in LDS; with a row stride of
// an odd number of slots, the 16 rows that a half-wave reads at one chunk fall
// into 16 different bank groups.  The values of a tile are staged as they lie
// in v, a row of dv bf16 values per key, each row taking VSL = dv/8 + 2 slots
// (the last two are padding): the matrix product reads them with the
// transposing 8-byte LDS read, which hands each lane four consecutive keys of
// one channel.  Every operand read is a per-lane base plus an immediate
// offset.  The K tile occupies slots [0, 64 KSL) of a buffer and the value
// tile the next 64 VSL; copy instruction j of a tile (a direct global->LDS
// copy of 16 bytes per lane) fills slots [64 j, 64 j + 64): lane L slot
// 64 j + L.  A padding slot holds a copy of its row's last chunk.
template <int D>
RESOLVENT_HD constexpr int pad_kslots() { return D / 8 + 1; }
template <int DV>
RESOLVENT_HD constexpr int pad_vslots() { return DV / 8 + 2; }
template <int D>
RESOLVENT_HD constexpr int pad_kcopies() { return pad_kslots<D>(); }  // BK rows x KSL slots / 64
template <int DV>
RESOLVENT_HD constexpr int pad_vcopies() { return pad_vslots<DV>(); }  // BK rows x VSL slots / 64
// The NC = KSL + VSL copy instructions of a tile are shared by waves
// 1..NWAVES-1 (wave 0 copies the gate data): copying wave w issues, as its
// i-th of pad_copies_per_wave, instruction j = w - 1 + (NWAVES - 1) i, the
// last one repeated past NC (the same bytes to the same slots).
template <int D, int DV>
RESOLVENT_HD constexpr int pad_copies() { return pad_kcopies<D>() + pad_vcopies<DV>(); }
template <int D, int DV>
RESOLVENT_HD constexpr int pad_copies_per_wave() {
    return (pad_copies<D, DV>() + NWAVES - 2) / (NWAVES - 1);
}
template <int D, int DV>
RESOLVENT_HD inline int pad_copy_j(int w, int i) {
    const int j = w - 1 + (NWAVES - 1) * i;
    return j < pad_copies<D, DV>() ? j : pad_copies<D, DV>() - 1;
}
// The key whose values row q of a value tile holds: inside each group of 8
// rows, rows 2e and 2e + 1 hold keys e and 4 + e.  A half-wave's transposing
// read then takes four rows two apart (4 x 64 bytes at a stride of two rows),
// which fall into distinct bank groups for the row stride of dv/8 + 2 slots.
RESOLVENT_HD constexpr int pad_vrow_key(int q) { return (q & ~7) | ((q & 1) << 2) | ((q & 7) >> 1); }
// Source byte offset of copy instruction j, lane `lane`, relative to the
// tile's first key row: for j < KSL inside the K rows of the tile (rows of 2d
// bytes), otherwise inside its value rows (2 dv bytes; value row r of the
// tile takes key pad_vrow_key(r)).  (The whole tile inside the sequence; see
// the ragged forms below.)
template <int D, int DV>
RESOLVENT_HD inline uint32_t pad_copy_src(int j, int lane) {
    constexpr int KSL = pad_kslots<D>(), VSL = pad_vslots<DV>();
    if (j < KSL) {
        const int p = 64 * j + lane, r = p / KSL;
        const int c = p % KSL < KSL - 1 ? p % KSL : KSL - 2;
        return uint32_t(r * D * 2 + 16 * c);
    }
    const int p = 64 * (j - KSL) + lane, r = p / VSL;
    const int c = p % VSL < DV / 8 ? p % VSL : DV / 8 - 1;
    return uint32_t(pad_vrow_key(r) * DV * 2 + 16 * c);
}
// The K copy source of tile t when the tile reaches past key n - 1 (or lies
// wholly past it, as own tiles of the last query tile can): rows past it
// repeat key n - 1 (their entries are masked).  Relative to the head's first
// key row (32 bits for n <= 2^22).
template <int D>
RESOLVENT_HD inline uint32_t pad_kcopy_src_ragged(int j, int lane, int64_t n, int64_t t) {
    constexpr int KSL = pad_kslots<D>();
    const int p = 64 * j + lane, r = p / KSL;
    const int c = p % KSL < KSL - 1 ? p % KSL : KSL - 2;
    const int64_t key = t * BK + r < n ? t * BK + r : n - 1;
    return uint32_t(key * D * 2 + 16 * c);
}
// The same for the value copies (copy jv = j - KSL of the value tile):
// relative to the head's first value row.
template <int DV>
RESOLVENT_HD inline uint32_t pad_vcopy_src_ragged(int jv, int lane, int64_t n, int64_t t) {
    constexpr int VSL = pad_vslots<DV>();
    const int p = 64 * jv + lane, r = pad_vrow_key(p / VSL);
    const int c = p % VSL < DV / 8 ? p % VSL : DV / 8 - 1;
    const int64_t key = t * BK + r < n ? t * BK + r : n - 1;
    return uint32_t(key * DV * 2 + 16 * c);
}
// Byte offsets, inside a buffer, of the operand reads of a 32x32x16 bf16
// product.  K: lane (qi, h) reads row kb + qi, chunk 2s + h (step s).
// Values: the A operand of O^T += V^T W~^T for channels 32 db .. 32 db + 31 and
// the 16 keys kb + 16 kc .. of chunk kc is two transposing 8-byte reads
// (s = 0, 1).  In the read, each group of 16 lanes addresses a 4 x 4 grid of
// 8-byte pieces (four keys by four groups of four channels) and lane i
// receives channel (i & 3) of the pieces of lanes (i >> 2) + 4 e, e = 0..3;
// the addresses below hand lane l four keys kb + 16 kc + 8 s + 4 (l >> 5) + e
// of channel 32 db + (l & 31), the keys of the W~ operand's k order (the
// lane's eight logits are the keys 8 (e >> 2) + 4 h + (e & 3) of the chunk),
// from the value rows that hold them (pad_vrow_key: rows kb + 16 kc + 8 s +
// (l >> 5) + 2 e).
template <int D>
RESOLVENT_HD constexpr int pad_kread(int kb, int s, int qi, int h) {
    return (kb + qi) * 16 * pad_kslots<D>() + 16 * (2 * s + h);
}
template <int D, int DV>
RESOLVENT_HD constexpr int pad_vread_tr(int kb, int kc, int db, int s, int lane) {
    return 16 * BK * pad_kslots<D>() +
           (kb + 16 * kc + 8 * s + (lane >> 5) + 2 * ((lane & 15) >> 2)) * 16 * pad_vslots<DV>() +
           2 * (32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}

// Float index, inside a gate plane [BH][n_pad], of the datum lane `lane`
// copies for key tile t: S_j of key t*BK + lane (a tile before the query
// tile), or a_{j+1} (own) -- one past the head's last position this is the
// first entry of the next row, or of the next plane for the last head, still
// inside the workspace and only ever multiplied into an entry above the
// diagonal.
RESOLVENT_HD inline int64_t gate_src(int64_t bh, int64_t n_pad, int64_t t, int lane, bool own) {
    return bh * n_pad + t * BK + lane + (own ? 1 : 0);
}

// Everything a launch needs, in device pointers.
struct Problem {
    const void *q, *k, *v;
    const float *u, *theta;
    float *o_re, *o_im;
    int32_t *status;
    unsigned char *ws;
    Layout L;
    double g;
    float c;            // qk * log2(e) / sqrt(d), the logit scale in log2 units
    float beta;
    int beta_mode;      // 0: beta == 0, 1: beta == 1, 2: general
    bool qk_zero;
    bool v_f32;         // v stored as float32 (bf16 path converts when staging)
};

// Status := OK, then the gates and their in-tile scans of make_layout into
// the workspace (resolvent_kernels.hip).  u, theta hold ldu positions per head
// (0: L.n).  Returns a hipError_t.
int launch_gates(const Layout &L, const float *u, const float *theta, double g,
                 unsigned char *ws, int32_t *status, void *stream, int64_t ldu = 0);

// The chain-corner scan (chain_kernels.hip): the gates, then the three scan
// kernels.  v is [BH][n][dv] bf16 (v_f32 false) or float32.  Returns a
// hipError_t.
int launch_chain(const ChainLayout &C, const float *u, const float *theta, const void *v,
                 bool v_f32, double g, float *o_re, float *o_im, unsigned char *ws,
                 int32_t *status, void *stream);

// One decode step (decode_kernels.hip): the chunk partials (with their
// gates) and their merge.  c is the logit scale qk log2(e)/sqrt(d).
// Returns a hipError_t.
int launch_decode(const DecodeLayout &DL, const void *q, const void *k, const float *u,
                  const float *theta, const void *v, int64_t cap, bool qk_f32, bool v_f32,
                  double g, float c, float beta, int beta_mode, bool qk_zero, float *o_re,
                  float *o_im, unsigned char *ws, int32_t *status, void *stream);
// The path-product matrices of `batch` gate sequences of length n, f64
// (export_kernels.hip).  Returns a hipError_t.
int launch_path_product(const double *a_re, const double *a_im, int64_t batch, int64_t n,
                        double *g_re, double *g_im, void *stream);
// The operator W of every head, float32 (export_kernels.hip).  Returns a
// hipError_t.
int launch_operator(const OperatorLayout &OL, const void *q, const void *k, const float *u,
                    const float *theta, bool qk_f32, double g, float c, float beta,
                    int beta_mode, bool qk_zero, float *w_re, float *w_im, unsigned char *ws,
                    int32_t *status, void *stream);
// One step of the gated chain per (head, channel), in place (decode_kernels.hip).
int launch_chain_step(float *y_re, float *y_im, const float *u, const float *theta,
                      const void *v, bool v_f32, double g, int64_t BH, int64_t dv,
                      int32_t *status, void *stream);

// Kernel launcher (resolvent_kernels.hip).  marks, when not null, are four
// HIP events recorded on the stream before the first kernel, before the fused
// forward kernel, after it, and after the last kernel.  Returns a hipError_t.
int launch_forward(const Problem &P, void *stream, void *const *marks);

}  // namespace resolvent
