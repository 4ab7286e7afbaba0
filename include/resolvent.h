/*
 * resolvent.h -- C ABI of the MI355X (gfx950) forward pass of the resolvent
 * operator head.
 *
 * The operation is the one the "Resolvent Operator" page (teerth.dev,
 * Aether-Lang/integrated/resolvent) defines in its section "Object".  For one
 * causal head of length n, with queries and keys q_i, k_j in R^d, raw gate
 * magnitudes u_k, phases theta_k, real values V_j and switches (beta, qk, g):
 *
 *   s_ij  = <q_i, k_j> / sqrt(d)                      scaled logit
 *   m_k   = clamp(lerp(1, u_k, g), 0, 1), theta'_k = g theta_k
 *   a_k   = m_k e^{i theta'_k}                        the gate
 *   G_ij  = prod_{k=j+1..i} a_k, G_ii = 1             the path product
 *   R_ij  = prod_{k=j+1..i} m_k = |G_ij|
 *   Z_i   = sum_{j<=i} R_ij e^{qk s_ij}               the row normaliser
 *   W_ij  = G_ij e^{qk s_ij} / Z_i^beta  (j <= i),  0 (j > i)
 *   O_i   = sum_{j<=i} W_ij V_j                       complex readout
 *
 * Z_i^beta is evaluated in the log domain with a shift by the largest live
 * logit (live: R_ij > 0), as in the page's section "Evaluation and refusals".
 * The corners are softmax attention (1,1,0), the unnormalised exponential
 * kernel (0,1,0) and the gated-chain path product (0,0,1) (section "The three
 * corners").  G is formed only as a product of gates -- never through a
 * logarithm or a division -- so a closed gate (m_k = 0) gives exact zeros
 * (Lean table, no_prefix_scan_represents_a_zero_gate and pathProd_eq_zero_iff).
 *
 * Everything runs on the device, asynchronously, on the caller's stream.  The
 * library allocates nothing, keeps no state between calls and is thread-safe;
 * the caller owns every buffer.
 */
#ifndef RESOLVENT_H
#define RESOLVENT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes: the return value of every call and the device status word. */
enum resolvent_status {
    RESOLVENT_OK = 0,
    RESOLVENT_NONFINITE = 1,   /* refused input ("Evaluation and refusals")  */
    RESOLVENT_BAD_SHAPE = 2,   /* negative size, or head_dim 0 with n > 0     */
    RESOLVENT_BAD_ARG = 3,     /* null/misaligned pointer, small workspace    */
    RESOLVENT_UNSUPPORTED = 4, /* head_dim or dtype pair this build lacks     */
    RESOLVENT_DEVICE_ERROR = 5, /* a HIP launch failed                        */
    RESOLVENT_TOO_LARGE = 6     /* beyond resolvent_forward_noalloc's scratch  */
};

/* Storage types of q, k and v. */
enum resolvent_dtype { RESOLVENT_BF16 = 0, RESOLVENT_F32 = 1 };

/*
 * resolvent_workspace_bytes -- device workspace that resolvent_forward needs
 * for this shape and these storage types (0 for an empty problem, and also 0
 * for an invalid or unsupported one, which resolvent_forward rejects).
 * The workspace holds the gates, their in-tile scans, the tile products, the
 * per-tile extrema of q and k and, only when fp32 values meet bf16 q and k, a
 * bf16 copy of v; it grows linearly with n.  Its contents are scratch between calls.
 */
size_t resolvent_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d,
                                 int32_t qk_dtype, int32_t v_dtype);

/*
 * resolvent_forward -- O = readout of the resolvent head for B*H independent
 * heads (section "Object" of the page; the Rust API's operator + readout with
 * value_dim = head_dim).
 *
 * Arguments (all device pointers; 16-byte aligned; contiguous row-major):
 *   q, k        [B, H, n, d] in qk_dtype (RESOLVENT_BF16 or RESOLVENT_F32)
 *   u, theta    [B, H, n] float32: raw gate magnitudes and phases; u_0 and
 *               theta_0 are checked although a_0 is never read
 *   v           [B, H, n, d] in v_dtype
 *   beta,qk,g   the switches, as the page's Switches (f64)
 *   d           head_dim; this build supports d = 64 and d = 128
 *   o_re, o_im  [B, H, n, d] float32 outputs (real and imaginary planes)
 *   workspace   at least resolvent_workspace_bytes(...) bytes of device memory
 *   status_dev  one int32 of device memory: the call sets it to RESOLVENT_OK
 *               and the kernels set it to RESOLVENT_NONFINITE when they refuse
 *               an input; read it after synchronising the stream
 *   stream      HIP stream to enqueue on (NULL: the null stream)
 *
 * Dtype pairs: (BF16, BF16) and (BF16, F32) run the bf16 MFMA path (an fp32 v
 * is rounded to bf16 when it is staged); (F32, F32) runs the fp32 MFMA path.
 *
 * Returns, before anything is enqueued:
 *   RESOLVENT_BAD_SHAPE   a negative size; d == 0 with n, B, H > 0
 *   RESOLVENT_OK          n == 0, B == 0 or H == 0 ("empty in, empty out"):
 *                         nothing is enqueued and nothing is written
 *   RESOLVENT_NONFINITE   a non-finite switch, or qk*log2(e)/sqrt(d) not
 *                         representable in float32
 *   RESOLVENT_UNSUPPORTED another d or dtype pair
 *   RESOLVENT_BAD_ARG     a null or misaligned pointer, a small workspace
 *   RESOLVENT_DEVICE_ERROR a launch failed (status_dev is then unspecified)
 * and RESOLVENT_OK once the work is enqueued.  On the device the status word
 * becomes RESOLVENT_NONFINITE for a non-finite q, k, u or theta, an
 * overflowing g*theta_k (evaluated in f64) or a logit qk*s_ij (j <= i) whose
 * float32 value overflows; the outputs are then unspecified.  A non-finite v
 * is not refused (the page refuses operator inputs only) and leaves the
 * outputs unspecified.  Outside beta = 1, a readout whose true value exceeds
 * the float32 range is unspecified.
 */
int32_t resolvent_forward(const void *q, const void *k, const float *u, const float *theta,
                          const void *v, double beta, double qk, double g, int64_t B,
                          int64_t H, int64_t n, int64_t d, int32_t qk_dtype, int32_t v_dtype,
                          float *o_re, float *o_im, void *workspace, size_t workspace_bytes,
                          int32_t *status_dev, hipStream_t stream);

/*
 * resolvent_forward_marked -- resolvent_forward, plus measurement marks: when
 * marks is not NULL it points to four HIP events (created by the caller, with
 * timing enabled) that are recorded on the stream before the first kernel,
 * right before and right after the fused forward kernel, and after the last
 * kernel, so hipEventElapsedTime brackets each stage.  Same arguments,
 * checks and return codes as resolvent_forward otherwise.
 */
int32_t resolvent_forward_marked(const void *q, const void *k, const float *u,
                                 const float *theta, const void *v, double beta, double qk,
                                 double g, int64_t B, int64_t H, int64_t n, int64_t d,
                                 int32_t qk_dtype, int32_t v_dtype, float *o_re, float *o_im,
                                 void *workspace, size_t workspace_bytes, int32_t *status_dev,
                                 hipStream_t stream, hipEvent_t *marks);

/*
 * resolvent_forward_noalloc -- resolvent_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument; the workspace is a
 * fixed array of RESOLVENT_NOALLOC_SCRATCH_BYTES bytes inside the library,
 * one per device, held from the library's first use on that device until the
 * process ends.  The call allocates nothing; the caller still owns q, k, u,
 * theta, v, o_re, o_im and status_dev, with the meanings, layouts and checks
 * of resolvent_forward.
 *
 * Returns RESOLVENT_TOO_LARGE, before anything is enqueued, when
 * resolvent_workspace_bytes(B, H, n, d, qk_dtype, v_dtype) exceeds
 * RESOLVENT_NOALLOC_SCRATCH_BYTES (64 MiB: for example B*H = 16 heads of
 * n = 8192 at d = 128 in bf16 need 36.6 MiB); RESOLVENT_DEVICE_ERROR when the
 * array's device address cannot be obtained; otherwise what resolvent_forward
 * returns.  The stream must belong to the current device.  Every call on a
 * device uses that device's one array, so calls that overlap in time on one
 * device (two streams, two threads) race and give unspecified outputs; calls
 * ordered on one stream are safe.  Each call clears on the device whatever
 * of the array must start at zero, so what an earlier call left there does
 * not matter.
 */
#define RESOLVENT_NOALLOC_SCRATCH_BYTES (64u << 20)

size_t resolvent_noalloc_scratch_bytes(void);

int32_t resolvent_forward_noalloc(const void *q, const void *k, const float *u,
                                  const float *theta, const void *v, double beta, double qk,
                                  double g, int64_t B, int64_t H, int64_t n, int64_t d,
                                  int32_t qk_dtype, int32_t v_dtype, float *o_re, float *o_im,
                                  int32_t *status_dev, hipStream_t stream);

/*
 * resolvent_workspace_bytes_grouped -- device workspace for
 * resolvent_forward_grouped (0 for an empty, invalid or unsupported
 * problem, which resolvent_forward_grouped rejects).
 */
size_t resolvent_workspace_bytes_grouped(int64_t B, int64_t H, int64_t Hkv, int64_t n,
                                         int64_t d, int64_t dv, int32_t qk_dtype,
                                         int32_t v_dtype);

/*
 * resolvent_forward_grouped -- resolvent_forward with the page's value_dim
 * free (section "Rust API": the readout takes V as [seq, value_dim]) and with
 * keys and values shared by groups of heads: H query heads read Hkv k/v heads,
 * query head h of batch entry b using k/v head h / (H / Hkv) of that entry.
 * Each query head keeps its own gates (u, theta) and its own operator; only k
 * and v are shared.  resolvent_forward(..., H, n, d, ...) is
 * resolvent_forward_grouped(..., H, H, n, d, d, ...).
 *
 * Arguments as for resolvent_forward, except:
 *   q           [B, H, n, d]
 *   k           [B, Hkv, n, d]
 *   v           [B, Hkv, n, dv]
 *   u, theta    [B, H, n]
 *   Hkv         k/v heads: 1 <= Hkv, H a multiple of Hkv
 *   dv          value channels: 64 or 128 (d is 64 or 128 as well)
 *   o_re, o_im  [B, H, n, dv]
 *   workspace   at least resolvent_workspace_bytes_grouped(...) bytes
 *
 * Returns as resolvent_forward, with RESOLVENT_BAD_SHAPE also for Hkv <= 0
 * or H not a multiple of Hkv (when n, B, H > 0), and RESOLVENT_UNSUPPORTED
 * for another dv.
 */
int32_t resolvent_forward_grouped(const void *q, const void *k, const float *u,
                                  const float *theta, const void *v, double beta, double qk,
                                  double g, int64_t B, int64_t H, int64_t Hkv, int64_t n,
                                  int64_t d, int64_t dv, int32_t qk_dtype, int32_t v_dtype,
                                  float *o_re, float *o_im, void *workspace,
                                  size_t workspace_bytes, int32_t *status_dev,
                                  hipStream_t stream);

/*
 * resolvent_counters_offset -- byte offset inside the workspace of two uint32
 * counters that a call leaves behind: [0] the number of (query tile, key tile)
 * pairs before the diagonal that the fused kernel evaluated (it stops early
 * once every earlier path product is exactly 0 in float32), [1] reserved.
 * SIZE_MAX when resolvent_workspace_bytes would return 0.
 */
size_t resolvent_counters_offset(int64_t B, int64_t H, int64_t n, int64_t d, int32_t qk_dtype,
                                 int32_t v_dtype);

/*
 * resolvent_tile_shape -- the tiling the counters above refer to: *bq query
 * rows per query tile, *bk keys per key tile.  A counted (query tile, key
 * tile) pair stands for bq * bk (query, key) entries.  Either pointer may be
 * NULL.
 */
void resolvent_tile_shape(int32_t *bq, int32_t *bk);

/*
 * resolvent_chain_workspace_bytes -- device workspace that resolvent_chain
 * needs (0 for an empty problem, and also 0 for an invalid or unsupported
 * one, which resolvent_chain rejects).  It holds the gates, their in-tile
 * scans and tile products, and two complex floats per (head, 64-position
 * tile, value channel).  Its contents are scratch between calls.
 */
size_t resolvent_chain_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t dv);

/*
 * resolvent_chain -- the path-product corner of the head (the page's section
 * "The path-product corner is a resolvent"): O_i = sum_{j<=i} G_ij V_j, the
 * readout at switches (beta, qk, g) = (0, 0, g), computed as the gated chain
 * y_i = a_i y_{i-1} + V_i, y_0 = V_0, per value channel (O(n dv) work; q and k
 * play no part at qk = 0).  For a given g its result equals resolvent_forward
 * at (0, 0, g) up to rounding.
 *
 * Arguments (device pointers; contiguous row-major):
 *   u, theta    [B, H, n] float32 raw gate magnitudes and phases, 4-byte
 *               aligned; every entry is checked although a_0 is never read
 *   v           [B, H, n, dv] in v_dtype (RESOLVENT_BF16 or RESOLVENT_F32),
 *               aligned to its element size
 *   g           the gate switch (f64)
 *   dv          value channels: a multiple of 64, at most 4096
 *   o_re, o_im  [B, H, n, dv] float32 outputs, 4-byte aligned
 *   workspace   at least resolvent_chain_workspace_bytes(...) bytes, 256-byte
 *               aligned
 *   status_dev  one int32 of device memory, as for resolvent_forward
 *   stream      HIP stream to enqueue on (NULL: the null stream)
 *
 * Returns, before anything is enqueued: RESOLVENT_BAD_SHAPE for a negative
 * size or dv == 0 with n, B, H > 0; RESOLVENT_OK with nothing enqueued when
 * n, B or H is 0; RESOLVENT_NONFINITE for a non-finite g; RESOLVENT_UNSUPPORTED
 * for a dv that is not a multiple of 64 or exceeds 4096, another dtype, or a
 * size past the limits of resolvent_forward; RESOLVENT_BAD_ARG for a null or
 * misaligned pointer or a small workspace; RESOLVENT_DEVICE_ERROR when a
 * launch fails; RESOLVENT_OK once the work is enqueued.  On the device the
 * status word becomes RESOLVENT_NONFINITE for a non-finite u or theta or an
 * overflowing g*theta_k; the outputs are then unspecified.  A non-finite v is
 * not refused and leaves the outputs unspecified.
 */
int32_t resolvent_chain(const float *u, const float *theta, const void *v, double g, int64_t B,
                        int64_t H, int64_t n, int64_t dv, int32_t v_dtype, float *o_re,
                        float *o_im, void *workspace, size_t workspace_bytes,
                        int32_t *status_dev, hipStream_t stream);

/*
 * resolvent_decode_workspace_bytes -- device workspace for resolvent_decode
 * (0 for an empty, invalid or unsupported problem).
 */
size_t resolvent_decode_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t n, int64_t d,
                                        int64_t dv, int32_t qk_dtype, int32_t v_dtype);

/*
 * resolvent_decode -- one decode step: the readout of the newest position
 * i = n-1 of every query head (section "Object" of the "Resolvent Operator"
 * page, its last row; the decode shape of decodeGQA on the Op Specs page:
 * query head h of a batch entry reads k/v head h / (H / Hkv)), for a new
 * query against the cached keys and values of positions 0..n-1, the new
 * position's key and value included.  O(n (d + dv)) per head: the gates and
 * their products are formed from u, theta afresh, the keys are split over
 * workgroups of 4 key tiles whose partial sums are merged with the same
 * max shift as the forward pass.  Equal, up to rounding, to row n-1 of
 * resolvent_forward_grouped on the same inputs; the weights stay float32
 * (they are not rounded to bf16 as in the forward's bf16 path).
 *
 * Arguments (device pointers; row-major, each head's positions cap apart, so
 * that a cache allocated for cap positions and filled to n is passed as is):
 *   q           [B, H, d] the newest position's query (qk_dtype)
 *   k           [B, Hkv, cap, d] keys; positions 0..n-1 are read (qk_dtype)
 *   u, theta    [B, H, cap] float32 gate inputs, per query head; positions
 *               0..n-1 are read
 *   v           [B, Hkv, cap, dv] values (v_dtype); positions 0..n-1 are read
 *   beta,qk,g   the switches (f64)
 *   Hkv         k/v heads, dividing H
 *   n, cap      positions in the cache (the newest is n-1) and allocated
 *               positions per head, cap >= n
 *   d, dv       64 or 128 each
 *   o_re, o_im  [B, H, dv] float32 outputs
 *   workspace   at least resolvent_decode_workspace_bytes(...) bytes,
 *               256-byte aligned
 *   status_dev, stream  as for resolvent_forward
 * q, k and v are 16-byte aligned; u, theta, o_re, o_im and status_dev 4-byte.
 *
 * Returns, before anything is enqueued, the codes of resolvent_forward_grouped
 * for the same conditions, RESOLVENT_BAD_SHAPE also for cap < n, (RESOLVENT_OK
 * with nothing enqueued when n, B or H is 0).  On the device the status word becomes RESOLVENT_NONFINITE for a
 * non-finite q, k (any position), u or theta, an overflowing g*theta_k or a
 * float32 logit qk*s_ij (j <= n-1) that overflows; the outputs are then
 * unspecified.
 */
int32_t resolvent_decode(const void *q, const void *k, const float *u, const float *theta,
                         const void *v, double beta, double qk, double g, int64_t B, int64_t H,
                         int64_t Hkv, int64_t n, int64_t cap, int64_t d, int64_t dv,
                         int32_t qk_dtype, int32_t v_dtype, float *o_re, float *o_im,
                         void *workspace, size_t workspace_bytes, int32_t *status_dev,
                         hipStream_t stream);

/*
 * resolvent_chain_step -- one decode step of the chain corner (switches
 * (0, 0, g); section "The path-product corner is a resolvent"): the state
 * y = O_{i-1} [B, H, dv] (complex, planar float32, in place) becomes
 * O_i = a_i y + V_i, with a_i = gate(blend(u_i, theta_i, g)) from u, theta
 * [B, H] float32 and V_i [B, H, dv] (v_dtype).  O(1) per head and channel;
 * starting from y = 0 it reproduces resolvent_chain position by position.
 * Returns RESOLVENT_BAD_SHAPE for a negative size, RESOLVENT_OK with nothing
 * enqueued when B, H or dv is 0, RESOLVENT_NONFINITE for a non-finite g,
 * RESOLVENT_UNSUPPORTED for another dtype, dv > 4096 or B H > 2^24,
 * RESOLVENT_BAD_ARG for a null or misaligned pointer; on the device the status
 * word becomes RESOLVENT_NONFINITE for a non-finite u, theta or g*theta (the
 * state of that head is then left as it was).  The caller sets status_dev to
 * RESOLVENT_OK beforehand: this call never clears it.
 */
int32_t resolvent_chain_step(float *y_re, float *y_im, const float *u, const float *theta,
                             const void *v, double g, int64_t B, int64_t H, int64_t dv,
                             int32_t v_dtype, int32_t *status_dev, hipStream_t stream);

/*
 * resolvent_operator_workspace_bytes -- device workspace for
 * resolvent_operator (0 for an empty, invalid or unsupported problem).
 */
size_t resolvent_operator_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d,
                                          int32_t qk_dtype);

/*
 * resolvent_operator -- the operator W of every head, materialised: the
 * "operator" of the "Resolvent Operator" page's Rust API (section "Object":
 * W_ij = G_ij e^{qk s_ij} / Z_i^beta for j <= i, 0 above the diagonal),
 * row-major [n, n] per head, for inspection at small n (the hot path never
 * forms W).  float32 weights from float32 logits and f64 gate products, the
 * arithmetic of the decode step applied to every row.
 *
 * Arguments (device pointers; contiguous row-major):
 *   q, k        [B, H, n, d] (qk_dtype: RESOLVENT_BF16 or RESOLVENT_F32),
 *               16-byte aligned
 *   u, theta    [B, H, n] float32
 *   beta,qk,g   the switches (f64)
 *   d           64 or 128; n <= 65536 and B H n < 2^31
 *   w_re, w_im  [B, H, n, n] float32 outputs
 *   workspace   at least resolvent_operator_workspace_bytes(...) bytes,
 *               256-byte aligned
 *   status_dev, stream  as for resolvent_forward
 * Returns the codes of resolvent_forward for the same conditions before
 * anything is enqueued (RESOLVENT_OK with nothing enqueued when n, B or H is
 * 0); on the device the status word becomes RESOLVENT_NONFINITE for a
 * non-finite q, k, u or theta, an overflowing g*theta_k or a float32 logit
 * that overflows (the outputs are then unspecified).
 */
int32_t resolvent_operator(const void *q, const void *k, const float *u, const float *theta,
                           double beta, double qk, double g, int64_t B, int64_t H, int64_t n,
                           int64_t d, int32_t qk_dtype, float *w_re, float *w_im,
                           void *workspace, size_t workspace_bytes, int32_t *status_dev,
                           hipStream_t stream);

/*
 * resolvent_path_product -- the "path_product" of the "Resolvent Operator"
 * page's Rust API for `batch` gate sequences: G_ij = a_{j+1} a_{j+2} ... a_i
 * for j < i, G_ii = 1, 0 above the diagonal, row-major [n, n] each, in f64.
 * Each row is accumulated from k = i down to k = j + 1, the order the page
 * fixes, without fused multiply-adds: the result is that definition evaluated
 * in that order, to the bit.  a_0 is never read.
 *
 * Arguments (device pointers, 8-byte aligned):
 *   a_re, a_im  [batch, n] the gates (f64)
 *   g_re, g_im  [batch, n, n] outputs (f64)
 * Returns RESOLVENT_BAD_SHAPE for a negative size, RESOLVENT_OK with nothing
 * enqueued when batch or n is 0, RESOLVENT_UNSUPPORTED for n > 65536 or
 * batch > 2^24, RESOLVENT_BAD_ARG for a null or misaligned pointer,
 * RESOLVENT_DEVICE_ERROR if the launch failed, else RESOLVENT_OK once the
 * work is enqueued.  No refusal: non-finite gates propagate as in the page's
 * definition.
 */
int32_t resolvent_path_product(const double *a_re, const double *a_im, int64_t batch, int64_t n,
                               double *g_re, double *g_im, hipStream_t stream);

/*
 * resolvent_status_str -- a static, human-readable name of a status code.
 */
const char *resolvent_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* RESOLVENT_H */
