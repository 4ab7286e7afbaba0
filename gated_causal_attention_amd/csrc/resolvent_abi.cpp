// resolvent_abi.cpp -- the C entry points declared in include/resolvent.h:
// argument, shape and switch checks (all before any HIP call, so they can be
// exercised without a GPU), workspace sizing, and the launch.
#include "resolvent.h"

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "layout.h"

using namespace resolvent;

namespace {

bool supported(int64_t d, int32_t qk_dtype, int32_t v_dtype) {
    if (d != 64 && d != 128) return false;
    if (qk_dtype == RESOLVENT_BF16) return v_dtype == RESOLVENT_BF16 || v_dtype == RESOLVENT_F32;
    if (qk_dtype == RESOLVENT_F32) return v_dtype == RESOLVENT_F32;
    return false;
}

// Limits that keep every launch grid and in-kernel index in range (the tile
// copies address a head with 32-bit offsets: n * d * 4 bytes < 2^31).
bool within_limits(int64_t B, int64_t H, int64_t n) {
    const int64_t maxn = int64_t(1) << 22;
    if (n > maxn || B > (int64_t(1) << 24) || H > (int64_t(1) << 24)) return false;
    const int64_t BH = B * H;
    if (BH > (int64_t(1) << 24)) return false;
    const int64_t n_pad = (n + BQ - 1) / BQ * BQ;
    return BH * (n_pad / BK) < (int64_t(1) << 31);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The exports write an [n, n] matrix per head: n is capped, and one workgroup
// per (head, row) must fit a 1-D grid.
constexpr int64_t kMaxExportN = 65536;
bool operator_supported(int64_t B, int64_t H, int64_t n, int64_t d, int32_t qk_dtype) {
    if (d != 64 && d != 128) return false;
    if (qk_dtype != RESOLVENT_BF16 && qk_dtype != RESOLVENT_F32) return false;
    if (n > kMaxExportN || B > (int64_t(1) << 24) || H > (int64_t(1) << 24)) return false;
    return B * H <= (int64_t(1) << 24) && B * H * n < (int64_t(1) << 31);
}

bool supported_dv(int64_t dv) { return dv == 64 || dv == 128; }

size_t workspace_grouped(int64_t B, int64_t H, int64_t Hkv, int64_t n, int64_t d, int64_t dv,
                         int32_t qk_dtype, int32_t v_dtype) {
    if (B <= 0 || H <= 0 || Hkv <= 0 || n <= 0 || d <= 0 || dv <= 0 || H % Hkv != 0) return 0;
    if (!supported(d, qk_dtype, v_dtype) || !supported_dv(dv) || !within_limits(B, H, n))
        return 0;
    return make_layout(B, H, n, d, qk_dtype == RESOLVENT_BF16, Hkv, dv, v_dtype == RESOLVENT_F32)
        .total;
}

int32_t forward_impl(const void *q, const void *k, const float *u, const float *theta,
                     const void *v, double beta, double qk, double g, int64_t B, int64_t H,
                     int64_t Hkv, int64_t n, int64_t d, int64_t dv, int32_t qk_dtype,
                     int32_t v_dtype, float *o_re, float *o_im, void *workspace,
                     size_t workspace_bytes, int32_t *status_dev, hipStream_t stream,
                     hipEvent_t *marks) {
    if (B < 0 || H < 0 || Hkv < 0 || n < 0 || d < 0 || dv < 0) return RESOLVENT_BAD_SHAPE;
    if (B == 0 || H == 0 || n == 0) return RESOLVENT_OK;  // empty in, empty out
    if (d == 0 || dv == 0 || Hkv == 0 || H % Hkv != 0) return RESOLVENT_BAD_SHAPE;
    if (!std::isfinite(beta) || !std::isfinite(qk) || !std::isfinite(g))
        return RESOLVENT_NONFINITE;
    if (!supported(d, qk_dtype, v_dtype) || !supported_dv(dv) || !within_limits(B, H, n))
        return RESOLVENT_UNSUPPORTED;
    if (!q || !k || !u || !theta || !v || !o_re || !o_im || !status_dev || !workspace)
        return RESOLVENT_BAD_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_re, 16) ||
        !aligned(o_im, 16) || !aligned(u, 4) || !aligned(theta, 4) || !aligned(status_dev, 4) ||
        !aligned(workspace, 256))
        return RESOLVENT_BAD_ARG;
    const Layout L =
        make_layout(B, H, n, d, qk_dtype == RESOLVENT_BF16, Hkv, dv, v_dtype == RESOLVENT_F32);
    if (workspace_bytes < L.total) return RESOLVENT_BAD_ARG;

    // logit scale in log2 units; the device computes logits in float32
    const double c = qk * 1.4426950408889634074 / std::sqrt((double)d);
    if (qk != 0.0 && !(std::fabs(c) <= (double)FLT_MAX)) return RESOLVENT_NONFINITE;

    Problem P;
    P.q = q;
    P.k = k;
    P.v = v;
    P.u = u;
    P.theta = theta;
    P.o_re = o_re;
    P.o_im = o_im;
    P.status = status_dev;
    P.ws = static_cast<unsigned char *>(workspace);
    P.L = L;
    P.g = g;
    P.c = (float)c;
    P.beta = (float)beta;
    P.beta_mode = beta == 0.0 ? 0 : (beta == 1.0 ? 1 : 2);
    P.qk_zero = (qk == 0.0);
    P.v_f32 = (v_dtype == RESOLVENT_F32);
    const int err = launch_forward(P, stream, reinterpret_cast<void *const *>(marks));
    return err == 0 ? RESOLVENT_OK : RESOLVENT_DEVICE_ERROR;
}

}  // namespace

extern "C" {

size_t resolvent_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, int32_t qk_dtype,
                                 int32_t v_dtype) {
    if (B <= 0 || H <= 0 || n <= 0 || d <= 0) return 0;
    if (!supported(d, qk_dtype, v_dtype) || !within_limits(B, H, n)) return 0;
    return make_layout(B, H, n, d, qk_dtype == RESOLVENT_BF16, 0, 0, v_dtype == RESOLVENT_F32).total;
}

size_t resolvent_counters_offset(int64_t B, int64_t H, int64_t n, int64_t d, int32_t qk_dtype,
                                 int32_t v_dtype) {
    if (resolvent_workspace_bytes(B, H, n, d, qk_dtype, v_dtype) == 0) return SIZE_MAX;
    return make_layout(B, H, n, d, qk_dtype == RESOLVENT_BF16, 0, 0, v_dtype == RESOLVENT_F32)
        .counters;
}

void resolvent_tile_shape(int32_t *bq, int32_t *bk) {
    if (bq) *bq = BQ;
    if (bk) *bk = BK;
}

int32_t resolvent_forward_marked(const void *q, const void *k, const float *u,
                                 const float *theta, const void *v, double beta, double qk,
                                 double g, int64_t B, int64_t H, int64_t n, int64_t d,
                                 int32_t qk_dtype, int32_t v_dtype, float *o_re, float *o_im,
                                 void *workspace, size_t workspace_bytes, int32_t *status_dev,
                                 hipStream_t stream, hipEvent_t *marks) {
    return forward_impl(q, k, u, theta, v, beta, qk, g, B, H, H, n, d, d, qk_dtype, v_dtype,
                        o_re, o_im, workspace, workspace_bytes, status_dev, stream, marks);
}

size_t resolvent_workspace_bytes_grouped(int64_t B, int64_t H, int64_t Hkv, int64_t n,
                                         int64_t d, int64_t dv, int32_t qk_dtype,
                                         int32_t v_dtype) {
    return workspace_grouped(B, H, Hkv, n, d, dv, qk_dtype, v_dtype);
}

int32_t resolvent_forward_grouped(const void *q, const void *k, const float *u,
                                  const float *theta, const void *v, double beta, double qk,
                                  double g, int64_t B, int64_t H, int64_t Hkv, int64_t n,
                                  int64_t d, int64_t dv, int32_t qk_dtype, int32_t v_dtype,
                                  float *o_re, float *o_im, void *workspace,
                                  size_t workspace_bytes, int32_t *status_dev,
                                  hipStream_t stream) {
    return forward_impl(q, k, u, theta, v, beta, qk, g, B, H, Hkv, n, d, dv, qk_dtype, v_dtype,
                        o_re, o_im, workspace, workspace_bytes, status_dev, stream, nullptr);
}

int32_t resolvent_forward(const void *q, const void *k, const float *u, const float *theta,
                          const void *v, double beta, double qk, double g, int64_t B,
                          int64_t H, int64_t n, int64_t d, int32_t qk_dtype, int32_t v_dtype,
                          float *o_re, float *o_im, void *workspace, size_t workspace_bytes,
                          int32_t *status_dev, hipStream_t stream) {
    return resolvent_forward_marked(q, k, u, theta, v, beta, qk, g, B, H, n, d, qk_dtype,
                                    v_dtype, o_re, o_im, workspace, workspace_bytes, status_dev,
                                    stream, nullptr);
}

size_t resolvent_chain_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t dv) {
    if (B <= 0 || H <= 0 || n <= 0 || dv <= 0) return 0;
    if (dv % 64 != 0 || dv > 4096 || !within_limits(B, H, n)) return 0;
    return make_chain_layout(B, H, n, dv).total;
}

int32_t resolvent_chain(const float *u, const float *theta, const void *v, double g, int64_t B,
                        int64_t H, int64_t n, int64_t dv, int32_t v_dtype, float *o_re,
                        float *o_im, void *workspace, size_t workspace_bytes,
                        int32_t *status_dev, hipStream_t stream) {
    if (B < 0 || H < 0 || n < 0 || dv < 0) return RESOLVENT_BAD_SHAPE;
    if (B == 0 || H == 0 || n == 0) return RESOLVENT_OK;  // empty in, empty out
    if (dv == 0) return RESOLVENT_BAD_SHAPE;
    if (!std::isfinite(g)) return RESOLVENT_NONFINITE;
    if (dv % 64 != 0 || dv > 4096 || !within_limits(B, H, n) ||
        (v_dtype != RESOLVENT_BF16 && v_dtype != RESOLVENT_F32))
        return RESOLVENT_UNSUPPORTED;
    if (!u || !theta || !v || !o_re || !o_im || !status_dev || !workspace) return RESOLVENT_BAD_ARG;
    if (!aligned(u, 4) || !aligned(theta, 4) || !aligned(v, v_dtype == RESOLVENT_F32 ? 4 : 2) ||
        !aligned(o_re, 4) || !aligned(o_im, 4) || !aligned(status_dev, 4) ||
        !aligned(workspace, 256))
        return RESOLVENT_BAD_ARG;
    const ChainLayout C = make_chain_layout(B, H, n, dv);
    if (workspace_bytes < C.total) return RESOLVENT_BAD_ARG;
    const int err = launch_chain(C, u, theta, v, v_dtype == RESOLVENT_F32, g, o_re, o_im,
                                 static_cast<unsigned char *>(workspace), status_dev, stream);
    return err == 0 ? RESOLVENT_OK : RESOLVENT_DEVICE_ERROR;
}

size_t resolvent_decode_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t n, int64_t d,
                                        int64_t dv, int32_t qk_dtype, int32_t v_dtype) {
    if (B <= 0 || H <= 0 || Hkv <= 0 || n <= 0 || d <= 0 || dv <= 0 || H % Hkv != 0) return 0;
    if (!supported(d, qk_dtype, v_dtype) || !supported_dv(dv) || !within_limits(B, H, n))
        return 0;
    return make_decode_layout(B, H, Hkv, n, d, dv).total;
}

int32_t resolvent_decode(const void *q, const void *k, const float *u, const float *theta,
                         const void *v, double beta, double qk, double g, int64_t B, int64_t H,
                         int64_t Hkv, int64_t n, int64_t cap, int64_t d, int64_t dv,
                         int32_t qk_dtype, int32_t v_dtype, float *o_re, float *o_im,
                         void *workspace, size_t workspace_bytes, int32_t *status_dev,
                         hipStream_t stream) {
    if (B < 0 || H < 0 || Hkv < 0 || n < 0 || cap < n || d < 0 || dv < 0)
        return RESOLVENT_BAD_SHAPE;
    if (B == 0 || H == 0 || n == 0) return RESOLVENT_OK;  // no position, no readout
    if (d == 0 || dv == 0 || Hkv == 0 || H % Hkv != 0) return RESOLVENT_BAD_SHAPE;
    if (!std::isfinite(beta) || !std::isfinite(qk) || !std::isfinite(g))
        return RESOLVENT_NONFINITE;
    if (!supported(d, qk_dtype, v_dtype) || !supported_dv(dv) || !within_limits(B, H, n) ||
        !within_limits(B, H, cap))
        return RESOLVENT_UNSUPPORTED;
    if (!q || !k || !u || !theta || !v || !o_re || !o_im || !status_dev || !workspace)
        return RESOLVENT_BAD_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_re, 4) ||
        !aligned(o_im, 4) || !aligned(u, 4) || !aligned(theta, 4) || !aligned(status_dev, 4) ||
        !aligned(workspace, 256))
        return RESOLVENT_BAD_ARG;
    const DecodeLayout DL = make_decode_layout(B, H, Hkv, n, d, dv);
    if (workspace_bytes < DL.total) return RESOLVENT_BAD_ARG;
    const double c = qk * 1.4426950408889634074 / std::sqrt((double)d);
    if (qk != 0.0 && !(std::fabs(c) <= (double)FLT_MAX)) return RESOLVENT_NONFINITE;
    const int err = launch_decode(DL, q, k, u, theta, v, cap, qk_dtype == RESOLVENT_F32,
                                  v_dtype == RESOLVENT_F32, g, (float)c, (float)beta,
                                  beta == 0.0 ? 0 : (beta == 1.0 ? 1 : 2), qk == 0.0, o_re, o_im,
                                  static_cast<unsigned char *>(workspace), status_dev, stream);
    return err == 0 ? RESOLVENT_OK : RESOLVENT_DEVICE_ERROR;
}

int32_t resolvent_chain_step(float *y_re, float *y_im, const float *u, const float *theta,
                             const void *v, double g, int64_t B, int64_t H, int64_t dv,
                             int32_t v_dtype, int32_t *status_dev, hipStream_t stream) {
    if (B < 0 || H < 0 || dv < 0) return RESOLVENT_BAD_SHAPE;
    if (B == 0 || H == 0 || dv == 0) return RESOLVENT_OK;
    if (!std::isfinite(g)) return RESOLVENT_NONFINITE;
    if ((v_dtype != RESOLVENT_BF16 && v_dtype != RESOLVENT_F32) || B * H > (int64_t(1) << 24) ||
        dv > 4096)
        return RESOLVENT_UNSUPPORTED;
    if (!y_re || !y_im || !u || !theta || !v || !status_dev) return RESOLVENT_BAD_ARG;
    if (!aligned(y_re, 4) || !aligned(y_im, 4) || !aligned(u, 4) || !aligned(theta, 4) ||
        !aligned(v, v_dtype == RESOLVENT_F32 ? 4 : 2) || !aligned(status_dev, 4))
        return RESOLVENT_BAD_ARG;
    const int err = launch_chain_step(y_re, y_im, u, theta, v, v_dtype == RESOLVENT_F32, g, B * H,
                                      dv, status_dev, stream);
    return err == 0 ? RESOLVENT_OK : RESOLVENT_DEVICE_ERROR;
}

size_t resolvent_operator_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d,
                                          int32_t qk_dtype) {
    if (B <= 0 || H <= 0 || n <= 0 || d <= 0) return 0;
    if (!operator_supported(B, H, n, d, qk_dtype)) return 0;
    return make_operator_layout(B, H, n, d).total;
}

int32_t resolvent_operator(const void *q, const void *k, const float *u, const float *theta,
                           double beta, double qk, double g, int64_t B, int64_t H, int64_t n,
                           int64_t d, int32_t qk_dtype, float *w_re, float *w_im,
                           void *workspace, size_t workspace_bytes, int32_t *status_dev,
                           hipStream_t stream) {
    if (B < 0 || H < 0 || n < 0 || d < 0) return RESOLVENT_BAD_SHAPE;
    if (B == 0 || H == 0 || n == 0) return RESOLVENT_OK;
    if (d == 0) return RESOLVENT_BAD_SHAPE;
    if (!std::isfinite(beta) || !std::isfinite(qk) || !std::isfinite(g))
        return RESOLVENT_NONFINITE;
    if (!operator_supported(B, H, n, d, qk_dtype)) return RESOLVENT_UNSUPPORTED;
    if (!q || !k || !u || !theta || !w_re || !w_im || !status_dev || !workspace)
        return RESOLVENT_BAD_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(u, 4) || !aligned(theta, 4) ||
        !aligned(w_re, 4) || !aligned(w_im, 4) || !aligned(status_dev, 4) ||
        !aligned(workspace, 256))
        return RESOLVENT_BAD_ARG;
    const OperatorLayout OL = make_operator_layout(B, H, n, d);
    if (workspace_bytes < OL.total) return RESOLVENT_BAD_ARG;
    const double c = qk * 1.4426950408889634074 / std::sqrt((double)d);
    if (qk != 0.0 && !(std::fabs(c) <= (double)FLT_MAX)) return RESOLVENT_NONFINITE;
    const int err = launch_operator(OL, q, k, u, theta, qk_dtype == RESOLVENT_F32, g, (float)c,
                                    (float)beta, beta == 0.0 ? 0 : (beta == 1.0 ? 1 : 2),
                                    qk == 0.0, w_re, w_im,
                                    static_cast<unsigned char *>(workspace), status_dev, stream);
    return err == 0 ? RESOLVENT_OK : RESOLVENT_DEVICE_ERROR;
}

int32_t resolvent_path_product(const double *a_re, const double *a_im, int64_t batch, int64_t n,
                               double *g_re, double *g_im, hipStream_t stream) {
    if (batch < 0 || n < 0) return RESOLVENT_BAD_SHAPE;
    if (batch == 0 || n == 0) return RESOLVENT_OK;
    if (n > kMaxExportN || batch > (int64_t(1) << 24) || batch * ((n + 63) / 64) >= (int64_t(1) << 31))
        return RESOLVENT_UNSUPPORTED;
    if (!a_re || !a_im || !g_re || !g_im) return RESOLVENT_BAD_ARG;
    if (!aligned(a_re, 8) || !aligned(a_im, 8) || !aligned(g_re, 8) || !aligned(g_im, 8))
        return RESOLVENT_BAD_ARG;
    const int err = launch_path_product(a_re, a_im, batch, n, g_re, g_im, stream);
    return err == 0 ? RESOLVENT_OK : RESOLVENT_DEVICE_ERROR;
}

const char *resolvent_status_str(int32_t status) {
    switch (status) {
        case RESOLVENT_OK: return "ok";
        case RESOLVENT_NONFINITE: return "non-finite input refused";
        case RESOLVENT_BAD_SHAPE: return "bad shape";
        case RESOLVENT_BAD_ARG: return "bad argument";
        case RESOLVENT_UNSUPPORTED: return "unsupported head_dim or dtype";
        case RESOLVENT_DEVICE_ERROR: return "device error";
        case RESOLVENT_TOO_LARGE: return "problem exceeds the no-allocation scratch";
        default: return "unknown status";
    }
}

}  // extern "C"
