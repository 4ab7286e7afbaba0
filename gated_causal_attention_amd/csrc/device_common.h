// device_common.h -- device helpers shared by the decode and export kernels:
// gates and their products in f64, 16-byte row loads, wave reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace resolvent {
namespace dev {

// A gate or a product of gates: complex value and modulus (f64).
struct Cg {
    double re, im, m;
};
__device__ __forceinline__ Cg cg_one() { return {1.0, 0.0, 1.0}; }
__device__ __forceinline__ Cg cg_mul(Cg a, Cg b) {
    return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re, a.m * b.m};
}
__device__ __forceinline__ Cg cg_down(Cg a, int o) {
    return {__shfl_down(a.re, o), __shfl_down(a.im, o), __shfl_down(a.m, o)};
}
__device__ __forceinline__ Cg cg_lane(Cg a, int l) {
    return {__shfl(a.re, l), __shfl(a.im, l), __shfl(a.m, l)};
}

// Gate of one position (section "Object": blend, then modulus and phase):
// l = clamp((1-g) + g u, 0, 1), a = l e^{i g theta}, |a| = l, in f64 as the
// forward pass's gates kernel evaluates it.
__device__ __forceinline__ Cg gate_of(float uu, float tt, double g, bool &bad) {
#pragma clang fp contract(off)
    double l = (1.0 - g) * 1.0 + g * (double)uu;
    l = l < 0.0 ? 0.0 : (l > 1.0 ? 1.0 : l);
    const double tp = g * (double)tt;
    if (!isfinite(uu) || !isfinite(tt) || !isfinite(tp)) bad = true;
    return {l * cos(tp), l * sin(tp), l};
}

// 16 bytes at element offset e (a multiple of 4 resp. 8 elements).
template <bool F32>
__device__ __forceinline__ uint4 load16(const void *p, int64_t e) {
    return *reinterpret_cast<const uint4 *>(static_cast<const char *>(p) + e * (F32 ? 4 : 2));
}
// The 4 (fp32) or 8 (bf16) values of a 16-byte word.
template <bool F32>
__device__ __forceinline__ void unpack16(uint4 w, float *x) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(u[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(u[e] << 16);
            x[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
    }
}

// x f for the final scale of a readout or weight: an exactly zero x stays
// (signed) zero when f overflows to inf ("Evaluation and refusals": an
// overflowing weight reads +inf, a zero lane of a product stays 0, never NaN).
__device__ __forceinline__ float scale_keep_zero(float x, float f) { return x == 0.0f ? x : x * f; }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

}  // namespace dev
}  // namespace resolvent
