// Shared device/host helpers for the gfx950 S4 filter kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// ---- complex float helpers (interleaved re/im, torch.complex64 layout) ----
__device__ __forceinline__ float2 c_add(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 c_sub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 c_mul(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 c_conj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 c_scale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
// multiply by -i (forward) or +i (inverse)
template <bool INV>
__device__ __forceinline__ float2 c_mul_mi(float2 a) {
    return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// ---- complex double helpers (discretisation runs in float64) ----
__device__ __forceinline__ double2 z_add(double2 a, double2 b) { return make_double2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ double2 z_sub(double2 a, double2 b) { return make_double2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ double2 z_mul(double2 a, double2 b) {
    return make_double2(fma(a.x, b.x, -a.y * b.y), fma(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ double2 z_conj(double2 a) { return make_double2(a.x, -a.y); }
__device__ __forceinline__ double2 z_scale(double2 a, double s) { return make_double2(a.x * s, a.y * s); }
__device__ __forceinline__ bool z_is_zero(double2 a) { return a.x == 0.0 && a.y == 0.0; }
// 1/a by scaled division (Smith's method), finite for any nonzero finite a
__device__ __forceinline__ double2 z_inv(double2 a) {
    if (fabs(a.x) >= fabs(a.y)) {
        double t = a.y / a.x, d = a.x + a.y * t;
        return make_double2(1.0 / d, -t / d);
    }
    double t = a.x / a.y, d = a.x * t + a.y;
    return make_double2(t / d, -1.0 / d);
}
__device__ __forceinline__ double2 z_from(float2 a) { return make_double2((double)a.x, (double)a.y); }
__device__ __forceinline__ float2 c_from(double2 a) { return make_float2((float)a.x, (float)a.y); }

__device__ __forceinline__ float2 c_nan() { return make_float2(__builtin_nanf(""), __builtin_nanf("")); }

// exp(-2 pi i * num/den) (INV=false) or exp(+2 pi i * num/den); num/den must be
// exact in float (den a power of two, num < 2^24).
template <bool INV>
__device__ __forceinline__ float2 root_of_unity(int num, int den) {
    float s, c;
    sincospif(2.0f * (float)num / (float)den, &s, &c);
    return make_float2(c, INV ? s : -s);
}

// integer helpers shared by host and device
__host__ __device__ constexpr int ilog2_exact(long long v) {
    int l = 0;
    while ((1LL << l) < v) ++l;
    return l;
}

// ---- workspace layout (one definition for sizing and for the entry points) ----
struct WsLayout {
    size_t roots = 0, roots_bytes = 0;     // [H, M] complex64: root values H(z_k)
    size_t tstat = 0, tstat_bytes = 0;     // [H, tiles] int32: per-root-tile statuses
    size_t tant = 0, tant_bytes = 0;       // [M] float64: tan(pi k/M)
    size_t khat = 0, khat_bytes = 0;       // [H, 2, M] complex64: conv spectra (cyclic, twisted)
    size_t tw = 0, tw_bytes = 0;           // [M] complex64: exp(-i pi j/M), the conv's twiddles
    size_t big = 0, big_bytes = 0;         // scratch of the multi-pass transforms (M > 16384)
    size_t kbuf = 0, kbuf_bytes = 0;       // [H, L] complex64: the kernel (complex output, no K_out given)
    size_t khat2 = 0, khat2_bytes = 0;     // [H, 2, M] complex64: spectra of Im K (complex output, shared-transform lengths)
    size_t tw4 = 0, tw4_bytes = 0;         // [2M] complex64: exp(-i pi j/(2M)), the wave-structured transforms' twiddles
    size_t cprep = 0, cprep_bytes = 0;     // [H] per-channel records of the split-precision root values (ranks 2, 3)
    size_t total = 0;
};

constexpr int kMaxLdsLogM = 14;           // M <= 16384 runs LDS-resident
// multi-pass convolution: row pairs per chunk (the intermediate of a chunk,
// 2 M complex per pair, is the workspace's multi-pass region; 128 pairs at
// M = 65536 is 134 MB, inside the 256 MB Infinity Cache)
constexpr int kConvChunkPairs = 128;
constexpr int kMaxLogM = 16;              // M <= 65536 supported
constexpr int kCauchyThreads = 256;

}  // namespace ssm
