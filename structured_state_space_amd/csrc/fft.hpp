// Register/LDS Stockham FFT for gfx950 workgroups.
//
// The transform follows the radix-two DFT of the pages' definition block
// ("Radix-two discrete Fourier transform": forward root exp(-2 pi i/M), the
// inverse uses the conjugate root; scaling is left to the caller), computed
// as a self-sorting Stockham FFT with radix-2^LOGE passes:
//
//   * N = 2^LOGN points, E = 2^LOGE points per thread, T = N/E threads.
//   * Register layout before and after the transform: thread t holds
//     v[e] = x[t + T*e], e < E (natural order, coalesced global access).
//   * Pass with radix R and span Ns: butterfly b = t + i*T (i < E/R) takes
//     x[b + q*N/R] = v[i + q*E/R], multiplies by exp(-+2 pi i q k/(Ns R)) with
//     k = b mod Ns, does an R-point DFT in registers, and writes output q to
//     (b/Ns)*Ns*R + k + q*Ns.  Between passes the data goes through LDS; the
//     last pass's outputs land in the thread's own register slots, so it needs
//     no exchange.  A transform with P passes does P-1 LDS round trips.
//   * The first pass takes the remainder radix (LOGN mod LOGE), so it carries
//     no twiddles.
//
// LDS addresses are padded by one complex every 16 to spread the strided
// writes of the early passes over more banks.
#pragma once

#include "common.hpp"

namespace ssm {

__host__ __device__ constexpr int lds_pad(int i) { return i + (i >> 4); }
__host__ __device__ constexpr int lds_padded_size(int n) { return n + (n >> 4) + 1; }

// a * exp(-+ 2 pi i K/R) for a compile-time K < R/2, R <= 16
template <int R, int K, bool INV>
__device__ __forceinline__ float2 mul_root(float2 a) {
    constexpr int K16 = K * (16 / R);
    if constexpr (K16 == 0) {
        return a;
    } else if constexpr (K16 == 4) {
        return c_mul_mi<INV>(a);
    } else {
        constexpr float C1 = 0.92387953251128674f, S1 = 0.38268343236508977f, H2 = 0.70710678118654752f;
        constexpr float cs = K16 == 1 ? C1 : K16 == 2 ? H2 : K16 == 3 ? S1 : K16 == 5 ? -S1 : K16 == 6 ? -H2 : -C1;
        constexpr float sn = K16 == 1 ? S1 : K16 == 2 ? H2 : K16 == 3 ? C1 : K16 == 5 ? C1 : K16 == 6 ? H2 : S1;
        return c_mul(a, make_float2(cs, INV ? sn : -sn));
    }
}

template <int R, bool INV, int K = 0>
__device__ __forceinline__ void dft_combine(float2 (&x)[R], const float2 (&e)[R / 2], const float2 (&o)[R / 2]) {
    if constexpr (K < R / 2) {
        const float2 t = mul_root<R, K, INV>(o[K]);
        x[K] = c_add(e[K], t);
        x[K + R / 2] = c_sub(e[K], t);
        dft_combine<R, INV, K + 1>(x, e, o);
    }
}

// In-register R-point DFT, natural order in and out (radix-2 decimation in time).
template <int R, bool INV>
__device__ __forceinline__ void dft_reg(float2 (&x)[R]) {
    if constexpr (R == 2) {
        const float2 a = x[0], b = x[1];
        x[0] = c_add(a, b);
        x[1] = c_sub(a, b);
    } else if constexpr (R > 2) {
        float2 e[R / 2], o[R / 2];
#pragma unroll
        for (int p = 0; p < R / 2; ++p) {
            e[p] = x[2 * p];
            o[p] = x[2 * p + 1];
        }
        dft_reg<R / 2, INV>(e);
        dft_reg<R / 2, INV>(o);
        dft_combine<R, INV>(x, e, o);
    }
}

template <int LOGN, int LOGE, bool INV, int LR, int LS, bool LAST>
__device__ __forceinline__ void stockham_pass(float2 (&v)[1 << LOGE], float2* lds, int t) {
    constexpr int E = 1 << LOGE, N = 1 << LOGN, T = N >> LOGE, R = 1 << LR, NB = E / R, NS = 1 << LS;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int b = t + i * T;
        float2 x[R];
#pragma unroll
        for (int q = 0; q < R; ++q) x[q] = v[i + q * NB];
        if constexpr (NS > 1) {
            const int k = b & (NS - 1);
            const float2 w = root_of_unity<INV>(k, NS * R);
            float2 wq = w;
#pragma unroll
            for (int q = 1; q < R; ++q) {
                x[q] = c_mul(x[q], wq);
                if (q + 1 < R) wq = c_mul(wq, w);
            }
        }
        dft_reg<R, INV>(x);
        if constexpr (LAST) {
#pragma unroll
            for (int q = 0; q < R; ++q) v[i + q * NB] = x[q];
        } else {
            const int base = ((b >> LS) << (LS + LR)) + (b & (NS - 1));
#pragma unroll
            for (int q = 0; q < R; ++q) lds[lds_pad(base + q * NS)] = x[q];
        }
    }
    if constexpr (!LAST) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = lds[lds_pad(t + T * e)];
        __syncthreads();
    }
}

// passes of radix 2^LRMAX, the remainder radix first
template <int LOGN, int LOGE, int LRMAX, bool INV, int P = 0, int LS = 0>
__device__ __forceinline__ void fft_passes(float2 (&v)[1 << LOGE], float2* lds, int t) {
    if constexpr (LOGN > 0) {
        constexpr int REM = LOGN % LRMAX;
        constexpr int NP = LOGN / LRMAX + (REM ? 1 : 0);
        if constexpr (P < NP) {
            constexpr int LR = (P == 0 && REM) ? REM : LRMAX;
            stockham_pass<LOGN, LOGE, INV, LR, LS, P == NP - 1>(v, lds, t);
            fft_passes<LOGN, LOGE, LRMAX, INV, P + 1, LS + LR>(v, lds, t);
        }
    }
}

// Unscaled forward (INV=false) or inverse (INV=true) transform of N = 2^LOGN
// points held as v[e] = x[t + T e]; every thread of the workgroup must call it
// (it contains workgroup barriers).  lds: lds_padded_size(N) complex per
// transform.  Requires LOGE <= LOGN (or LOGN == 0).  Butterflies are at most
// radix 16; a thread with E > 16 points runs E/16 butterflies per pass.
template <int LOGN, int LOGE, bool INV>
__device__ __forceinline__ void fft_block(float2 (&v)[1 << LOGE], float2* lds, int t) {
    static_assert(LOGN == 0 || (LOGE >= 1 && LOGE <= LOGN), "bad FFT split");
    fft_passes<LOGN, LOGE, (LOGE < 4 ? LOGE : 4), INV>(v, lds, t);
}

// elements per thread used for an M-point transform: 16, or 32 at M = 16384 so
// that one transform fits a 512-thread workgroup
__host__ __device__ constexpr int fft_loge(int logn) { return logn < 4 ? logn : (logn >= 14 ? 5 : 4); }

}  // namespace ssm
