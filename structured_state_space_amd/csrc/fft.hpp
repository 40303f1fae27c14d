// Register/LDS Stockham FFT for gfx950 workgroups.
//
// The transform follows the radix-two DFT of the pages' definition block
// ("Radix-two discrete Fourier transform": forward root exp(-2 pi i/M), the
// inverse uses the conjugate root; scaling is left to the caller), computed
// as a self-sorting Stockham FFT with radix <= 16 passes:
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
//   * The first pass takes the remainder radix, so it carries no twiddles.
//   * NV independent vectors of the same size can be transformed together:
//     they share the twiddles and the workgroup barriers of every exchange.
//   * Twiddles come from a functor tw(k, n) = exp(-2 pi i k/n) (forward sign);
//     the inverse conjugates it.  Powers w^q are formed by repeated products.
//
// LDS addresses are padded by one complex every 16 to spread the strided
// writes of the early passes over more banks.
#pragma once

#include "common.hpp"

namespace ssm {

__host__ __device__ constexpr int lds_pad(int i) { return i + (i >> 4); }

// Synchronisation of an LDS exchange: the workgroup barrier, or (WAVE: the
// transform is held by a single wavefront) a wave-level barrier with release /
// acquire fences, which orders the wave's own LDS writes and reads.
template <bool WAVE>
__device__ __forceinline__ void lds_sync() {
    if constexpr (WAVE) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        __syncthreads();
    }
}
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

// Twiddle sources: get<P, n>(i, k) = exp(-2 pi i k/n) for butterfly i of pass P.

// exact sin/cos of pi*num/den (den a power of two), computed where used
struct TwiddleSincos {
    template <int P, int n>
    __device__ __forceinline__ float2 get(int, int k) const { return root_of_unity<false>(k, n); }
};

// lookup in tab[j] = exp(-i pi j/M), j < M (the 2M-th roots), for lengths n
// dividing M: exp(-2 pi i k/n) is entry 2kM/n, and the upper half follows
// from exp(-i pi (j + M)/M) = -exp(-i pi j/M)
__device__ __forceinline__ float2 table_root(const float2* tab, int logm, int k, int logn) {
    const int i = k << (logm + 1 - logn);  // 2kM/n < 2M (n divides M)
    const int m = 1 << logm;
    const float2 w = tab[i & (m - 1)];
    return i >= m ? make_float2(-w.x, -w.y) : w;
}

// all pass twiddles of one thread, read from the table once and kept in
// registers: every transform of the same plan (forward or inverse) reuses them
template <int LOGN, int LOGE, int LRMAX = (LOGE < 4 ? LOGE : 4)>
struct TwiddleRegs {
    static constexpr int E = 1 << LOGE, T = (1 << LOGN) >> LOGE;
    static constexpr int REM = LOGN > 0 ? LOGN % LRMAX : 0;
    static constexpr int NP = LOGN > 0 ? LOGN / LRMAX + (REM ? 1 : 0) : 0;
    static constexpr int NBMAX = E >= 2 ? E / 2 : 1;
    float2 w[NP > 0 ? NP : 1][NBMAX];

    __device__ __forceinline__ TwiddleRegs(const float2* tab, int logm, int t) {
        int ls = 0;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int lr = (p == 0 && REM) ? REM : LRMAX;
            const int ns = 1 << ls;
#pragma unroll
            for (int i = 0; i < NBMAX; ++i)
                if (i < (E >> lr) && ns > 1) w[p][i] = table_root(tab, logm, (t + i * T) & (ns - 1), ls + lr);
            ls += lr;
        }
    }
    template <int P, int n>
    __device__ __forceinline__ float2 get(int i, int) const { return w[P][i]; }
};

template <int NV, int LOGN, int LOGE, bool INV, int P, int LR, int LS, bool LAST, bool SHARED, bool WAVE, class TW>
__device__ __forceinline__ void stockham_pass(float2 (&v)[NV][1 << LOGE], float2* const (&lds)[NV], int t,
                                              const TW& tw) {
    constexpr int E = 1 << LOGE, N = 1 << LOGN, T = N >> LOGE, R = 1 << LR, NB = E / R, NS = 1 << LS;
    if constexpr (NS > 1) {  // twiddles, shared by the NV vectors
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            float2 w = tw.template get<P, NS * R>(i, (t + i * T) & (NS - 1));
            if (INV) w.y = -w.y;
            // the powers of w are formed here, per pass and call: an empty asm
            // keeps the compiler from hoisting or sharing them across passes and
            // transforms, where their registers would stay live (and spill)
            asm volatile("" : "+v"(w.x), "+v"(w.y));
            float2 wq = w;
#pragma unroll
            for (int q = 1; q < R; ++q) {
#pragma unroll
                for (int s = 0; s < NV; ++s) v[s][i + q * NB] = c_mul(v[s][i + q * NB], wq);
                if (q + 1 < R) wq = c_mul(wq, w);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < NV; ++s) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int b = t + i * T;
            float2 x[R];
#pragma unroll
            for (int q = 0; q < R; ++q) x[q] = v[s][i + q * NB];
            dft_reg<R, INV>(x);
            if constexpr (LAST) {
#pragma unroll
                for (int q = 0; q < R; ++q) v[s][i + q * NB] = x[q];
            } else {
                // lds_pad(base + q NS) = lds_pad(base) + q NS + (q NS >> 4) for these
                // power-of-two strides, so one address register serves the R
                // stores (compile-time offsets)
                float2* const pb = lds[s] + lds_pad(((b >> LS) << (LS + LR)) + (b & (NS - 1)));
#pragma unroll
                for (int q = 0; q < R; ++q) pb[q * NS + ((q * NS) >> 4)] = x[q];
            }
        }
        if constexpr (!LAST && SHARED) {  // one buffer for all vectors: exchange them in turn
            lds_sync<WAVE>();
            const float2* const pr = lds[s] + lds_pad(t);  // lds_pad(t + T e) = lds_pad(t) + T e + (T e >> 4)
#pragma unroll
            for (int e = 0; e < E; ++e) v[s][e] = pr[T * e + ((T * e) >> 4)];
            lds_sync<WAVE>();
        }
    }
    if constexpr (!LAST && !SHARED) {
        lds_sync<WAVE>();
#pragma unroll
        for (int s = 0; s < NV; ++s) {
            const float2* const pr = lds[s] + lds_pad(t);  // lds_pad(t + T e) = lds_pad(t) + T e + (T e >> 4)
#pragma unroll
            for (int e = 0; e < E; ++e) v[s][e] = pr[T * e + ((T * e) >> 4)];
        }
        lds_sync<WAVE>();
    }
}

// passes of radix 2^LRMAX, the remainder radix first
template <int NV, int LOGN, int LOGE, int LRMAX, bool INV, bool SHARED, bool WAVE, class TW, int P = 0,
          int LS = 0>
__device__ __forceinline__ void fft_passes(float2 (&v)[NV][1 << LOGE], float2* const (&lds)[NV], int t,
                                           const TW& tw) {
    if constexpr (LOGN > 0) {
        constexpr int REM = LOGN % LRMAX;
        constexpr int NP = LOGN / LRMAX + (REM ? 1 : 0);
        if constexpr (P < NP) {
            constexpr int LR = (P == 0 && REM) ? REM : LRMAX;
            stockham_pass<NV, LOGN, LOGE, INV, P, LR, LS, P == NP - 1, SHARED, WAVE>(v, lds, t, tw);
            fft_passes<NV, LOGN, LOGE, LRMAX, INV, SHARED, WAVE, TW, P + 1, LS + LR>(v, lds, t, tw);
        }
    }
}

// Unscaled forward (INV=false) or inverse (INV=true) transforms of NV vectors of
// N = 2^LOGN points, each held as v[s][e] = x_s[t + T e]; every thread of the
// workgroup must call it (it contains workgroup barriers), unless WAVE: then
// the T = N/E threads are exactly one wavefront, only that wave calls it, and
// the exchanges synchronise the wave alone.  lds[s]:
// lds_padded_size(N) complex per vector; SHARED: all lds[s] are one buffer and
// the vectors are exchanged in turn.  Requires LOGE <= LOGN (or LOGN == 0).
// Butterflies are at most radix 16; a thread with E > 16 points runs E/16
// butterflies per pass.
template <int NV, int LOGN, int LOGE, bool INV, bool SHARED = false, int LRMAX = (LOGE < 4 ? LOGE : 4),
          bool WAVE = false, class TW>
__device__ __forceinline__ void fft_multi(float2 (&v)[NV][1 << LOGE], float2* const (&lds)[NV], int t,
                                          const TW& tw) {
    static_assert(!WAVE || (LOGN - LOGE) == 6, "a wave-level transform takes exactly 64 threads");
    static_assert(LOGN == 0 || (LOGE >= 1 && LOGE <= LOGN), "bad FFT split");
    static_assert(LOGN == 0 || (LRMAX >= 1 && LRMAX <= LOGE && LRMAX <= 4), "bad radix");
    fft_passes<NV, LOGN, LOGE, LRMAX, INV, SHARED, WAVE, TW>(v, lds, t, tw);
}

// single vector, sin/cos twiddles
template <int LOGN, int LOGE, bool INV>
__device__ __forceinline__ void fft_block(float2 (&v)[1 << LOGE], float2* lds, int t) {
    float2(&vv)[1][1 << LOGE] = *reinterpret_cast<float2(*)[1][1 << LOGE]>(&v);
    float2* const l[1] = {lds};
    fft_multi<1, LOGN, LOGE, INV>(vv, l, t, TwiddleSincos{});
}

// elements per thread used for an M-point transform: 16, or 32 at M = 16384 so
// that one transform fits a 512-thread workgroup
__host__ __device__ constexpr int fft_loge(int logn) { return logn < 4 ? logn : (logn >= 14 ? 5 : 4); }

}  // namespace ssm
