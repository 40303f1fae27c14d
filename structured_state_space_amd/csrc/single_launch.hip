// The whole filter path in one launch for 1024-point transforms: one
// 1024-thread workgroup per channel computes the channel's root values, its
// kernel and spectra, and the convolution of all its batch rows.
//
// Sources: "Recurrent, LSTM, and structured state-space models" -- S4
// Algorithm 1 / App. C (root values of the truncated generating function at
// the M-th roots of unity, the kernel as the first L coefficients of their
// inverse transform), DPLR block (y = K * u + D u) and radix-two DFT block
// (exact linear product by zero padding).
//
// Used where every channel's rows fit one workgroup (at most four row pairs)
// and there are enough channels to give every CU a workgroup.  Against the
// two-launch form it keeps the root values in LDS, loads the input rows while
// the root values are being finished, and has no second launch.
//
// Phase A (all 1024 threads, one root each): as the root-value kernel with one
// root per thread (roots.hpp: sums on the matrix cores); the twiddles
// exp(-i pi j/M) go to LDS; the root values to LDS.
// Phase B: each transform is held by one 64-lane wave, so its LDS exchanges
// synchronise that wave alone; the workgroup barrier is met only between
// stages, by every wave.  z-half i = 2p + c is row pair p's input
// z = u_{2p} + i u_{2p+1}, twisted by exp(-i pi j/M) when c = 1 (the two halves
// of the zero-padded product, as in the convolution kernel).  Waves 1-8 own
// z-halves 0-7.
//   B1: wave 0 transforms the conjugated root values (the inverse transform of
//       the root values: the kernel); waves 1-8 their z-halves (1024 points,
//       16 per lane, radix-16 passes).
//   B2: the kernel's cyclic and twisted spectra, each split over four waves
//       (0 and 9-15) by one radix-4 decimation-in-frequency step: a 256-point
//       transform per wave.
//   B3: waves 1-8 multiply by the spectrum of their half and inverse-
//       transform; the twisted halves are untwisted and added to the cyclic
//       ones through LDS; rows are stored.
// With no rows (Bsz = 0) the launch is the kernel generator's: phase A (the
// root values also written out when asked for) and the kernel transform of
// B1, then it returns.
#include <float.h>

#include "common.hpp"
#include "fft.hpp"
#include "roots.hpp"

namespace ssm {

namespace {

constexpr int kLogM1 = 10, kM1 = 1 << kLogM1;
constexpr int kThreads1 = 1024;
constexpr int kLogE1 = 4, kE1 = 1 << kLogE1, kT1 = kM1 >> kLogE1;  // 16 points per lane, one wave per transform
static_assert(kT1 == 64, "phase B transforms are one wave each");
constexpr int kPairs1 = 4;                                          // row pairs per channel
constexpr int kBufs1 = 2 * kPairs1 + 1;                             // exchange buffers: waves 0 .. 2 kPairs1
constexpr int kLdsV1 = lds_padded_size(kM1);
// spectra stage: four 256-point transforms per spectrum, one wave each
constexpr int kLogN2 = 8, kN2 = 1 << kLogN2, kLogE2 = 2, kE2 = 1 << kLogE2, kT2 = kN2 >> kLogE2;
static_assert(kT2 == 64 && 4 * kN2 == kM1, "spectra split: four one-wave transforms of M/4 points");
static_assert(8 * lds_padded_size(kN2) <= kBufs1 * kLdsV1, "spectra split: exchange buffers");
static_assert(4 * lds_padded_size(kN2) <= 2 * kM1, "kernel transform split: exchange buffers in the spectra array");

// a * (-i)^k for a runtime k in 0..3
__device__ __forceinline__ float2 c_mul_mi_pow(float2 a, int k) {
    const float2 r = (k & 1) ? make_float2(a.y, -a.x) : a;
    return (k & 2) ? make_float2(-r.x, -r.y) : r;
}

template <int RK>
__global__ __launch_bounds__(kThreads1) void filter_m1024_kernel(
    int Bsz, int H, int N, int L, const float2* __restrict__ Lambda, const float2* __restrict__ P,
    const float2* __restrict__ Q, const float2* __restrict__ Bv, const float2* __restrict__ Ct,
    const float* __restrict__ dt, const float* __restrict__ D, const float* __restrict__ u, float* __restrict__ y,
    float2* __restrict__ K_out, int32_t* __restrict__ status, float2* __restrict__ roots_out) {
    constexpr int M = kM1, E = kE1, T = kT1;
    constexpr int F = Fam<RK>::F, kChunk = Fam<RK>::CHUNK, U = sweep_unroll<RK, 1>();
    __shared__ float2 hdr[kChunk];
    __shared__ float4 wt[kChunk * Fam<RK>::WROW];
    __shared__ float2 twl[M];       // exp(-i pi j/M)
    __shared__ float2 rootl[M];     // root values
    __shared__ float kl[M];         // real kernel taps (+D), scaled 1/(2M)
    __shared__ float2 khl[2][M];    // cyclic and twisted spectra
    // exchange buffers: wave w <= 8 uses buffer w for its 1024-point transforms;
    // the spectra stage (waves 0 and 9-15) uses the start of the array
    __shared__ float2 fbuf[kBufs1][kLdsV1];
    __shared__ int blk_status;
    __shared__ double2 red[kThreads1 / 64];

    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t hbase = (size_t)h * N;
    // wave index (uniform: roles are scalar branches) and lane; waves 1-8 own
    // z-half zi = wave - 1 of row pair pr
    const int wv = __builtin_amdgcn_readfirstlane(tid / T);
    const int t = tid - wv * T;
    const bool zwave = wv >= 1 && wv <= 2 * kPairs1;
    const int zi = zwave ? wv - 1 : 0;
    const int pr = zi >> 1, half = zi & 1;
    const int npb = (Bsz + 1) / 2;
    const bool pact = zwave && pr < npb;
    const int b1 = 2 * pr;
    const bool has2 = pact && b1 + 1 < Bsz;
    const size_t row1 = pact ? ((size_t)b1 * H + h) * (size_t)L : 0;
    const size_t row2 = has2 ? row1 + (size_t)H * L : row1;

    float2 z[E];

    // ---- phase A: root values, one per thread (k = tid) ----
    // one state's inputs (lambda_n, C~_n, B_n, Q_n, P_n) for staging
    struct StateIn {
        float2 lam, uu[RK + 1], vv[RK + 1];
    };
    auto load_state = [&](int n) {
        StateIn si;
        const size_t hn = hbase + n;
        si.lam = Lambda[hn];
        si.uu[0] = Ct[hn];
        si.vv[0] = Bv[hn];
#pragma unroll
        for (int j = 0; j < RK; ++j) {
            si.uu[1 + j] = Q[hn * RK + j];
            si.vv[1 + j] = P[hn * RK + j];
        }
        return si;
    };
    // the first chunk's inputs are loaded before anything else, so that their
    // latency overlaps the float64 twiddle and tangent work below
    StateIn first{};
    if (tid < min(kChunk, N)) first = load_state(tid);
    if (tid == 0) blk_status = 0;
    const float dtv = dt[h];
    const bool bad_dt = !(dtv > 0.0f) || !(dtv <= FLT_MAX);  // uniform
    const int k = tid;
    double sn, cs;
    sincospi((double)k / (double)M, &sn, &cs);
    twl[k] = make_float2((float)cs, (float)-sn);
    const double tk = (2 * k == M) ? 0.0 : sn / cs;
    const double a = bad_dt ? 0.0 : 2.0 / (double)dtv;
    const float st[1] = {(float)(a * tk)};
    RootAcc<RK> acc[1];
    acc_zero<RK>(acc[0]);
    // issue priority falls with progress through the states so that the
    // block's waves advance together (the phase ends at a barrier)
    const int q1 = N / 4, q2 = N / 2, q3 = (3 * N) / 4;
    __builtin_amdgcn_s_setprio(3);
    double m1x = 0.0, m1y = 0.0;
    for (int n0 = 0; n0 < N; n0 += kChunk) {
        const int nch = min(kChunk, N - n0);
        const int npad = (nch + U - 1) / U * U;
        if (n0 > 0) __syncthreads();  // the previous chunk's sweep is done with the table
        if (tid >= nch && tid < npad) stage_pad<RK>(hdr + tid, wt + tid * Fam<RK>::WROW);
        if (tid < nch) {
            const StateIn si = n0 == 0 ? first : load_state(n0 + tid);
            // z = -1 takes (dt/2) C~^* B: partial sums in float64
            m1x += (double)si.uu[0].x * si.vv[0].x + (double)si.uu[0].y * si.vv[0].y;
            m1y += (double)si.uu[0].x * si.vv[0].y - (double)si.uu[0].y * si.vv[0].x;
            stage_state<RK>(hdr + tid, wt + tid * Fam<RK>::WROW, si.lam, si.uu, si.vv);
        }
        __syncthreads();
        sweep_chunk<RK, 1, U, true>(hdr, wt, npad, n0, q1, q2, q3, st, acc);
    }
    __builtin_amdgcn_s_setprio(0);
    // the z-half's input rows, fetched after the sweep (loads in flight during
    // it were measured to slow it by more than their latency costs here, where
    // the barrier wait and the root finish hide it)
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = t + T * e;
        const bool in = pact && j < L;
        z[e] = make_float2(in ? u[row1 + j] : 0.0f, (in && has2) ? u[row2 + j] : 0.0f);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        m1x += __shfl_xor(m1x, o, 64);
        m1y += __shfl_xor(m1y, o, 64);
    }
    if ((tid & 63) == 0) red[tid >> 6] = make_double2(m1x, m1y);
    __syncthreads();
    int my_status = 0;
    float2 sums[F];
    acc_unpack<RK>(acc[0], sums);
    float2 Hk;
    if (2 * k == M) {  // z = -1: (dt/2) C~^* B
        double2 m1 = make_double2(0.0, 0.0);
#pragma unroll
        for (int wv = 0; wv < kThreads1 / 64; ++wv) {
            m1.x += red[wv].x;
            m1.y += red[wv].y;
        }
        Hk = make_float2((float)(0.5 * dtv * m1.x), (float)(0.5 * dtv * m1.y));
    } else {
        Hk = finish_root<RK>(sums, st[0], (float)tk, N, hbase, Lambda, P, Q, Bv, Ct, my_status);
    }
    if (bad_dt) {
        my_status = SSM_ST_INVALID_STEP;
        Hk = c_nan();
    }
    rootl[k] = Hk;
    if (roots_out) roots_out[(size_t)h * M + k] = Hk;
    if (my_status) atomicMax(&blk_status, my_status);
    __syncthreads();
    const int chst = blk_status;
    if (tid == 0 && status) status[h] = chst;

    // ---- phase B ----
    const TwiddleRegs<kLogM1, kLogE1> tw(twl, kLogM1, t);
    float2* const mine[1] = {fbuf[min(wv, kBufs1 - 1)]};  // used by waves 0-8 only
    float2 x[1][E];
    const float invM = 1.0f / (float)M, sc = 1.0f / (float)(2 * M);

    // B1: the kernel's inverse transform, as the forward transform of the
    // conjugated root values, split over waves 0, 9, 10 and 11 (one per SIMD
    // beside the z-waves' two each) by one radix-4 step of decimation in
    // frequency, as in B2; their exchange buffers are the spectra array,
    // which B2 fills only after the barrier
    if (wv == 0 || (wv >= 9 && wv <= 11)) {
        const int q = wv == 0 ? 0 : wv - 8;
        float2 w[1][kE2];
#pragma unroll
        for (int e = 0; e < kE2; ++e) {
            const int m = t + kT2 * e;
            float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) acc = c_add(acc, c_mul_mi_pow(c_conj(rootl[m + kN2 * pp]), (pp * q) & 3));
            w[0][e] = c_mul(acc, table_root(twl, kLogM1, (m * q) & (M - 1), kLogM1));
        }
        const TwiddleRegs<kLogN2, kLogE2> tw2(twl, kLogM1, t);
        float2* const buf2[1] = {&khl[0][0] + q * lds_padded_size(kN2)};
        fft_multi<1, kLogN2, kLogE2, false, false, kLogE2, true>(w, buf2, t, tw2);
#pragma unroll
        for (int e = 0; e < kE2; ++e) {
            const int j = 4 * (t + kT2 * e) + q;
            const float2 kv = c_scale(c_conj(w[0][e]), invM);
            if (K_out && j < L) K_out[(size_t)h * L + j] = chst ? c_nan() : kv;
            float kr = j < L ? kv.x : 0.0f;
            if (j == 0 && D) kr += D[h];
            kl[j] = kr * sc;
        }
    } else if (zwave && Bsz > 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[0][e] = half ? c_mul(z[e], twl[t + T * e]) : z[e];
        fft_multi<1, kLogM1, kLogE1, false, false, 4, true>(x, mine, t, tw);
    }
    __syncthreads();
    if (Bsz == 0) return;  // the kernel alone (uniform: no barrier follows for anyone)

    // B2: the cyclic (c = 0) and twisted (c = 1) spectra, each split over four
    // of the free waves (0 and 9-15) by one radix-4 step of decimation in
    // frequency: with j = m + 256 p and k = 4 s + q,
    //   X[4s + q] = sum_m w256^{ms} [w1024^{mq} sum_p x[m + 256 p] (-i)^{pq}],
    // so wave q forms its 256 inputs from the taps in LDS and runs a 256-point
    // transform (4 points per lane); the exchange buffers of waves 0-2 are free
    if (wv == 0 || wv >= 9) {
        const int idx = wv == 0 ? 0 : wv - 8;
        const int c = idx >> 2, q = idx & 3;
        float2 w[1][kE2];
#pragma unroll
        for (int e = 0; e < kE2; ++e) {
            const int m = t + kT2 * e;
            float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const int j = m + kN2 * pp;
                const float2 xv = c ? c_scale(twl[j], kl[j]) : make_float2(kl[j], 0.0f);
                acc = c_add(acc, c_mul_mi_pow(xv, (pp * q) & 3));
            }
            w[0][e] = c_mul(acc, table_root(twl, kLogM1, (m * q) & (M - 1), kLogM1));
        }
        const TwiddleRegs<kLogN2, kLogE2> tw2(twl, kLogM1, t);
        float2* const buf2[1] = {&fbuf[0][0] + idx * lds_padded_size(kN2)};
        fft_multi<1, kLogN2, kLogE2, false, false, kLogE2, true>(w, buf2, t, tw2);
#pragma unroll
        for (int e = 0; e < kE2; ++e) khl[c][4 * (t + kT2 * e) + q] = w[0][e];
    }
    __syncthreads();

    // B3
    if (zwave) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[0][e] = c_mul(x[0][e], khl[half][t + T * e]);
        fft_multi<1, kLogM1, kLogE1, true, false, 4, true>(x, mine, t, tw);
        if (half) {  // the transform's last exchange is behind it: the buffer is free
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int j = t + T * e;
                fbuf[wv][j] = c_mul(x[0][e], c_conj(twl[j]));
            }
        }
    }
    __syncthreads();
    if (zwave && !half && pact) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = t + T * e;
            if (j < L) {
                float2 o = c_add(x[0][e], fbuf[wv + 1][j]);
                if (chst) o = c_nan();
                // streaming stores: the rows are not read again here, and
                // fewer dirty lines are left for the end-of-kernel write-back
                __builtin_nontemporal_store(o.x, &y[row1 + j]);
                if (has2) __builtin_nontemporal_store(o.y, &y[row2 + j]);
            }
        }
    }
}

}  // namespace

// Bsz = 0: the kernel (and the root values) alone, no spectra and no rows
bool single_launch_fits(int64_t Bsz, int64_t H, int64_t M) {
    return M == kM1 && (Bsz + 1) / 2 <= kPairs1 && H >= 256;
}

hipError_t launch_single(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, const float2* Lambda,
                         const float2* P, const float2* Q, const float2* Bv, const float2* Ct, const float* dt,
                         const float* D, const float* u, float* y, float2* K_out, int32_t* status,
                         hipStream_t stream, float2* roots_out) {
#define SSM_SINGLE(RK)                                                                                        \
    if (r == RK) {                                                                                            \
        hipLaunchKernelGGL((filter_m1024_kernel<RK>), dim3((unsigned)H), dim3(kThreads1), 0, stream, (int)Bsz, \
                           (int)H, (int)N, (int)L, Lambda, P, Q, Bv, Ct, dt, D, u, y, K_out, status, roots_out); \
        return hipGetLastError();                                                                             \
    }
    SSM_SINGLE(1) SSM_SINGLE(2) SSM_SINGLE(3) SSM_SINGLE(4)
#undef SSM_SINGLE
    return hipErrorInvalidValue;
}

}  // namespace ssm
