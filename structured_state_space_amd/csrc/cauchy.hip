// Root values H(z_k) of the S4 filter mode (vector ALU + matrix cores).
//
// Source: "Recurrent, LSTM, and structured state-space models", block for S4
// Algorithm 1 / App. C (filter mode).  For z = z_k = exp(-2 pi i k/M), k != M/2,
//   s(z) = (2/dt)(1-z)/(1+z) = i a tan(pi k/M),   2/(1+z) = 1 + i tan(pi k/M),
// with a = 2/dt, so each denominator s(z_k) - lambda_n = -Re(lambda_n) + i(a t_k -
// Im(lambda_n)).  The (r+1)^2 sums
//   rho_uv(k) = sum_n conj(u_n) v_n / (s(z_k) - lambda_n),  u in {C~, Q_a}, v in {B, P_b}
// are the resolvent products u^* R(z_k) v of the page; then
//   W = I_r + rho_QP,  H = (1 + i t_k) (rho_C~B - rho_C~P W^{-1} rho_QB),
// and z = -1 (k = M/2) takes the page's finite value (dt/2) C~^* B.  This is the
// resolvent expression itself; it equals the page's mu-form Cauchy products
// S_uv(z) = (2/(1+z)) u^* R v term by term, but keeps the denominators' real part
// exactly -Re(lambda_n), which float32 needs when a = 2/dt is large.
//
// Work split: one workgroup per (channel, tile of 256*RPT roots).  Per chunk of
// states the workgroup stages a header (x^2, Im lambda) and the weight block of
// each state in LDS (roots.hpp); every thread then sweeps the chunk for its RPT
// roots: per (root, state) one reciprocal and a multiply on the vector ALU
// (with d = x + i y, x = -Re lambda, y = a t_k - Im lambda: inv = 1/|d|^2 and
// y inv), and the products with the weights on the matrix cores, four real
// columns per 4x4x1 instruction.
// Exact zeros: a zero denominator makes the sums NaN; such roots are re-checked
// with an exact test (-Re lambda == 0 and a t_k - Im lambda == 0 in float32) and
// flagged resonant-diagonal.  A W with an exactly zero pivot (partial pivoting,
// |re|+|im| order) is flagged resonant-correction.
#include <float.h>

#include "common.hpp"
#include "roots.hpp"
#include "wfft.hpp"

namespace ssm {

namespace {

// Per-root tables, once per call: tan(pi k/M) in float64 (0 at k = M/2, which
// takes the finite z = -1 formula) and exp(-i pi k/M) for the later transforms.
__global__ __launch_bounds__(256) void root_tables_kernel(int M, double* __restrict__ tant,
                                                          float2* __restrict__ twtab) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= M) return;
    double sn, cs;
    sincospi((double)k / (double)M, &sn, &cs);
    tant[k] = (2 * k == M) ? 0.0 : sn / cs;
    twtab[k] = make_float2((float)cs, (float)-sn);
}

template <int RK, int RPT>
// rank 1: registers capped for four waves per SIMD (fits without spills;
// measured faster than three waves with more registers)
__global__ __launch_bounds__(kCauchyThreads) __attribute__((amdgpu_waves_per_eu(RK == 1 ? 4 : 1))) void cauchy_roots_kernel(
    int M, int scr_logm, int N, int tiles, const float2* __restrict__ Lambda, const float2* __restrict__ P,
    const float2* __restrict__ Q, const float2* __restrict__ Bv, const float2* __restrict__ Ct,
    const float* __restrict__ dt, float2* __restrict__ roots, int32_t* __restrict__ tile_status,
    const double* __restrict__ tant, float2* __restrict__ twtab) {
    constexpr int F = Fam<RK>::F, kChunk = Fam<RK>::CHUNK, U = sweep_unroll<RK, RPT>();
    // tan(pi k/M) from the per-call table when each thread has several roots;
    // otherwise computed here, and this grid also writes the twiddle table
    constexpr bool TAB = RPT >= 4;
    if constexpr (!TAB)
        for (int j = blockIdx.x * kCauchyThreads + threadIdx.x; j < M; j += gridDim.x * kCauchyThreads) {
            double sn, cs;
            sincospi((double)j / (double)M, &sn, &cs);
            twtab[j] = make_float2((float)cs, (float)-sn);
        }
    __shared__ float2 hdr[kChunk];
    __shared__ float4 wt[kChunk * Fam<RK>::WROW];
    __shared__ int blk_status;
    __shared__ double2 red[kCauchyThreads / 64];

    const int h = blockIdx.x / tiles;
    const int tile = blockIdx.x - h * tiles;
    const int tid = threadIdx.x;
    const size_t hbase = (size_t)h * N;
    const float dtv = dt[h];


    if (!(dtv > 0.0f) || !(dtv <= FLT_MAX)) {  // uniform over the workgroup
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int k = tile * (kCauchyThreads * RPT) + i * kCauchyThreads + tid;
            if (k < M) roots[(size_t)h * M + k] = c_nan();
        }
        if (tid == 0) tile_status[blockIdx.x] = SSM_ST_INVALID_STEP;
        return;
    }
    if (tid == 0) blk_status = 0;

    const double a = 2.0 / (double)dtv;
    float st[RPT], tf[RPT];
    int kk[RPT], kf[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        // the output position; the root it holds is the same index in natural
        // order, or (scr_logm > 0) the frequency of that position in the
        // wave-structured transforms' scrambled order
        const int pos = tile * (kCauchyThreads * RPT) + i * kCauchyThreads + tid;
        const int k = (scr_logm > 0 && pos < M) ? wf_freq_rt(scr_logm, pos) : pos;
        kk[i] = pos;
        kf[i] = k;
        st[i] = 0.0f;
        tf[i] = 0.0f;
        if (k < M) {
            double t;
            if constexpr (TAB) {
                t = tant[k];
            } else {
                double sn, cs;
                sincospi((double)k / (double)M, &sn, &cs);
                t = (2 * k == M) ? 0.0 : sn / cs;
            }
            st[i] = (float)(a * t);
            tf[i] = (float)t;
        }
    }

    RootAcc<RK> acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc_zero<RK>(acc[i]);

    double m1x = 0.0, m1y = 0.0;
    // Small grids (one or two roots per thread) are a single round of
    // workgroups, four per CU.  Issue priority then falls with progress through
    // the states (3 in the first quarter, 0 in the last), so that the
    // workgroups sharing a CU advance together instead of oldest-first, which
    // leaves the last one to finish alone with nothing to hide its latencies.
    constexpr bool FAIR = RPT <= 2;
    const int q1 = N / 4, q2 = N / 2, q3 = (3 * N) / 4;
    if constexpr (FAIR) __builtin_amdgcn_s_setprio(3);
    for (int n0 = 0; n0 < N; n0 += kChunk) {
        const int nch = min(kChunk, N - n0);
        const int npad = (nch + U - 1) / U * U;
        __syncthreads();
        for (int nn = tid; nn < npad; nn += kCauchyThreads) {
            if (nn >= nch) {
                stage_pad<RK>(hdr + nn, wt + nn * Fam<RK>::WROW);
                continue;
            }
            const size_t hn = hbase + n0 + nn;
            const float2 lam = Lambda[hn];
            float2 uu[RK + 1], vv[RK + 1];
            uu[0] = Ct[hn];
            vv[0] = Bv[hn];
            // z = -1 takes (dt/2) C~^* B: partial sums in float64, reduced after the sweep
            m1x += (double)uu[0].x * vv[0].x + (double)uu[0].y * vv[0].y;
            m1y += (double)uu[0].x * vv[0].y - (double)uu[0].y * vv[0].x;
#pragma unroll
            for (int j = 0; j < RK; ++j) {
                uu[1 + j] = Q[hn * RK + j];
                vv[1 + j] = P[hn * RK + j];
            }
            stage_state<RK>(hdr + nn, wt + nn * Fam<RK>::WROW, lam, uu, vv);
        }
        __syncthreads();
        sweep_chunk<RK, RPT, U, FAIR>(hdr, wt, npad, n0, q1, q2, q3, st, acc);
    }

    if constexpr (FAIR) __builtin_amdgcn_s_setprio(0);
    // reduce the z = -1 partial sums when this tile holds k = M/2 (uniform test)
    const int k_lo = tile * (kCauchyThreads * RPT);
    const int pos_m1 = scr_logm > 0 ? 512 : M / 2;  // where the root z = -1 (k = M/2) is stored
    const bool has_m1 = M >= 2 && k_lo <= pos_m1 && pos_m1 < k_lo + kCauchyThreads * RPT;
    double2 m1 = make_double2(0.0, 0.0);
    if (has_m1) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            m1x += __shfl_xor(m1x, o, 64);
            m1y += __shfl_xor(m1y, o, 64);
        }
        if ((tid & 63) == 0) red[tid >> 6] = make_double2(m1x, m1y);
        __syncthreads();
#pragma unroll
        for (int wv = 0; wv < kCauchyThreads / 64; ++wv) {
            m1.x += red[wv].x;
            m1.y += red[wv].y;
        }
    }

    int my_status = 0;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        float2 sums[F];
        acc_unpack<RK>(acc[i], sums);  // every lane, before the range test
        const int pos = kk[i], k = kf[i];
        if (pos >= M) continue;
        const float2 H = 2 * k == M ? make_float2((float)(0.5 * dtv * m1.x), (float)(0.5 * dtv * m1.y))
                                    : finish_root<RK>(sums, st[i], tf[i], N, hbase, Lambda, P, Q, Bv, Ct, my_status);
        roots[(size_t)h * M + pos] = H;
    }
    if (my_status) atomicMax(&blk_status, my_status);
    __syncthreads();
    if (tid == 0) tile_status[blockIdx.x] = blk_status;
}

template <int RK, int RPT>
hipError_t launch_rk(int64_t H, int64_t N, int64_t M, int scr_logm, const float2* Lambda, const float2* P,
                     const float2* Q, const float2* Bv, const float2* Ct, const float* dt, float2* roots,
                     int32_t* tstat, float2* twtab, double* tant, hipStream_t stream) {
    if (RPT >= 4) {
        hipLaunchKernelGGL(root_tables_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, stream, (int)M, tant,
                           twtab);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    const int tiles = (int)((M + kCauchyThreads * RPT - 1) / (kCauchyThreads * RPT));
    const int64_t blocks = H * tiles;
    hipLaunchKernelGGL((cauchy_roots_kernel<RK, RPT>), dim3((unsigned)blocks), dim3(kCauchyThreads), 0, stream,
                       (int)M, scr_logm, (int)N, tiles, Lambda, P, Q, Bv, Ct, dt, roots, tstat, tant, twtab);
    return hipGetLastError();
}

}  // namespace

// roots per thread: up to 4 for r = 1 and 2 for r = 2 (more sums share each
// staged weight row; these were measured fastest, the accumulators of more
// roots crowd out waves), while the grid keeps at least 1024 workgroups
int cauchy_rpt(int64_t H, int64_t r, int64_t M) {
    const int max_rpt = r == 1 ? 4 : r == 2 ? 2 : 1;
    int rpt = max_rpt;
    while (rpt > 1 && H * ((M + (int64_t)kCauchyThreads * rpt - 1) / ((int64_t)kCauchyThreads * rpt)) < 1024)
        rpt >>= 1;
    return rpt;
}

int64_t cauchy_tiles(int64_t H, int64_t r, int64_t M) {
    const int64_t per = (int64_t)kCauchyThreads * cauchy_rpt(H, r, M);
    return (M + per - 1) / per;
}

// scrambled: store the root values in the order the wave-structured
// transforms take them (M >= 1024), not in natural order
hipError_t launch_cauchy(int64_t H, int64_t N, int64_t r, int64_t M, const float2* Lambda, const float2* P,
                         const float2* Q, const float2* Bv, const float2* Ct, const float* dt, float2* roots,
                         int32_t* tile_status, float2* twtab, double* tant, hipStream_t stream, bool scrambled) {
    const int rpt = cauchy_rpt(H, r, M);
    const int scr_logm = scrambled ? ilog2_exact(M) : 0;
    if (scrambled && M < 1024) return hipErrorInvalidValue;
#define SSM_CAUCHY(RK, RPT)                                                                                   \
    if (r == RK && rpt == RPT)                                                                                \
        return launch_rk<RK, RPT>(H, N, M, scr_logm, Lambda, P, Q, Bv, Ct, dt, roots, tile_status, twtab, tant, \
                                  stream);
    SSM_CAUCHY(1, 4) SSM_CAUCHY(1, 2) SSM_CAUCHY(1, 1) SSM_CAUCHY(2, 2) SSM_CAUCHY(2, 1)
    SSM_CAUCHY(3, 1) SSM_CAUCHY(4, 1)
#undef SSM_CAUCHY
    return hipErrorInvalidValue;
}

}  // namespace ssm
