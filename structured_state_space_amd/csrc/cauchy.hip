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
// Two kernels.  The float32 one (rank 1 below 128 states or 4096 roots, rank
// 4): one workgroup per (channel, tile of 256*RPT roots).  Per chunk of states
// the workgroup stages a header (x^2, Im lambda) and the weight block of each
// state in LDS (roots.hpp); every thread then sweeps the chunk for its RPT
// roots: per (root, state) one reciprocal and a multiply on the vector ALU
// (with d = x + i y, x = -Re lambda, y = a t_k - Im lambda: inv = 1/|d|^2 and
// y inv), and the products with the weights on the matrix cores, four real
// columns per 4x4x1 instruction.  The split-precision one (the other shapes):
// a per-channel record kernel, then a sweep on the float16 matrix cores in
// high and low parts, where waves of roots far from the poles sum a moment
// expansion instead of the states (see its section below).
// Exact zeros: a zero denominator makes the sums NaN; such roots are re-checked
// with an exact test (-Re lambda == 0 and a t_k - Im lambda == 0 in float32) and
// flagged resonant-diagonal.  A W with an exactly zero pivot (partial pivoting,
// |re|+|im| order; rank 2 in the split-precision kernel, which solves by
// Cramer's rule: det W exactly zero) is flagged resonant-correction.
#include <float.h>

#include "common.hpp"
#include "roots.hpp"
#include "wfft.hpp"

namespace ssm {

namespace {

// Per-root tables, once per call: tan(pi k/M) in float64 for the root held at
// each output position (0 at k = M/2, which takes the finite z = -1 formula;
// scr_logm > 0: positions in the wave-structured transforms' order, else
// natural order) and exp(-i pi j/M) for the later transforms.
__device__ __forceinline__ void root_tables_at(int j, int M, int scr_logm, double* __restrict__ tant,
                                               float2* __restrict__ twtab) {
    if (j >= M) return;
    double sn, cs;
    sincospi((double)j / (double)M, &sn, &cs);
    twtab[j] = make_float2((float)cs, (float)-sn);
    const int k = scr_logm > 0 ? wf_freq_rt(scr_logm, j) : j;
    if (k != j) sincospi((double)k / (double)M, &sn, &cs);
    tant[j] = (2 * k == M) ? 0.0 : sn / cs;
}
// exp(-i pi j/(2M)), j < 2M: the wave-structured transforms' table
__device__ __forceinline__ void tw4_at(int j, int M, float2* __restrict__ tw4) {
    if (j >= 2 * M) return;
    double sn, cs;
    sincospi((double)j / (double)(2 * M), &sn, &cs);
    tw4[j] = make_float2((float)cs, (float)-sn);
}
// the root tables, then (tw4 given: workgroups from ceil(M/256) on) the
// transforms' table
__global__ __launch_bounds__(256) void root_tables_kernel(int M, int scr_logm, double* __restrict__ tant,
                                                          float2* __restrict__ twtab, float2* __restrict__ tw4) {
    const int ntab = (M + 255) / 256, b = (int)blockIdx.x;
    if (b < ntab)
        root_tables_at(b * 256 + (int)threadIdx.x, M, scr_logm, tant, twtab);
    else
        tw4_at((b - ntab) * 256 + (int)threadIdx.x, M, tw4);
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
    // the first chunk's state inputs are loaded before anything else, so that
    // their latency overlaps the step check and the tangents
    float2 f_lam = make_float2(0.0f, 0.0f), f_uu[RK + 1], f_vv[RK + 1];
    const bool f_has = tid < min(kChunk, N);
    if (f_has) {
        const size_t hn = hbase + tid;
        f_lam = Lambda[hn];
        f_uu[0] = Ct[hn];
        f_vv[0] = Bv[hn];
#pragma unroll
        for (int j = 0; j < RK; ++j) {
            f_uu[1 + j] = Q[hn * RK + j];
            f_vv[1 + j] = P[hn * RK + j];
        }
    }
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
                t = tant[pos];
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
            float2 lam, uu[RK + 1], vv[RK + 1];
            if (n0 == 0 && nn == tid) {  // the prefetched state (nn = tid < nch on the first chunk)
                lam = f_lam;
#pragma unroll
                for (int j = 0; j <= RK; ++j) {
                    uu[j] = f_uu[j];
                    vv[j] = f_vv[j];
                }
            } else {
                lam = Lambda[hn];
                uu[0] = Ct[hn];
                vv[0] = Bv[hn];
#pragma unroll
                for (int j = 0; j < RK; ++j) {
                    uu[1 + j] = Q[hn * RK + j];
                    vv[1 + j] = P[hn * RK + j];
                }
            }
            // z = -1 takes (dt/2) C~^* B: partial sums in float64, reduced after the sweep
            m1x += (double)uu[0].x * vv[0].x + (double)uu[0].y * vv[0].y;
            m1y += (double)uu[0].x * vv[0].y - (double)uu[0].y * vv[0].x;
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

// ---------------------------------------------------------------------------
// Ranks 2 and 3: the sums on the float16 matrix cores in split precision.
// Per root k and state n the Cauchy entry g = 1/d, d = s_k - lambda_n, is
// formed in float32 and scaled by the per-root sigma_k = sqrt(st^2 + X^2 + R^2)
// (st = a t_k, X and R the largest |Re lambda| and |Im lambda| of the channel),
// so that |d_n| <= sqrt(2) sigma_k for every state: every scaled entry has
// |g sigma| >= 1/sqrt(2), a normal float16 value.  Near a resonance |g sigma| may
// pass the float16 range; the conversion then gives an infinity, the sums are
// not finite and the root takes the float32 recheck of the finish.  The weights
// are scaled by the per-family tau_f (largest weight component), so |b| <= 1.
// Both operands are split into float16 high and low parts, a = a_h + a_l (a_h
// the rounding of a, a_l the rounding of the remainder a - a_h), and each
// product is taken as a_h b_h + a_h b_l + a_l b_h with float32 accumulation:
// three v_mfma_f32_32x32x16_f16 per block of 8 states and 32 roots.  The
// dropped a_l b_l and the roundings of the low parts leave about 2^-21 of each
// product.
// Layout of one instruction: A is the weights, 32 columns x 16 (column 2 f + p:
// the real and imaginary parts p of family f; k = 2 s + c for the 8 states s of
// the block and the components c of g = gx + i gy), B the Cauchy entries, 16 x
// 32 roots, and C is 32 columns x 32 roots.  Lane l holds row l % 32 and k =
// 8 (l / 32) + 0..7 of A (column l % 32's weights of four states), column l % 32
// and the same k of B (root l % 32's entries of those states, both
// components), and rows 8 (v / 4) + 4 (l / 32) + v % 4 of C's column l % 32.
// Re(w g) = w.x gx - w.y gy and Im(w g) = w.y gx + w.x gy give the weight
// entries (gx, gy): column 2f: (w.x, -w.y), column 2f + 1: (w.y, w.x).
//
// The per-channel part (the scales, the split weight blocks in the order the
// sweep reads them, the state headers and the z = -1 sum) is formed once per
// channel by a small kernel and copied to LDS by each root workgroup.
// ---------------------------------------------------------------------------
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef float f16v __attribute__((ext_vector_type(16)));
constexpr int kHChunk = 64;  // states staged in LDS at a time (8 blocks of 8)
constexpr int kHBlockBytes = 2048;  // one block of 8 states: [lane half][hi, lo][32 columns] x 16 bytes

// Far roots.  Around the centre c of the channel's poles (their mean) with
// radius R = max |lambda_n - c|, a root with |s - c| > R has
//   rho_f(s) = (1/R) sum_{j >= 0} Mt_{j,f} v^(j+1),  v = R/(s - c),  |v| < 1,
//   Mt_{j,f} = sum_n w_{f,n} ((lambda_n - c)/R)^j,
// the expansion of each 1/(s - lambda_n) in powers of (lambda_n - c)/(s - c).
// The sums are then the same product as over the states, with pseudo-states j:
// moments in place of weights and the powers v^(j+1) in place of the Cauchy
// entries.  A wave keeps J = 8 nfb terms (nfb = 1..5 blocks), the fewest with
// |v|^J <= 2^-24 for all its roots (|v| <= 2^(-3/nfb): 1/8 to 0.66, i.e.
// |s - c| >= kFarRatio[nfb - 1] R): the dropped tail is below
// 2^-24 (1 + |v|)/(1 - |v|) <= 5 2^-24 of the sum of |terms|.
constexpr int kFarJ = 40;  // terms at most (5 blocks of 8)
constexpr float kFarRatio[kFarJ / 8] = {8.0f, 2.8284271f, 2.0f, 1.6817928f, 1.5157166f};  // 2^(3/nfb)

// One channel's record: the weight blocks (npad / 8 x 2048 bytes), the
// headers x = -Re lambda, x^2, Im lambda (npad floats each; padding states
// x = 0, x^2 = 1), the moment blocks of the far roots (kFarJ / 8 x 2048 bytes),
// then 256 bytes of scales: tau_f (16 floats), X^2 + R^2 and the z = -1 sum
// C~^* B (float64), and at 96 the moments' tau_f (16 floats), c (2 floats),
// R and 1/R (floats); R = 0 (a single pole position, or non-finite poles)
// turns the far form off.
struct HRec {
    int64_t npad, hdr, far, scal, bytes;
    __host__ __device__ explicit HRec(int64_t N) {
        npad = (N + 7) & ~(int64_t)7;
        hdr = npad / 8 * kHBlockBytes;
        far = hdr + 3 * npad * 4;
        scal = far + kFarJ / 8 * kHBlockBytes;
        bytes = scal + 256;
    }
};

// (a, b) as float16 high and low parts: hi the rounding, lo the rounding of the
// float32 remainder.  Each remainder is one v_fma_mix_f32, -hi * 1 + a with the
// float16 half converted inside the instruction: the same value as converting
// and subtracting (the product is exact, one rounding), one instruction instead
// of two.  (Where a is itself a product the compiler fuses that product into a
// mixed FMA on its own; the far form's powers are not products at this point.)
__device__ __forceinline__ void split_pair(float a, float b, h2& hi, h2& lo) {
    const f2v v = {a, b};
    hi = __builtin_convertvector(v, h2);
    const unsigned hb = __builtin_bit_cast(unsigned, hi);
    float ra, rb;
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(hb), "v"(a));
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(hb), "v"(b));
    const f2v r = {ra, rb};
    lo = __builtin_convertvector(r, h2);
}

__device__ __forceinline__ double2 c_mul_d(double2 a, double2 b) {
    return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

template <int RK>
// Workgroups H.. of the same grid write the per-call root tables, and after
// them (tw4 given) the wave-structured transforms' table
// tw4[j] = exp(-i pi j/(2M)), j < 2M.
__global__ __launch_bounds__(256) void cauchy_h_prep_kernel(int H, int N, const float2* __restrict__ Lambda,
                                                            const float2* __restrict__ P, const float2* __restrict__ Q,
                                                            const float2* __restrict__ Bv,
                                                            const float2* __restrict__ Ct, char* __restrict__ prep,
                                                            int M, int scr_logm, double* __restrict__ tant,
                                                            float2* __restrict__ twtab, float2* __restrict__ tw4) {
    if ((int)blockIdx.x >= H) {  // uniform over the workgroup
        const int b = (int)blockIdx.x - H, ntab = (M + 255) / 256;
        if (b < ntab) {
            root_tables_at(b * 256 + (int)threadIdx.x, M, scr_logm, tant, twtab);
        } else {
            const int j = (b - ntab) * 256 + (int)threadIdx.x;
            tw4_at(j, M, tw4);
        }
        return;
    }
    constexpr int F = Fam<RK>::F;
    const HRec rec(N);
    const int h = blockIdx.x, tid = threadIdx.x;
    const size_t hbase = (size_t)h * N;
    char* const out = prep + (size_t)h * rec.bytes;
    float* const hx = reinterpret_cast<float*>(out + rec.hdr);
    const int npad = (int)rec.npad;
    const bool one = npad <= 256;  // one chunk: the vectors loaded for the scales stay in LDS
    __shared__ unsigned int mx_bits[F + 2];  // tau_f, X^2, R^2 (non-negative floats order as integers)
    __shared__ double2 red[4];
    __shared__ float2 sl[256], sc[256], sb[256], sp[256 * RK], sq[256 * RK];
    if (tid < F + 2) mx_bits[tid] = 0u;

    // one chunk of 256 states: this thread's state, the vectors zero past N
    // (its headers: x = 0, x^2 = 1 there), staged in LDS
    auto stage = [&](int n0) {
        const int n = n0 + tid;
        float2 lam = make_float2(0.0f, 0.0f), c = lam, b = lam;
        float2 pv[RK], qv[RK];
#pragma unroll
        for (int j = 0; j < RK; ++j) pv[j] = qv[j] = lam;
        if (n < N) {
            const size_t hn = hbase + n;
            lam = Lambda[hn];
            c = Ct[hn];
            b = Bv[hn];
#pragma unroll
            for (int j = 0; j < RK; ++j) {
                pv[j] = P[hn * RK + j];
                qv[j] = Q[hn * RK + j];
            }
        }
        if (n < npad) {
            sl[tid] = lam;
            sc[tid] = c;
            sb[tid] = b;
#pragma unroll
            for (int j = 0; j < RK; ++j) {
                sp[tid * RK + j] = pv[j];
                sq[tid * RK + j] = qv[j];
            }
            hx[n] = -lam.x;
            hx[npad + n] = n < N ? lam.x * lam.x : 1.0f;
            hx[2 * npad + n] = lam.y;
        }
    };

    // the scales (largest weight component per family, X^2, R^2) and the
    // z = -1 sum (dt/2) C~^* B in float64
    double m1x = 0.0, m1y = 0.0, lsx = 0.0, lsy = 0.0;
    __shared__ double2 lsum[4];
    {
        float tl[F + 2];
#pragma unroll
        for (int f = 0; f < F + 2; ++f) tl[f] = 0.0f;
        if (one) {
            stage(0);
            __syncthreads();
        }
        for (int n = tid; n < N; n += 256) {
            float2 lam, uu[RK + 1], vv[RK + 1];
            if (one) {
                lam = sl[n];
                uu[0] = sc[n];
                vv[0] = sb[n];
#pragma unroll
                for (int j = 0; j < RK; ++j) {
                    uu[1 + j] = sq[n * RK + j];
                    vv[1 + j] = sp[n * RK + j];
                }
            } else {
                const size_t hn = hbase + n;
                lam = Lambda[hn];
                uu[0] = Ct[hn];
                vv[0] = Bv[hn];
#pragma unroll
                for (int j = 0; j < RK; ++j) {
                    uu[1 + j] = Q[hn * RK + j];
                    vv[1 + j] = P[hn * RK + j];
                }
            }
            tl[F] = fmaxf(tl[F], lam.x * lam.x);
            tl[F + 1] = fmaxf(tl[F + 1], lam.y * lam.y);
            lsx += lam.x;
            lsy += lam.y;
            m1x += (double)uu[0].x * vv[0].x + (double)uu[0].y * vv[0].y;
            m1y += (double)uu[0].x * vv[0].y - (double)uu[0].y * vv[0].x;
#pragma unroll
            for (int iu = 0; iu <= RK; ++iu)
#pragma unroll
                for (int iv = 0; iv <= RK; ++iv) {
                    const float2 w = c_mul(c_conj(uu[iu]), vv[iv]);
                    const int f = iu * (RK + 1) + iv;
                    tl[f] = fmaxf(tl[f], fmaxf(fabsf(w.x), fabsf(w.y)));
                }
        }
        // wave reductions by shuffles, then one LDS atomic per wave and value
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
            for (int f = 0; f < F + 2; ++f) tl[f] = fmaxf(tl[f], __shfl_xor(tl[f], o, 64));
            m1x += __shfl_xor(m1x, o, 64);
            m1y += __shfl_xor(m1y, o, 64);
            lsx += __shfl_xor(lsx, o, 64);
            lsy += __shfl_xor(lsy, o, 64);
        }
        if ((tid & 63) == 0) {
#pragma unroll
            for (int f = 0; f < F + 2; ++f)
                if (tl[f] > 0.0f) atomicMax(&mx_bits[f], __float_as_uint(tl[f]));
            red[tid >> 6] = make_double2(m1x, m1y);
            lsum[tid >> 6] = make_double2(lsx, lsy);
        }
    }
    __syncthreads();
    if (tid < 16) {
        reinterpret_cast<float*>(out + rec.scal)[tid] = tid < F ? __uint_as_float(mx_bits[tid]) : 0.0f;
    } else if (tid == 16) {
        double* const sd = reinterpret_cast<double*>(out + rec.scal + 64);
        sd[0] = (double)__uint_as_float(mx_bits[F]) + (double)__uint_as_float(mx_bits[F + 1]);
        sd[1] = red[0].x + red[1].x + red[2].x + red[3].x;
        sd[2] = red[0].y + red[1].y + red[2].y + red[3].y;
    }
    // the weight blocks, per chunk of 256 states: one 16-byte group (block,
    // lane half, column) per item, hi and lo
    for (int n0 = 0; n0 < npad; n0 += 256) {
        const int nch = min(256, npad - n0);
        if (!one) {
            __syncthreads();  // the previous chunk's readers are done
            stage(n0);
            __syncthreads();
        }
        const int items = nch / 8 * 64;
        for (int it = tid; it < items; it += 256) {
            const int kbl = it >> 6, lh = (it >> 5) & 1, col = it & 31, f = col >> 1;
            const int iu = f / (RK + 1), iv = f - iu * (RK + 1);
            float itau = 0.0f;
            if (f < F) {
                const float t = __uint_as_float(mx_bits[f]);
                itau = t > 0.0f ? 1.0f / t : 0.0f;
            }
            h8 hi8, lo8;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = 8 * kbl + 4 * lh + q;
                float2 w = make_float2(0.0f, 0.0f);
                if (f < F) {
                    const float2 u = iu == 0 ? sc[nl] : sq[nl * RK + iu - 1];
                    const float2 v = iv == 0 ? sb[nl] : sp[nl * RK + iv - 1];
                    w = c_mul(c_conj(u), v);  // zero for padding states
                }
                const float wx = w.x * itau, wy = w.y * itau;
                h2 hi, lo;
                if (col & 1)
                    split_pair(wy, wx, hi, lo);  // column 2f + 1: (w.y, w.x)
                else
                    split_pair(wx, -wy, hi, lo);  // column 2f: (w.x, -w.y)
                hi8[2 * q] = hi[0];
                hi8[2 * q + 1] = hi[1];
                lo8[2 * q] = lo[0];
                lo8[2 * q + 1] = lo[1];
            }
            h8* const dst =
                reinterpret_cast<h8*>(out + (size_t)(n0 / 8 + kbl) * kHBlockBytes + lh * 1024 + col * 16);
            dst[0] = hi8;
            dst[32] = lo8;
        }
    }
    // ---- far roots: the poles' centre c and radius R (float64), the moments
    //      Mt_{j,f}, their scales, and the moment blocks ----
    __shared__ double rmax[4];
    // states per sub-chunk of the moment sums: 32 at ranks 2 and 3 keeps the
    // kernel's LDS at 30 and 38 KB (five and four workgroups per CU); rank 1
    // fits 64 (34 KB), half the sub-chunk barriers for its longer state vectors
    constexpr int kSub = RK == 1 ? 64 : 32;
    __shared__ float2 qp[kSub][kFarJ];  // powers ((lambda_n - c)/R)^j of kSub states (formed in float64)
    __shared__ float2 mt[kFarJ * F];
    __shared__ float2 wsub[kSub * F];   // the weights of kSub states
    __shared__ float tauf[F];
    const double cx = (lsum[0].x + lsum[1].x + lsum[2].x + lsum[3].x) / (double)N;
    const double cy = (lsum[0].y + lsum[1].y + lsum[2].y + lsum[3].y) / (double)N;
    auto lam_at = [&](int n) -> float2 {  // state n of the staged chunk n0 (one) or from HBM
        return one ? sl[n] : Lambda[hbase + n];
    };
    {
        double r2 = 0.0;
        for (int n = tid; n < N; n += 256) {
            const float2 lam = lam_at(n);
            const double dx = (double)lam.x - cx, dy = (double)lam.y - cy;
            r2 = fmax(r2, dx * dx + dy * dy);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) r2 = fmax(r2, __shfl_xor(r2, o, 64));
        if ((tid & 63) == 0) rmax[tid >> 6] = r2;
    }
    __syncthreads();
    const double R2 = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
    double R = sqrt(R2);
    if (!(R >= 1e-30) || !(R <= 1e30)) R = 0.0;  // a single pole position or non-finite poles: no far form
    const double iR = R > 0.0 ? 1.0 / R : 0.0;
    constexpr int NM = kFarJ * F;  // moments, (j, f) = (i / F, i % F), three per thread at most
    constexpr int NMT = (NM + 255) / 256;
    static_assert(NMT <= 3, "three moments per thread");
    // The sums in float32: the moment blocks keep about 22 bits (float16 high
    // and low parts), which a 64-term float32 sum of these products matches.
    float2 macc[NMT];
#pragma unroll
    for (int i2 = 0; i2 < NMT; ++i2) macc[i2] = make_float2(0.0f, 0.0f);
    for (int n0 = 0; n0 < N; n0 += 256) {
        const int nch = min(256, N - n0);
        if (!one) {
            __syncthreads();  // the previous chunk's readers are done
            stage(n0);
        }
        for (int sub = 0; sub < nch; sub += kSub) {
            __syncthreads();  // staged states visible; the previous sub-chunk's powers and weights are read
            const int nsub = min(kSub, nch - sub);
            if (tid < 4 * kSub) {   // 4 threads per state, each 10 consecutive powers from q^(10 k)
                static_assert(kFarJ == 40, "4 x 10 powers");
                const int m = tid >> 2, k = tid & 3;
                double2 q = make_double2(0.0, 0.0), pw = make_double2(0.0, 0.0);
                if (m < nsub) {
                    const float2 lam = sl[sub + m];
                    q = make_double2(((double)lam.x - cx) * iR, ((double)lam.y - cy) * iR);
                    pw = make_double2(1.0, 0.0);
                    // q^(10 k) = (q^10)^k, q^10 = ((q^2)^2 q)^2
                    const double2 q2 = c_mul_d(q, q), q5 = c_mul_d(c_mul_d(q2, q2), q), q10 = c_mul_d(q5, q5);
                    for (int i = 0; i < k; ++i) pw = c_mul_d(pw, q10);
                }
#pragma unroll
                for (int j = 0; j < 10; ++j) {
                    qp[m][10 * k + j] = make_float2((float)pw.x, (float)pw.y);
                    pw = c_mul_d(pw, q);
                }
            }
            // the weights of the sub-chunk's states (zero past it)
            for (int i = tid; i < kSub * F; i += 256) {
                const int m = i / F, f = i - m * F;
                const int iu = f / (RK + 1), iv = f - iu * (RK + 1);
                float2 w = make_float2(0.0f, 0.0f);
                if (m < nsub) {
                    const int ml = sub + m;
                    const float2 uu = iu == 0 ? sc[ml] : sq[ml * RK + iu - 1];
                    const float2 vv = iv == 0 ? sb[ml] : sp[ml * RK + iv - 1];
                    w = c_mul(c_conj(uu), vv);
                }
                wsub[i] = w;
            }
            __syncthreads();
#pragma unroll
            for (int i2 = 0; i2 < NMT; ++i2) {
                const int idx = tid + 256 * i2;
                if (idx >= NM) continue;
                const int j = idx / F, f = idx - j * F;
                // two partial sums (even and odd states) to halve the FMA chain
                float2 a = macc[i2], b = make_float2(0.0f, 0.0f);
#pragma unroll 4
                for (int m = 0; m < kSub; m += 2) {
                    const float2 w0 = wsub[m * F + f], w1 = wsub[(m + 1) * F + f];
                    const float2 q0 = qp[m][j], q1 = qp[m + 1][j];
                    a.x = fmaf(w0.x, q0.x, fmaf(-w0.y, q0.y, a.x));
                    a.y = fmaf(w0.x, q0.y, fmaf(w0.y, q0.x, a.y));
                    b.x = fmaf(w1.x, q1.x, fmaf(-w1.y, q1.y, b.x));
                    b.y = fmaf(w1.x, q1.y, fmaf(w1.y, q1.x, b.y));
                }
                macc[i2] = make_float2(a.x + b.x, a.y + b.y);
            }
        }
    }
#pragma unroll
    for (int i2 = 0; i2 < NMT; ++i2)
        if (tid + 256 * i2 < NM) mt[tid + 256 * i2] = macc[i2];
    __syncthreads();
    // tau'_f: 8 threads per family (consecutive lanes) take every 8th moment,
    // then a shuffle maximum over the 8
    static_assert(8 * F <= 256 && kFarJ % 8 == 0, "8 threads per family");
    if (tid < 8 * F) {
        const int f = tid >> 3, g = tid & 7;
        float tm = 0.0f;
#pragma unroll
        for (int j = g; j < kFarJ; j += 8) {
            const float2 m = mt[j * F + f];
            tm = fmaxf(tm, fmaxf(fabsf(m.x), fabsf(m.y)));
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) tm = fmaxf(tm, __shfl_xor(tm, o, 64));
        if (g == 0) tauf[f] = tm;
    }
    __syncthreads();
    if (tid < 16) {
        reinterpret_cast<float*>(out + rec.scal + 96)[tid] = tid < F ? tauf[tid] : 0.0f;
    } else if (tid == 16) {
        float* const sf = reinterpret_cast<float*>(out + rec.scal + 160);
        sf[0] = (float)cx;
        sf[1] = (float)cy;
        sf[2] = (float)R;
        sf[3] = (float)iR;
    }
    // moment blocks: the same layout as the weight blocks, pseudo-state j in place of the state
    for (int it = tid; it < kFarJ / 8 * 64; it += 256) {
        const int kb = it >> 6, lh = (it >> 5) & 1, col = it & 31, f = col >> 1;
        float it_f = 0.0f;
        if (f < F) it_f = tauf[f] > 0.0f ? 1.0f / tauf[f] : 0.0f;
        h8 hi8, lo8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = 8 * kb + 4 * lh + q;
            float2 m = make_float2(0.0f, 0.0f);
            if (f < F) {
                const float2 md = mt[j * F + f];
                m = make_float2(md.x * it_f, md.y * it_f);
            }
            h2 hi, lo;
            if (col & 1)
                split_pair(m.y, m.x, hi, lo);  // column 2f + 1: (m.y, m.x)
            else
                split_pair(m.x, -m.y, hi, lo);  // column 2f: (m.x, -m.y)
            hi8[2 * q] = hi[0];
            hi8[2 * q + 1] = hi[1];
            lo8[2 * q] = lo[0];
            lo8[2 * q + 1] = lo[1];
        }
        h8* const dst = reinterpret_cast<h8*>(out + rec.far + (size_t)kb * kHBlockBytes + lh * 1024 + col * 16);
        dst[0] = hi8;
        dst[32] = lo8;
    }
}

// Rank 2 finish by Cramer's rule: with W = I + rho_QP (2 x 2) and
// v = adj(W) rho_QB, H = (1 + i t)(rho_C~B det W - rho_C~P v) / det W.  The
// families are f = 3 iu + iv (iu: C~, Q_1, Q_2; iv: B, P_1, P_2).  A non-finite
// sum takes the same exact re-check as the general finish; det W exactly zero
// is resonant-correction.
__device__ __forceinline__ float2 finish_root_r2(float2 (&acc)[9], float st, float tf, int N, size_t hbase,
                                                 const float2* Lambda, const float2* P, const float2* Q,
                                                 const float2* Bv, const float2* Ct, int& status) {
    bool finite = true;
#pragma unroll
    for (int f = 0; f < 9; ++f) finite = finite && isfinite(acc[f].x) && isfinite(acc[f].y);
    if (!finite && !root_recheck<2>(N, hbase, st, Lambda, P, Q, Bv, Ct, acc)) {
        status = max(status, SSM_ST_RESONANT_DIAGONAL);
        return c_nan();
    }
    const float2 w00 = make_float2(acc[4].x + 1.0f, acc[4].y), w01 = acc[5], w10 = acc[7];
    const float2 w11 = make_float2(acc[8].x + 1.0f, acc[8].y);
    const float2 det = c_sub(c_mul(w00, w11), c_mul(w01, w10));
    if (det.x == 0.0f && det.y == 0.0f) {
        status = max(status, SSM_ST_RESONANT_CORRECTION);
        return c_nan();
    }
    const float2 r0 = acc[3], r1 = acc[6];
    const float2 v0 = c_sub(c_mul(w11, r0), c_mul(w01, r1));
    const float2 v1 = c_sub(c_mul(w00, r1), c_mul(w10, r0));
    const float2 num = c_sub(c_mul(acc[0], det), c_add(c_mul(acc[1], v0), c_mul(acc[2], v1)));
    return c_mul(make_float2(1.0f, tf), cdivf(num, det));
}

// Whether the root s = i st is far from the poles' disc (|s - c| >= rf2 > 0,
// false when R = 0), with |s - c| = mx |e|: mx = max(|Re|, |Im|) of s - c and
// e = conj(s - c)/mx, |e| = ne in [1, sqrt 2] (no overflow in the square).
struct FarRoot {
    float ex, ey, ne, mx;
    bool far;
};
__device__ __forceinline__ FarRoot far_root(float st, float cx, float cy, float rf2) {
    FarRoot r;
    const float sy = st - cy;
    r.mx = fmaxf(fabsf(cx), fabsf(sy));
    const bool big = r.mx >= 0.5f * rf2 && r.mx <= FLT_MAX;
    const float im = big ? __builtin_amdgcn_rcpf(r.mx) : 0.0f;
    r.ex = -cx * im;
    r.ey = -sy * im;
    r.ne = __builtin_amdgcn_sqrtf(fmaf(r.ex, r.ex, r.ey * r.ey));  // in [1, 2]: the hardware square root
    const float d = r.mx * r.ne;
    r.far = big && d >= rf2 && d <= FLT_MAX;
    return r;
}

// Copy states [n0, n0 + 8 nkb) of a channel's record to LDS: the weight blocks
// (all loads issued before the stores) and the three header rows.
__device__ __forceinline__ void h_stage(char* smem, float* hx, const char* rp, int npad, int hdr, int n0, int nkb,
                                        int tid) {
    static_assert(kHChunk / 8 * (kHBlockBytes / 16) == 4 * kCauchyThreads, "four float4 per thread in a full chunk");
    const float4* const src = reinterpret_cast<const float4*>(rp + (size_t)(n0 / 8) * kHBlockBytes);
    float4* const dst = reinterpret_cast<float4*>(smem);
    const int total = nkb * (kHBlockBytes / 16);
    if (total == 4 * kCauchyThreads) {
        const float4 v0 = src[tid], v1 = src[tid + kCauchyThreads], v2 = src[tid + 2 * kCauchyThreads],
                     v3 = src[tid + 3 * kCauchyThreads];
        dst[tid] = v0;
        dst[tid + kCauchyThreads] = v1;
        dst[tid + 2 * kCauchyThreads] = v2;
        dst[tid + 3 * kCauchyThreads] = v3;
    } else {
        for (int i = tid; i < total; i += kCauchyThreads) dst[i] = src[i];
    }
    static_assert(3 * kHChunk <= kCauchyThreads, "one header value per thread");
    const int c = tid / kHChunk, n = tid % kHChunk;
    if (c < 3 && n < 8 * nkb) hx[c * kHChunk + n] = reinterpret_cast<const float*>(rp + hdr)[c * npad + n0 + n];
}

template <int RK, int RPT>
__global__ __launch_bounds__(kCauchyThreads) __attribute__((amdgpu_waves_per_eu(3))) void cauchy_h_kernel(
    int M, int pos_m1, int N, int tiles, int tpw, int xcd_remap, const float2* __restrict__ Lambda,
    const float2* __restrict__ P,
    const float2* __restrict__ Q, const float2* __restrict__ Bv, const float2* __restrict__ Ct,
    const float* __restrict__ dt, const char* __restrict__ prep, const double* __restrict__ tant,
    float2* __restrict__ roots, int32_t* __restrict__ tile_status) {
    constexpr int F = Fam<RK>::F, NC = 2 * F;
    static_assert(NC <= 32, "one block of 32 columns");
    constexpr int NB = 2 * RPT;  // blocks of 32 roots per wave
    constexpr int TILE = kCauchyThreads * RPT;
    // the staged chunk (weight blocks, then the headers), and each wave's C
    // block with a row per root
    __shared__ __align__(16) char smem[kHChunk / 8 * kHBlockBytes + 3 * kHChunk * 4];
    __shared__ __align__(16) char fsm[kFarJ / 8 * kHBlockBytes];  // the moment blocks
    __shared__ int blk_status;
    __shared__ int wnear[kCauchyThreads / 64];  // per wave: some root of this tile is near
    float* const hx = reinterpret_cast<float*>(smem + kHChunk / 8 * kHBlockBytes);  // x = -Re lambda
    float* const hx2 = hx + kHChunk;                                               // x^2
    float* const him = hx2 + kHChunk;                                              // Im lambda

    // this workgroup: tiles [t0, t1) of channel h (tpw tiles per workgroup)
    const int wpc = (tiles + tpw - 1) / tpw;
    int blk = blockIdx.x;
    if (xcd_remap) {  // the workgroups of one channel on one XCD (dispatch is round-robin over 8), so
                      // its record is fetched into one L2
        const int x = blk & 7, s = blk >> 3;
        blk = ((s / wpc) * 8 + x) * wpc + s % wpc;
    }
    const int h = blk / wpc;
    const int t0 = (blk - h * wpc) * tpw, t1 = min(t0 + tpw, tiles);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lh = lane >> 5, row = lane & 31;
    const size_t hbase = (size_t)h * N;
    const float dtv = dt[h];
    if (!(dtv > 0.0f) || !(dtv <= FLT_MAX)) {  // uniform over the workgroup
        for (int i = t0 * TILE + tid; i < t1 * TILE; i += kCauchyThreads)
            if (i < M) roots[(size_t)h * M + i] = c_nan();
        if (tid < t1 - t0) tile_status[(size_t)h * tiles + t0 + tid] = SSM_ST_INVALID_STEP;
        return;
    }
    const HRec rec(N);
    const char* const rp = prep + (size_t)h * rec.bytes;
    const float xr2 = (float)*reinterpret_cast<const double*>(rp + rec.scal + 64);
    const double a = 2.0 / (double)dtv;
    const bool one_chunk = N <= kHChunk;
    if (one_chunk) h_stage(smem, hx, rp, (int)rec.npad, (int)rec.hdr, 0, (N + 7) >> 3, tid);
    {
        const float4* const src = reinterpret_cast<const float4*>(rp + rec.far);
        for (int i = tid; i < kFarJ / 8 * kHBlockBytes / 16; i += kCauchyThreads)
            reinterpret_cast<float4*>(fsm)[i] = src[i];
    }
    if (tid == 0) blk_status = 0;
    __syncthreads();
    const float* const tau = reinterpret_cast<const float*>(rp + rec.scal);  // uniform loads at the finish
    const float* const tau_far = reinterpret_cast<const float*>(rp + rec.scal + 96);
    const float* const fc = reinterpret_cast<const float*>(rp + rec.scal + 160);
    const float cx = fc[0], cy = fc[1], rf = fc[2];
    const float rf2 = rf > 0.0f ? kFarRatio[kFarJ / 8 - 1] * rf : FLT_MAX * 2.0f;  // far: |v| <= 2^(-3/5)

    // One chunk of states: staged once, and the waves then run their tiles
    // without barriers (a wave of far roots goes on to its next tile while the
    // others sweep the states).  Several chunks: the workgroup stages each in
    // turn, and skips them when all its waves are far.
    int my_status = 0;
    for (int tile = t0; tile < t1; ++tile) {
        // this lane's roots: row l % 32 of the wave's NB blocks (vectors, not
        // arrays: the finish selects an element per lane half)
        typedef float fnb __attribute__((ext_vector_type(NB)));
        fnb st, sig, tf;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int pos = tile * TILE + wv * (32 * NB) + nb * 32 + row;
            const double t = pos < M ? tant[pos] : 0.0;
            st[nb] = (float)(a * t);
            tf[nb] = (float)t;
            // any sigma of the right size serves (the same value scales and
            // unscales); the floor keeps the hardware square root off subnormals
            sig[nb] = __builtin_amdgcn_sqrtf(fmaxf(fmaf(st[nb], st[nb], xr2), 1e-30f));
        }
        // the far form for the wave when every root it stores is far (the
        // roots past M and the z = -1 root, which has its own formula, do not vote)
        // and the terms it keeps: 8 nfb with |v|^(8 nfb) <= 2^-24 for all its roots
        bool lane_far = true;
        bool lane_more[kFarJ / 8 - 1] = {};  // some root needs more than 8 (j + 1) terms
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int pos = tile * TILE + wv * (32 * NB) + nb * 32 + row;
            const FarRoot fr = far_root(st[nb], cx, cy, rf2);
            const bool skip = pos >= M || pos == pos_m1;
            lane_far = lane_far && (fr.far || skip);
            const float d = fr.mx * fr.ne;  // |s - c|
#pragma unroll
            for (int j = 0; j < kFarJ / 8 - 1; ++j) lane_more[j] = lane_more[j] || (!skip && !(d >= kFarRatio[j] * rf));
        }
        const bool far = __builtin_amdgcn_ballot_w64(!lane_far) == 0;  // uniform over the wave
        int nfb = 1;
#pragma unroll
        for (int j = 0; j < kFarJ / 8 - 1; ++j) nfb += __builtin_amdgcn_ballot_w64(lane_more[j]) != 0 ? 1 : 0;
        bool any_near = true;
        if (!one_chunk) {
            if (lane == 0) wnear[wv] = far ? 0 : 1;
            __syncthreads();  // also: the previous tile's readers of the staged chunks are done
            any_near = false;
#pragma unroll
            for (int w = 0; w < kCauchyThreads / 64; ++w) any_near = any_near || wnear[w] != 0;
        }

        f16v acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[nb][v] = 0.0f;

        for (int n0 = 0; any_near && n0 < N; n0 += kHChunk) {
            const int nkb = (min(kHChunk, N - n0) + 7) >> 3;
            if (!one_chunk) {
                if (n0 > 0) __syncthreads();  // the previous chunk's readers are done
                h_stage(smem, hx, rp, (int)rec.npad, (int)rec.hdr, n0, nkb, tid);
                __syncthreads();
            }
            if (far) continue;
            const h8* const bsh = reinterpret_cast<const h8*>(smem) + lh * 64 + row;
            for (int kb = 0; kb < nkb; ++kb) {
                const float4 x4 = *reinterpret_cast<const float4*>(&hx[8 * kb + 4 * lh]);
                const float4 q4 = *reinterpret_cast<const float4*>(&hx2[8 * kb + 4 * lh]);
                const float4 i4 = *reinterpret_cast<const float4*>(&him[8 * kb + 4 * lh]);
                const h8 bh = bsh[kb * 128];
                const h8 bl = bsh[kb * 128 + 32];
                const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
                const float x2s[4] = {q4.x, q4.y, q4.z, q4.w};
                const float ims[4] = {i4.x, i4.y, i4.z, i4.w};
                h8 ah[NB], al[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float y = st[nb] - ims[q];
                        const float inv = __builtin_amdgcn_rcpf(fmaf(y, y, x2s[q])) * sig[nb];
                        h2 hi, lo;
                        split_pair(xs[q] * inv, -y * inv, hi, lo);
                        ah[nb][2 * q] = hi[0];
                        ah[nb][2 * q + 1] = hi[1];
                        al[nb][2 * q] = lo[0];
                        al[nb][2 * q + 1] = lo[1];
                    }
                // independent accumulators back to back
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bh, ah[nb], acc[nb], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bl, ah[nb], acc[nb], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bh, al[nb], acc[nb], 0, 0, 0);
            }
        }
        if (far) {
            // Cauchy-side entries u v^j, u = v/|v| = conj(s - c)/|s - c|, for
            // j = 8 kb + 4 (l / 32) + 0..3: the sums are the products with the
            // moment blocks times tau'_f/|s - c|
            f2v vv[NB], pw[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                // roots that are not far (past M, z = -1) take zero entries
                const FarRoot fr = far_root(st[nb], cx, cy, rf2);
                const bool ok = fr.far;
                const float dst = fr.mx * fr.ne;
                const float sc = ok ? __builtin_amdgcn_rcpf(fr.ne) : 0.0f;
                const f2v u = {fr.ex * sc, fr.ey * sc};  // conj(s - c)/|s - c|
                vv[nb] = u * (ok ? rf * __builtin_amdgcn_rcpf(dst) : 0.0f);
                sig[nb] = ok ? dst : 1.0f;  // |s - c|
                pw[nb] = u;
            }
            f2v v4[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const f2v v2 = {vv[nb].x * vv[nb].x - vv[nb].y * vv[nb].y, 2.0f * vv[nb].x * vv[nb].y};
                v4[nb] = (f2v){v2.x * v2.x - v2.y * v2.y, 2.0f * v2.x * v2.y};
                if (lh) pw[nb] = (f2v){pw[nb].x * v4[nb].x - pw[nb].y * v4[nb].y,
                                       pw[nb].x * v4[nb].y + pw[nb].y * v4[nb].x};
            }
            const h8* const fsh = reinterpret_cast<const h8*>(fsm) + lh * 64 + row;
#pragma unroll
            for (int kb = 0; kb < nfb; ++kb) {
                const h8 bh = fsh[kb * 128];
                const h8 bl = fsh[kb * 128 + 32];
                h8 ah[NB], al[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h2 hi, lo;
                        split_pair(pw[nb].x, pw[nb].y, hi, lo);
                        ah[nb][2 * q] = hi[0];
                        ah[nb][2 * q + 1] = hi[1];
                        al[nb][2 * q] = lo[0];
                        al[nb][2 * q + 1] = lo[1];
                        pw[nb] = (f2v){pw[nb].x * vv[nb].x - pw[nb].y * vv[nb].y,
                                       pw[nb].x * vv[nb].y + pw[nb].y * vv[nb].x};
                    }
                    // past the other lane half's four terms
                    pw[nb] = (f2v){pw[nb].x * v4[nb].x - pw[nb].y * v4[nb].y,
                                   pw[nb].x * v4[nb].y + pw[nb].y * v4[nb].x};
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bh, ah[nb], acc[nb], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bl, ah[nb], acc[nb], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bh, al[nb], acc[nb], 0, 0, 0);
            }
        }
        const float* const tsel = far ? tau_far : tau;

        // C has a row per column 2f + p and a column per root (the weights are
        // the instruction's A operand): lane l holds root l % 32 of its block in
        // rows 8 (v/4) + 4 (l/32) + v % 4.  One swap of lane halves gives each
        // lane all rows of one root, that of block l / 32: rows 8 (v/4) + v % 4
        // in lo_rows, 8 (v/4) + 4 + v % 4 in hi_rows.
        static_assert(NB == 2, "one root per lane at the finish");
        f16v lo_rows, hi_rows;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0][v]), __float_as_uint(acc[1][v]),
                                                             false, false);
            lo_rows[v] = __uint_as_float(sw[0]);
            hi_rows[v] = __uint_as_float(sw[1]);
        }
        {
            float2 sums[F];
            const float us = rcp_safe(lh ? sig[1] : sig[0]);
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const float ts = tsel[f] * us;
                const int r0 = 2 * f, r1 = 2 * f + 1;
                const float c0 = ((r0 >> 2) & 1) ? hi_rows[4 * (r0 >> 3) + (r0 & 3)] : lo_rows[4 * (r0 >> 3) + (r0 & 3)];
                const float c1 = ((r1 >> 2) & 1) ? hi_rows[4 * (r1 >> 3) + (r1 & 3)] : lo_rows[4 * (r1 >> 3) + (r1 & 3)];
                sums[f] = make_float2(c0 * ts, c1 * ts);
            }
            const float stv = lh ? st[1] : st[0];
            const float tfv = lh ? tf[1] : tf[0];
            const int pos = tile * TILE + wv * (32 * NB) + lh * 32 + row;
            if (pos < M) {
                float2 Hk;
                if (pos == pos_m1) {
                    const double* const m1 = reinterpret_cast<const double*>(rp + rec.scal + 72);
                    Hk = make_float2((float)(0.5 * dtv * m1[0]), (float)(0.5 * dtv * m1[1]));
                } else {
                    int st_root = 0;
                    if constexpr (RK == 2)
                        Hk = finish_root_r2(sums, stv, tfv, N, hbase, Lambda, P, Q, Bv, Ct, st_root);
                    else
                        Hk = finish_root<RK>(sums, stv, tfv, N, hbase, Lambda, P, Q, Bv, Ct, st_root);
                    my_status = max(my_status, st_root);
                }
                roots[(size_t)h * M + pos] = Hk;
            }
        }
    }
    // the workgroup's status in its first tile's entry (the readers take the
    // largest over a channel's entries), zero in the others
    __syncthreads();
    if (my_status) atomicMax(&blk_status, my_status);
    __syncthreads();
    if (tid < t1 - t0) tile_status[(size_t)h * tiles + t0 + tid] = tid == 0 ? blk_status : 0;
}

template <int RK, int RPT>
hipError_t launch_h(int64_t H, int64_t N, int64_t M, int scr_logm, const float2* Lambda, const float2* P,
                    const float2* Q, const float2* Bv, const float2* Ct, const float* dt, float2* roots,
                    int32_t* tstat, float2* twtab, double* tant, char* prep, float2* tw4, hipStream_t stream) {
    // the per-channel records, the root tables and (tw4 given) the transforms'
    // table in one launch
    const int64_t blocks0 = H + (M + 255) / 256 + (tw4 ? (2 * M + 255) / 256 : 0);
    hipLaunchKernelGGL((cauchy_h_prep_kernel<RK>), dim3((unsigned)blocks0), dim3(256), 0, stream, (int)H, (int)N,
                       Lambda, P, Q, Bv, Ct, prep, (int)M, scr_logm, tant, twtab, tw4);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const int tiles = (int)((M + kCauchyThreads * RPT - 1) / (kCauchyThreads * RPT));
    // tiles per workgroup: up to 4 while the grid keeps 8192 workgroups (the
    // staged weights are reused across a workgroup's tiles)
    int tpw = 1;
    while (tpw < 4 && tpw < tiles && H * ((tiles + 2 * tpw - 1) / (2 * tpw)) >= 8192) tpw *= 2;
    const int64_t blocks = H * ((tiles + tpw - 1) / tpw);
    const int pos_m1 = M < 2 ? -1 : scr_logm > 0 ? 512 : (int)(M / 2);  // where the root z = -1 is stored
    // the XCD mapping is a bijection on the grid when it holds whole groups of 8 channels
    const int xcd_remap = H % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((cauchy_h_kernel<RK, RPT>), dim3((unsigned)blocks), dim3(kCauchyThreads), 0, stream, (int)M,
                       pos_m1, (int)N, tiles, tpw, xcd_remap, Lambda, P, Q, Bv, Ct, dt, prep, tant, roots, tstat);
    return hipGetLastError();
}

template <int RK, int RPT>
hipError_t launch_rk(int64_t H, int64_t N, int64_t M, int scr_logm, const float2* Lambda, const float2* P,
                     const float2* Q, const float2* Bv, const float2* Ct, const float* dt, float2* roots,
                     int32_t* tstat, float2* twtab, double* tant, float2* tw4, hipStream_t stream) {
    // tw4 (nullable): the wave-structured transforms' table, written by the
    // tables launch (four roots per thread only)
    if (RPT >= 4) {
        const int64_t blocks0 = (M + 255) / 256 + (tw4 ? (2 * M + 255) / 256 : 0);
        hipLaunchKernelGGL(root_tables_kernel, dim3((unsigned)blocks0), dim3(256), 0, stream, (int)M, scr_logm, tant,
                           twtab, tw4);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    const int tiles = (int)((M + kCauchyThreads * RPT - 1) / (kCauchyThreads * RPT));
    const int64_t blocks = H * tiles;
    hipLaunchKernelGGL((cauchy_roots_kernel<RK, RPT>), dim3((unsigned)blocks), dim3(kCauchyThreads), 0, stream,
                       (int)M, scr_logm, (int)N, tiles, Lambda, P, Q, Bv, Ct, dt, roots, tstat, tant, twtab);
    return hipGetLastError();
}

}  // namespace

// roots per thread: up to 4 for r = 1 (more sums share each staged weight row;
// measured fastest, the accumulators of more roots crowd out waves), one for
// the split-precision kernel of ranks 2 and 3 (64 roots per wave, four waves
// per SIMD), while the grid keeps at least 1024 workgroups
// The split-precision kernel (matrix cores in float16 parts, with the far
// form for roots far from the poles) takes ranks 2 and 3, and rank 1 from 128
// states and 4096 roots: with 64 states the float32 kernel's sweep is cheaper
// (measured at 512 channels x 4096 roots: 67 against 78 us), with 256 the far
// form's savings win (256 channels x 65536 roots: 948 against 1478 us).
bool cauchy_split(int64_t N, int64_t r, int64_t M) { return r == 2 || r == 3 || (r == 1 && N >= 128 && M >= 4096); }

int cauchy_rpt(int64_t H, int64_t N, int64_t r, int64_t M) {
    const int max_rpt = r == 1 && !cauchy_split(N, r, M) ? 4 : 1;
    int rpt = max_rpt;
    while (rpt > 1 && H * ((M + (int64_t)kCauchyThreads * rpt - 1) / ((int64_t)kCauchyThreads * rpt)) < 1024)
        rpt >>= 1;
    return rpt;
}

int64_t cauchy_tiles(int64_t H, int64_t N, int64_t r, int64_t M) {
    const int64_t per = (int64_t)kCauchyThreads * cauchy_rpt(H, N, r, M);
    return (M + per - 1) / per;
}

// per-channel records of the split-precision path, else none
int64_t cauchy_prep_bytes(int64_t H, int64_t N, int64_t r, int64_t M) {
    return cauchy_split(N, r, M) ? H * HRec(N).bytes : 0;
}

// scrambled: store the root values in the order the wave-structured
// transforms take them (M >= 1024), not in natural order.  tw4 (nullable): the
// wave-structured transforms' table of 2M entries, written here when the
// split-precision kernel or the per-call root tables run (*tw4_done tells
// whether it was).
hipError_t launch_cauchy(int64_t H, int64_t N, int64_t r, int64_t M, const float2* Lambda, const float2* P,
                         const float2* Q, const float2* Bv, const float2* Ct, const float* dt, float2* roots,
                         int32_t* tile_status, float2* twtab, double* tant, void* prep, hipStream_t stream,
                         bool scrambled, float2* tw4, bool* tw4_done) {
    if (tw4_done) *tw4_done = false;
    const int rpt = cauchy_rpt(H, N, r, M);
    const bool split = cauchy_split(N, r, M);
    const int scr_logm = scrambled ? ilog2_exact(M) : 0;
    if (scrambled && M < 1024) return hipErrorInvalidValue;
#define SSM_CAUCHY(RK, RPT)                                                                                   \
    if (!split && r == RK && rpt == RPT) {                                                                    \
        if (tw4_done) *tw4_done = RPT >= 4 && tw4 != nullptr;                                                 \
        return launch_rk<RK, RPT>(H, N, M, scr_logm, Lambda, P, Q, Bv, Ct, dt, roots, tile_status, twtab, tant, \
                                  RPT >= 4 ? tw4 : nullptr, stream);                                          \
    }
#define SSM_CAUCHY_H(RK, RPT)                                                                                  \
    if (split && r == RK && rpt == RPT)                                                                        \
    {                                                                                                          \
        if (tw4_done) *tw4_done = tw4 != nullptr;                                                              \
        return launch_h<RK, RPT>(H, N, M, scr_logm, Lambda, P, Q, Bv, Ct, dt, roots, tile_status, twtab, tant,  \
                                 (char*)prep, tw4, stream);                                                    \
    }
    SSM_CAUCHY(1, 4) SSM_CAUCHY(1, 2) SSM_CAUCHY(1, 1)
    SSM_CAUCHY_H(1, 1) SSM_CAUCHY_H(2, 1) SSM_CAUCHY_H(3, 1)
    SSM_CAUCHY(4, 1)
#undef SSM_CAUCHY
#undef SSM_CAUCHY_H
    return hipErrorInvalidValue;
}

}  // namespace ssm
