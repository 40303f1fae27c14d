// Root values of the S4 filter mode: the pieces shared by the root-value
// kernels (per-chunk state tables in LDS, the sweep over a chunk, and the
// Woodbury finish of one root).
//
// Source: "Recurrent, LSTM, and structured state-space models", block for S4
// Algorithm 1 / App. C (filter mode): resolvent sums rho_uv(k) =
// sum_n conj(u_n) v_n / (s(z_k) - lambda_n) for u in {C~, Q_a}, v in {B, P_b},
// W = I_r + rho_QP, H = (1 + i t_k)(rho_C~B - rho_C~P W^{-1} rho_QB).
#pragma once

#include <float.h>

#include "common.hpp"

namespace ssm {

template <int RK>
struct Fam {
    static constexpr int F = (RK + 1) * (RK + 1);
    static constexpr int ROW = 1 + F;  // float4 per state, wide rows: header + one per family
    static constexpr int ROWN = 1 + (F + 1) / 2;  // narrow rows: header + a float2 per family
    // states staged in LDS at a time (<= 26 KB): the whole state vector for N up to this
    static constexpr int CHUNK = RK == 1 ? 256 : RK == 2 ? 128 : 64;
};

__device__ __forceinline__ float2 cdivf(float2 a, float2 b) {
    const float den = fmaf(b.x, b.x, b.y * b.y);
    const float inv = 1.0f / den;
    return make_float2(fmaf(a.x, b.x, a.y * b.y) * inv, fmaf(a.y, b.x, -a.x * b.y) * inv);
}

__device__ __forceinline__ float cabs1(float2 a) { return fabsf(a.x) + fabsf(a.y); }

// Solve W x = rhs in place (x returned in rhs), W r x r complex.  Gaussian
// elimination with partial pivoting; false when a pivot is exactly zero.
template <int RK>
__device__ __forceinline__ bool small_solve(float2 (&W)[RK][RK], float2 (&rhs)[RK]) {
#pragma unroll
    for (int c = 0; c < RK; ++c) {
#pragma unroll
        for (int r = c + 1; r < RK; ++r) {
            const bool sw = cabs1(W[r][c]) > cabs1(W[c][c]);
#pragma unroll
            for (int j = 0; j < RK; ++j) {
                const float2 a = W[c][j], b = W[r][j];
                W[c][j] = sw ? b : a;
                W[r][j] = sw ? a : b;
            }
            const float2 a = rhs[c], b = rhs[r];
            rhs[c] = sw ? b : a;
            rhs[r] = sw ? a : b;
        }
        if (W[c][c].x == 0.0f && W[c][c].y == 0.0f) return false;
#pragma unroll
        for (int r = c + 1; r < RK; ++r) {
            const float2 f = cdivf(W[r][c], W[c][c]);
#pragma unroll
            for (int j = c + 1; j < RK; ++j) W[r][j] = c_sub(W[r][j], c_mul(f, W[c][j]));
            rhs[r] = c_sub(rhs[r], c_mul(f, rhs[c]));
        }
    }
#pragma unroll
    for (int c = RK - 1; c >= 0; --c) {
        float2 s = rhs[c];
#pragma unroll
        for (int j = c + 1; j < RK; ++j) s = c_sub(s, c_mul(W[c][j], rhs[j]));
        rhs[c] = cdivf(s, W[c][c]);
    }
    return true;
}

// u vector of family row iu (0: C~, 1+a: Q_a), v vector of column iv (0: B, 1+b: P_b)
template <int RK>
__device__ __forceinline__ float2 fam_u(const float2* Ct, const float2* Q, size_t hn, int iu) {
    return iu == 0 ? Ct[hn] : Q[hn * RK + (iu - 1)];
}
template <int RK>
__device__ __forceinline__ float2 fam_v(const float2* Bv, const float2* P, size_t hn, int iv) {
    return iv == 0 ? Bv[hn] : P[hn * RK + (iv - 1)];
}

// Slow path for one root whose fast sums are not finite: exact resonance test,
// else the sums again with a scaled complex reciprocal.
template <int RK>
__device__ __forceinline__ bool root_recheck(int N, size_t hbase, float st, const float2* Lambda, const float2* P,
                                          const float2* Q, const float2* Bv, const float2* Ct,
                                          float2 (&acc)[Fam<RK>::F]) {
    for (int n = 0; n < N; ++n) {
        const float2 lam = Lambda[hbase + n];
        const float x = -lam.x, y = st - lam.y;
        if (x == 0.0f && y == 0.0f) return false;
    }
#pragma unroll
    for (int f = 0; f < Fam<RK>::F; ++f) acc[f] = make_float2(0.f, 0.f);
    for (int n = 0; n < N; ++n) {
        const float2 lam = Lambda[hbase + n];
        const float2 g = cdivf(make_float2(1.f, 0.f), make_float2(-lam.x, st - lam.y));
        const float2 gs = (isfinite(g.x) && isfinite(g.y))
                              ? g
                              : c_from(z_inv(make_double2(-(double)lam.x, (double)st - (double)lam.y)));
#pragma unroll
        for (int iu = 0; iu <= RK; ++iu)
#pragma unroll
            for (int iv = 0; iv <= RK; ++iv) {
                const float2 w = c_mul(c_conj(fam_u<RK>(Ct, Q, hbase + n, iu)), fam_v<RK>(Bv, P, hbase + n, iv));
                acc[iu * (RK + 1) + iv] = c_add(acc[iu * (RK + 1) + iv], c_mul(w, gs));
            }
    }
    return true;
}


// Stage one state's table row: header (x^2, Im lambda, x, 0) with x = -Re lambda,
// then per family f = iu (r+1) + iv the weight w = conj(u_iu) v_iv, either alone
// (narrow rows: a float2 per family, padded to whole float4) or with w x
// (wide rows: (w.x x, w.y x, w.y, -w.x), one float4 per family).
template <int RK, bool NARROW>
__device__ __forceinline__ void stage_row(float4* row, float2 lam, const float2 (&uu)[RK + 1],
                                          const float2 (&vv)[RK + 1]) {
    constexpr int F = Fam<RK>::F;
    const float x = -lam.x;
    row[0] = make_float4(x * x, lam.y, x, 0.f);
#pragma unroll
    for (int iu = 0; iu <= RK; ++iu)
#pragma unroll
        for (int iv = 0; iv <= RK; ++iv) {
            const float2 w = c_mul(c_conj(uu[iu]), vv[iv]);
            const int f = iu * (RK + 1) + iv;
            if constexpr (NARROW)
                reinterpret_cast<float2*>(row + 1)[f] = w;
            else
                row[1 + f] = make_float4(w.x * x, w.y * x, w.y, -w.x);
        }
    if constexpr (NARROW && (F & 1)) reinterpret_cast<float2*>(row + 1)[F] = make_float2(0.f, 0.f);
}

// Accumulate the nch staged states at tbl into the sums of RPT roots with
// st = a tan(pi k/M).  FAIR: the wave priority falls when the caller's progress
// count n0 + n reaches q1, q2, q3 (n0: states this thread swept before).
template <int RK, int RPT, bool NARROW, bool FAIR>
__device__ __forceinline__ void sweep_chunk(const float4* tbl, int nch, int n0, int q1, int q2, int q3,
                                            const float (&st)[RPT], float2 (&acc)[RPT][Fam<RK>::F]) {
    constexpr int F = Fam<RK>::F;
    constexpr int RW = NARROW ? Fam<RK>::ROWN : Fam<RK>::ROW;
    for (int n = 0; n < nch; ++n) {
        if constexpr (FAIR) {
            if (n0 + n == q1) __builtin_amdgcn_s_setprio(2);
            if (n0 + n == q2) __builtin_amdgcn_s_setprio(1);
            if (n0 + n == q3) __builtin_amdgcn_s_setprio(0);
        }
        const float4 hd = tbl[n * RW];
        float inv[RPT], p[RPT], q[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float y = st[i] - hd.y;
            const float den = fmaf(y, y, hd.x);
            inv[i] = __builtin_amdgcn_rcpf(den);
            p[i] = y * inv[i];
            if constexpr (NARROW) q[i] = hd.z * inv[i];  // x inv
        }
        if constexpr (NARROW) {
            const float2* wrow = reinterpret_cast<const float2*>(tbl + n * RW + 1);
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const float2 w = wrow[f];
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    acc[i][f].x = fmaf(w.x, q[i], acc[i][f].x);
                    acc[i][f].x = fmaf(w.y, p[i], acc[i][f].x);
                    acc[i][f].y = fmaf(w.y, q[i], acc[i][f].y);
                    acc[i][f].y = fmaf(-w.x, p[i], acc[i][f].y);  // negation is a free source modifier
                }
            }
        } else {
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const float4 w = tbl[n * RW + 1 + f];
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    acc[i][f].x = fmaf(w.x, inv[i], acc[i][f].x);
                    acc[i][f].x = fmaf(w.z, p[i], acc[i][f].x);
                    acc[i][f].y = fmaf(w.y, inv[i], acc[i][f].y);
                    acc[i][f].y = fmaf(w.w, p[i], acc[i][f].y);
                }
            }
        }
    }
}

// Root value from the finished sums of one root (k != M/2): a non-finite sum
// goes through the exact resonance test (status resonant-diagonal, NaN); a
// zero pivot of W gives resonant-correction (NaN).  status is max-updated.
template <int RK>
__device__ __forceinline__ float2 finish_root(float2 (&acc)[Fam<RK>::F], float st, float tf, int N, size_t hbase,
                                              const float2* Lambda, const float2* P, const float2* Q,
                                              const float2* Bv, const float2* Ct, int& status) {
    constexpr int F = Fam<RK>::F;
    bool finite = true;
#pragma unroll
    for (int f = 0; f < F; ++f) finite = finite && isfinite(acc[f].x) && isfinite(acc[f].y);
    if (!finite && !root_recheck<RK>(N, hbase, st, Lambda, P, Q, Bv, Ct, acc)) {
        status = max(status, SSM_ST_RESONANT_DIAGONAL);
        return c_nan();
    }
    float2 W[RK][RK], rhs[RK];
#pragma unroll
    for (int r1 = 0; r1 < RK; ++r1) {
        rhs[r1] = acc[(1 + r1) * (RK + 1)];
#pragma unroll
        for (int c1 = 0; c1 < RK; ++c1) {
            W[r1][c1] = acc[(1 + r1) * (RK + 1) + 1 + c1];
            if (r1 == c1) W[r1][c1].x += 1.0f;
        }
    }
    if (!small_solve<RK>(W, rhs)) {
        status = max(status, SSM_ST_RESONANT_CORRECTION);
        return c_nan();
    }
    float2 s = acc[0];
#pragma unroll
    for (int b1 = 0; b1 < RK; ++b1) s = c_sub(s, c_mul(acc[1 + b1], rhs[b1]));
    return c_mul(make_float2(1.0f, tf), s);
}

}  // namespace ssm
