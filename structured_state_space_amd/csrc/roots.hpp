// Root values of the S4 filter mode: the pieces shared by the root-value
// kernels (per-chunk state tables in LDS, the sweep over a chunk on the matrix
// cores, and the Woodbury finish of one root).
//
// Source: "Recurrent, LSTM, and structured state-space models", block for S4
// Algorithm 1 / App. C (filter mode): resolvent sums rho_uv(k) =
// sum_n conj(u_n) v_n / (s(z_k) - lambda_n) for u in {C~, Q_a}, v in {B, P_b},
// W = I_r + rho_QP, H = (1 + i t_k)(rho_C~B - rho_C~P W^{-1} rho_QB).
//
// The sums over the states are a product of two matrices: the Cauchy matrix
// g(k, n) = 1/(s(z_k) - lambda_n) of the roots against the weight matrix
// w(n, f) = conj(u_n) v_n of the (r+1)^2 families.  With d = x + i y
// (x = -Re lambda_n, y = a t_k - Im lambda_n) and inv = 1/|d|^2,
//   w g = [(w.x x) inv + w.y (y inv)] + i [(w.y x) inv - w.x (y inv)],
// so in real arithmetic a root contributes the two numbers (inv, y inv) per
// state and the weights form a 2 x (2 F) real block per state (columns: Re and
// Im of each family).  Each lane forms its root's (inv, y inv) on the vector
// ALU; the 4x4x1 fp32 matrix instruction (16 independent 4x4 outer products
// per wave, one per group of four lanes) multiplies them by four weight
// columns at a time and accumulates in fp32.
#pragma once

#include <float.h>

#include "common.hpp"

namespace ssm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int RK>
struct Fam {
    static constexpr int F = (RK + 1) * (RK + 1);
    static constexpr int G = (2 * F + 3) / 4;  // groups of four real columns
    static constexpr int G2 = (G + 1) / 2;     // float4 per lane slot per state: two groups (k = 0, 1 each)
    static constexpr int WROW = 4 * G2;        // float4 of weights per state (one slot per lane of a quad)
    // states staged in LDS at a time (<= 30 KB with the headers): the whole
    // state vector for N up to this
    static constexpr int CHUNK = RK == 1 ? 256 : RK == 2 ? 128 : 64;
    // accumulation chains per column group (separate chains for the two
    // rows of the weight block where registers allow)
    static constexpr int KS = G <= 2 ? 2 : 1;
};

// 1/d: the hardware reciprocal (1 ulp) where d and 1/d are normal numbers,
// the IEEE division elsewhere
__device__ __forceinline__ float rcp_safe(float d) {
    const float m = fabsf(d);
    return (m >= 1e-37f && m <= 1e37f) ? __builtin_amdgcn_rcpf(d) : 1.0f / d;
}

__device__ __forceinline__ float2 cdivf(float2 a, float2 b) {
    const float den = fmaf(b.x, b.x, b.y * b.y);
    const float inv = rcp_safe(den);
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


// Stage one state's table entries: header (x^2, Im lambda) with x = -Re lambda,
// and the weight block.  Column col = 2 f + part (part 0: Re, 1: Im) of family
// f = iu (r+1) + iv, with w = conj(u_iu) v_iv, has row 0 (the inv row)
// (w.x x | w.y x) and row 1 (the y inv row) (w.y | -w.x).  Column col is in
// group c = col / 4 at quad lane j = col % 4; lane slot j of the state holds the
// float4 (row 0 of c, row 1 of c, row 0 of c+1, row 1 of c+1) for each even c.
// Columns past 2F are zero.
template <int RK>
__device__ __forceinline__ void stage_state(float2* hdr, float4* wrow, float2 lam, const float2 (&uu)[RK + 1],
                                            const float2 (&vv)[RK + 1]) {
    constexpr int F = Fam<RK>::F, G2 = Fam<RK>::G2;
    const float x = -lam.x;
    *hdr = make_float2(x * x, lam.y);
    float v[4 * G2][4];
#pragma unroll
    for (int s = 0; s < 4 * G2; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[s][e] = 0.0f;
#pragma unroll
    for (int iu = 0; iu <= RK; ++iu)
#pragma unroll
        for (int iv = 0; iv <= RK; ++iv) {
            const float2 w = c_mul(c_conj(uu[iu]), vv[iv]);
            const int f = iu * (RK + 1) + iv;
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                const int col = 2 * f + part, c = col >> 2, j = col & 3;
                const int s = (c >> 1) * 4 + j, e = (c & 1) * 2;
                v[s][e] = part ? w.y * x : w.x * x;
                v[s][e + 1] = part ? -w.x : w.y;
            }
        }
    (void)F;
#pragma unroll
    for (int s = 0; s < 4 * G2; ++s) wrow[s] = make_float4(v[s][0], v[s][1], v[s][2], v[s][3]);
}

// A padding state: zero weights and a header that keeps |d|^2 >= 1 (finite).
template <int RK>
__device__ __forceinline__ void stage_pad(float2* hdr, float4* wrow) {
    *hdr = make_float2(1.0f, 0.0f);
#pragma unroll
    for (int s = 0; s < Fam<RK>::WROW; ++s) wrow[s] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// States per unrolled step of the sweep, sized so that the step's operands and
// the accumulators of RPT roots stay in registers.
template <int RK, int RPT>
constexpr int sweep_unroll() {
    return RK == 1 ? (8 / RPT > 1 ? 8 / RPT : 2) : RK == 2 ? (4 / RPT > 1 ? 4 / RPT : 1) : RK == 3 ? 2 : 1;
}

template <int RK>
struct RootAcc {
    f32x4 d[Fam<RK>::KS][Fam<RK>::G];
};

template <int RK>
__device__ __forceinline__ void acc_zero(RootAcc<RK>& a) {
#pragma unroll
    for (int k = 0; k < Fam<RK>::KS; ++k)
#pragma unroll
        for (int c = 0; c < Fam<RK>::G; ++c) a.d[k][c] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Accumulate npad staged states (a multiple of U) into the sums of RPT root
// sets (one root per lane each) with st = a tan(pi k/M).  All 64 lanes of the
// wave must be active.  Per group of U states: the LDS reads and the vector
// work first, then the matrix instructions (measured faster than letting them
// interleave).  FAIR: the wave priority falls when the caller's progress count
// n0 + n reaches q1, q2, q3.
template <int RK, int RPT, int U, bool FAIR>
__device__ __forceinline__ void sweep_chunk(const float2* hdr, const float4* wt, int npad, int n0, int q1, int q2,
                                            int q3, const float (&st)[RPT], RootAcc<RK> (&acc)[RPT]) {
    constexpr int G = Fam<RK>::G, G2 = Fam<RK>::G2, WROW = Fam<RK>::WROW, KS = Fam<RK>::KS;
    const int j = threadIdx.x & 3;
    for (int n = 0; n < npad; n += U) {
        if constexpr (FAIR) {
            const int p0 = n0 + n, p1 = p0 + U;
            if (p0 <= q1 && q1 < p1) __builtin_amdgcn_s_setprio(2);
            if (p0 <= q2 && q2 < p1) __builtin_amdgcn_s_setprio(1);
            if (p0 <= q3 && q3 < p1) __builtin_amdgcn_s_setprio(0);
        }
        float a0[RPT][U], a1[RPT][U];
        float4 b[U][G2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float2 hd = hdr[n + u];
#pragma unroll
            for (int c2 = 0; c2 < G2; ++c2) b[u][c2] = wt[(n + u) * WROW + c2 * 4 + j];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float yv = st[i] - hd.y;
                const float den = fmaf(yv, yv, hd.x);
                a0[i][u] = __builtin_amdgcn_rcpf(den);
                a1[i][u] = yv * a0[i][u];
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, U * (1 + G2), 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x2, 4 * U * RPT, 0);     // vector ALU
        // issue order: an accumulator recurs only after G (or 2G) other
        // instructions, so no instruction waits on the one before it
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < RPT; ++i)
#pragma unroll
                for (int k = 0; k < 2; ++k)
#pragma unroll
                    for (int c = 0; c < G; ++c) {
                        const float4 bb = b[u][c >> 1];
                        const float bk = k ? ((c & 1) ? bb.w : bb.y) : ((c & 1) ? bb.z : bb.x);
                        f32x4& d = acc[i].d[k < KS ? k : 0][c];
                        d = __builtin_amdgcn_mfma_f32_4x4x1f32(k ? a1[i][u] : a0[i][u], bk, d, 0, 0, 0);
                    }
        __builtin_amdgcn_sched_group_barrier(0x8, 2 * G * U * RPT, 0);  // matrix
    }
}

// Lane l of quad q holds, in element i of group c, the sum of column 4c + l for
// the root of lane 4q + i; transpose each quad's 4x4 blocks (two exchange
// steps across lanes l ^ 1 and l ^ 2) so that the lane holds its own root's
// columns, and unpack them into per-family complex sums.  All 64 lanes active.
template <int RK>
__device__ __forceinline__ void acc_unpack(const RootAcc<RK>& a, float2 (&out)[Fam<RK>::F]) {
    constexpr int F = Fam<RK>::F, G = Fam<RK>::G;
    const int l0 = threadIdx.x & 1, l1 = (threadIdx.x >> 1) & 1;
#pragma unroll
    for (int c = 0; c < G; ++c) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a.d[0][c][e] + (Fam<RK>::KS == 2 ? a.d[Fam<RK>::KS - 1][c][e] : 0.0f);
        // step 1: element (i1, 1 - l0) comes from the lane l ^ 1
#pragma unroll
        for (int i1 = 0; i1 < 2; ++i1) {
            const float send = l0 ? v[2 * i1] : v[2 * i1 + 1];
            const float recv =
                __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
            if (l0)
                v[2 * i1] = recv;
            else
                v[2 * i1 + 1] = recv;
        }
        // step 2: element (1 - l1, i0) comes from the lane l ^ 2
#pragma unroll
        for (int i0 = 0; i0 < 2; ++i0) {
            const float send = l1 ? v[i0] : v[2 + i0];
            const float recv =
                __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
            if (l1)
                v[i0] = recv;
            else
                v[2 + i0] = recv;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 4 * c + e;
            if (col < 2 * F) {
                if (col & 1)
                    out[col >> 1].y = v[e];
                else
                    out[col >> 1].x = v[e];
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
