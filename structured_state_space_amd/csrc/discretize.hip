// Bilinear discretisation of DPLR channels in float64, one wavefront per channel.
//
// Source: "Recurrent, LSTM, and structured state-space models", DPLR block
// (Abar = (I - dt A/2)^{-1}(I + dt A/2), Bbar = (I - dt A/2)^{-1} dt B, the
// truncated-output vector C~_M = (I - Abar^M)^* C) and the recurrent-solver
// passage of the Algorithm-1 block (d_j = 1 - alpha lambda_j, Woodbury core
// I_r + alpha Q^* D^{-1} P when no d_j is zero, else the bordered system when
// |Z| <= r, status singular-bilinear-matrix otherwise).
//
// G = D + alpha P Q^* with D = diag(d).  Every solve G x = b runs through one
// small matrix Mb of order r + s (s = |Z|):
//     [ I_r + alpha Q_J^* D_J^{-1} P_J   -Q_Z^* ] [ z   ]   [ Q_J^* D_J^{-1} b_J ]
//     [ alpha P_Z                         0     ] [ x_Z ] = [ b_Z                ]
//     x_J = D_J^{-1} (b_J - alpha P_J z)
// (s = 0 is the Woodbury form).  The adjoint G^* = conj(D) + alpha Q P^* has the
// same shape with P and Q exchanged; its top-left block is the conjugate
// transpose of G's.  Abar = G^{-1}(2I - G) = 2 G^{-1} - I, so Abar^* c = 2 G^{-*} c - c,
// and C~ = C - (Abar^*)^M C takes M such adjoint steps.
#include <float.h>

#include "bilinear.hpp"
#include "common.hpp"

namespace ssm {

namespace {

struct SmallMats {
    double2 Mb[kMaxOrder * kMaxOrder];
    double2 Mbinv[kMaxOrder * kMaxOrder];
    double2 Ma[kMaxOrder * kMaxOrder];
    double2 Mainv[kMaxOrder * kMaxOrder];
    double2 zc[4];  // values at Z read during an adjoint step
    int zidx[4];
    int s;
    int ok;
};

// C~ = C - (Abar^*)^M C for N <= 64 NPL, with the iteration state in
// registers: lane l holds states l + 64 e.  Each adjoint step is one DPP
// reduction of the r sums P^* D^{-*} c, the order r + s solve (the values at
// Z read by readlane), and the update c <- 2 G^{-*} c - c; no barrier.
template <int NPL, int RK>
__device__ void ctilde_in_registers(int N, int s, int M, double alpha, const double2* dinv, const float2* P,
                                    const float2* Q, size_t hb, const SmallMats& sm, const float2* C, float2* Ct,
                                    int lane) {
    const size_t hr = hb * RK;
    const int n = RK + s;
    double2 c[NPL], dc[NPL], pc[NPL][RK], qc[NPL][RK];
    int zs[NPL];
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        const bool live = j < N;
        c[e] = live ? z_from(C[hb + j]) : make_double2(0.0, 0.0);
        const double2 di = live ? dinv[j] : make_double2(0.0, 0.0);
        dc[e] = z_conj(di);
        zs[e] = -1;
        for (int z = 0; z < s; ++z)
            if (sm.zidx[z] == j) zs[e] = z;
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            const double2 p = live ? z_from(P[hr + (size_t)j * RK + a]) : make_double2(0.0, 0.0);
            const double2 q = live ? z_from(Q[hr + (size_t)j * RK + a]) : make_double2(0.0, 0.0);
            pc[e][a] = z_conj(z_mul(p, di));
            qc[e][a] = z_scale(q, alpha);
        }
    }
    int zl[4], ze[4];  // owner lane and slot of each state in Z (uniform)
#pragma unroll
    for (int z = 0; z < 4; ++z) {
        const int j = z < s ? sm.zidx[z] : 0;
        zl[z] = j % kWave;
        ze[z] = j / kWave;
    }
    // one adjoint step: the r sums P^* D^{-*} c over the states, then
    // c <- 2 x - c with x_J = conj(D_J^{-1}) (c_J - alpha Q_J sol), x_Z = sol_Z
    auto sums = [&](double2 (&rhs)[RK]) {
        double v[2 * RK];
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            double2 acc = make_double2(0.0, 0.0);
#pragma unroll
            for (int e = 0; e < NPL; ++e) acc = z_add(acc, z_mul(pc[e][a], c[e]));
            v[2 * a] = acc.x;
            v[2 * a + 1] = acc.y;
        }
        wave_allsum_d<2 * RK>(v);
#pragma unroll
        for (int a = 0; a < RK; ++a) rhs[a] = make_double2(v[2 * a], v[2 * a + 1]);
    };
    if (s == 0) {  // Woodbury form: the r x r inverse in registers
        double2 mi[RK][RK];
#pragma unroll
        for (int a = 0; a < RK; ++a)
#pragma unroll
            for (int b = 0; b < RK; ++b) mi[a][b] = sm.Mainv[a * kMaxOrder + b];
        for (int step = 0; step < M; ++step) {
            double2 rhs[RK], sol[RK];
            sums(rhs);
#pragma unroll
            for (int a = 0; a < RK; ++a) {
                double2 acc = make_double2(0.0, 0.0);
#pragma unroll
                for (int b = 0; b < RK; ++b) acc = z_add(acc, z_mul(mi[a][b], rhs[b]));
                sol[a] = acc;
            }
#pragma unroll
            for (int e = 0; e < NPL; ++e) {
                double2 t = c[e];
#pragma unroll
                for (int a = 0; a < RK; ++a) t = z_sub(t, z_mul(qc[e][a], sol[a]));
                const double2 x = z_mul(dc[e], t);
                c[e] = make_double2(2.0 * x.x - c[e].x, 2.0 * x.y - c[e].y);
            }
        }
    } else {  // bordered form: order r + s, the inverse read from LDS
        for (int step = 0; step < M; ++step) {
            double2 r0[RK];
            sums(r0);
            double2 rhs[kMaxOrder], sol[kMaxOrder];
#pragma unroll
            for (int a = 0; a < RK; ++a) rhs[a] = r0[a];
            for (int z = 0; z < s; ++z) {
                double2 cz = c[0];
#pragma unroll
                for (int e = 1; e < NPL; ++e)
                    if (ze[z] == e) cz = c[e];
                rhs[RK + z] = make_double2(readlane_d(cz.x, zl[z]), readlane_d(cz.y, zl[z]));
            }
            for (int a = 0; a < n; ++a) {
                double2 acc = make_double2(0.0, 0.0);
                for (int b = 0; b < n; ++b) acc = z_add(acc, z_mul(sm.Mainv[a * kMaxOrder + b], rhs[b]));
                sol[a] = acc;
            }
#pragma unroll
            for (int e = 0; e < NPL; ++e) {
                double2 t = c[e];
#pragma unroll
                for (int a = 0; a < RK; ++a) t = z_sub(t, z_mul(qc[e][a], sol[a]));
                double2 x = z_mul(dc[e], t);
                for (int z = 0; z < s; ++z)
                    if (zs[e] == z) x = sol[RK + z];
                c[e] = make_double2(2.0 * x.x - c[e].x, 2.0 * x.y - c[e].y);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        if (j < N) Ct[hb + j] = c_from(z_sub(z_from(C[hb + j]), c[e]));
    }
}

template <int NPL>
__device__ void ctilde_dispatch(int N, int r, int s, int M, double alpha, const double2* dinv, const float2* P,
                                const float2* Q, size_t hb, const SmallMats& sm, const float2* C, float2* Ct,
                                int lane) {
    switch (r) {
        case 1: ctilde_in_registers<NPL, 1>(N, s, M, alpha, dinv, P, Q, hb, sm, C, Ct, lane); break;
        case 2: ctilde_in_registers<NPL, 2>(N, s, M, alpha, dinv, P, Q, hb, sm, C, Ct, lane); break;
        case 3: ctilde_in_registers<NPL, 3>(N, s, M, alpha, dinv, P, Q, hb, sm, C, Ct, lane); break;
        default: ctilde_in_registers<NPL, 4>(N, s, M, alpha, dinv, P, Q, hb, sm, C, Ct, lane); break;
    }
}

__global__ __launch_bounds__(kWave) void discretize_kernel(int N, int r, int M, const float2* __restrict__ Lambda,
                                                           const float2* __restrict__ P, const float2* __restrict__ Q,
                                                           const float2* __restrict__ Bv, const float2* __restrict__ C,
                                                           const float* __restrict__ dt, float2* __restrict__ Bbar,
                                                           float2* __restrict__ Abar, float2* __restrict__ Ct,
                                                           int32_t* __restrict__ status) {
    extern __shared__ double2 dyn[];
    double2* cst = dyn;        // [N] adjoint-iteration state
    double2* dinv = dyn + N;   // [N] 1/d_j (0 for j in Z)
    __shared__ SmallMats sm;

    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const size_t hb = (size_t)h * N;
    const size_t hr = hb * r;
    const float dtf = dt[h];
    int st = SSM_ST_OK;

    if (!(dtf > 0.0f) || !(dtf <= FLT_MAX)) st = SSM_ST_INVALID_STEP;
    const double dtv = (double)dtf, alpha = 0.5 * dtv;

    if (st == SSM_ST_OK) {
        if (lane == 0) sm.s = 0;
        __syncthreads();
        for (int j0 = 0; j0 < N; j0 += kWave) {
            const int j = j0 + lane;
            bool isz = false;
            if (j < N) {
                const double2 lam = z_from(Lambda[hb + j]);
                const double2 d = make_double2(1.0 - alpha * lam.x, -alpha * lam.y);
                isz = z_is_zero(d);
                dinv[j] = isz ? make_double2(0.0, 0.0) : z_inv(d);
            }
            uint64_t mask = __ballot(isz);
            if (lane == 0) {
                while (mask) {
                    const int bit = __ffsll((unsigned long long)mask) - 1;
                    if (sm.s < 4) sm.zidx[sm.s] = j0 + bit;
                    sm.s++;
                    mask &= mask - 1;
                }
            }
        }
        __syncthreads();
        const int s = sm.s;
        if (s > r) st = SSM_ST_SINGULAR_BILINEAR;
        if (st == SSM_ST_OK) {
            // top-left block I + alpha Q_J^* D_J^{-1} P_J (wave reductions)
            for (int a = 0; a < r; ++a)
                for (int b = 0; b < r; ++b) {
                    double2 acc = make_double2(0.0, 0.0);
                    for (int j = lane; j < N; j += kWave) {
                        const double2 q = z_from(Q[hr + (size_t)j * r + a]);
                        const double2 p = z_from(P[hr + (size_t)j * r + b]);
                        acc = z_add(acc, z_mul(z_mul(z_conj(q), dinv[j]), p));
                    }
                    acc = wave_sum(acc);
                    if (lane == 0) {
                        const double2 tl = make_double2((a == b ? 1.0 : 0.0) + alpha * acc.x, alpha * acc.y);
                        sm.Mb[a * kMaxOrder + b] = tl;
                        sm.Ma[b * kMaxOrder + a] = z_conj(tl);
                    }
                }
            if (lane == 0) {
                const int n = r + s;
                for (int z = 0; z < s; ++z) {
                    const size_t jz = (size_t)sm.zidx[z];
                    for (int a = 0; a < r; ++a) {
                        const double2 q = z_from(Q[hr + jz * r + a]);
                        const double2 p = z_from(P[hr + jz * r + a]);
                        sm.Mb[a * kMaxOrder + r + z] = make_double2(-q.x, q.y);     // -conj(Q_za)
                        sm.Mb[(r + z) * kMaxOrder + a] = z_scale(p, alpha);        // alpha P_za
                        sm.Ma[a * kMaxOrder + r + z] = make_double2(-p.x, p.y);     // -conj(P_za)
                        sm.Ma[(r + z) * kMaxOrder + a] = z_scale(q, alpha);        // alpha Q_za
                    }
                    for (int z2 = 0; z2 < s; ++z2) {
                        sm.Mb[(r + z) * kMaxOrder + r + z2] = make_double2(0.0, 0.0);
                        sm.Ma[(r + z) * kMaxOrder + r + z2] = make_double2(0.0, 0.0);
                    }
                }
                sm.ok = small_inverse(sm.Mb, sm.Mbinv, n) && small_inverse(sm.Ma, sm.Mainv, n);
            }
            __syncthreads();
            if (!sm.ok) st = SSM_ST_SINGULAR_BILINEAR;
        }
    }

    if (st != SSM_ST_OK) {
        const float2 nan2 = c_nan();
        for (int j = lane; j < N; j += kWave) {
            if (Bbar) Bbar[hb + j] = nan2;
            if (Ct) Ct[hb + j] = nan2;
        }
        if (Abar)
            for (size_t e = lane; e < (size_t)N * N; e += kWave) Abar[(size_t)h * N * N + e] = nan2;
        if (lane == 0 && status) status[h] = st;
        return;
    }
    const int s = sm.s, n = r + s;

    // ---- Bbar = G^{-1} (dt B) ----
    if (Bbar) {
        double2 rhs[kMaxOrder];
        for (int a = 0; a < r; ++a) {
            double2 acc = make_double2(0.0, 0.0);
            for (int j = lane; j < N; j += kWave) {
                const double2 q = z_from(Q[hr + (size_t)j * r + a]);
                acc = z_add(acc, z_mul(z_mul(z_conj(q), dinv[j]), z_scale(z_from(Bv[hb + j]), dtv)));
            }
            rhs[a] = wave_sum(acc);
        }
        for (int z = 0; z < s; ++z) rhs[r + z] = z_scale(z_from(Bv[hb + sm.zidx[z]]), dtv);
        double2 sol[kMaxOrder];
        for (int i = 0; i < n; ++i) {
            double2 acc = make_double2(0.0, 0.0);
            for (int j = 0; j < n; ++j) acc = z_add(acc, z_mul(sm.Mbinv[i * kMaxOrder + j], rhs[j]));
            sol[i] = acc;
        }
        for (int j = lane; j < N; j += kWave) {
            double2 x;
            if (!z_is_zero(dinv[j])) {
                double2 t = z_scale(z_from(Bv[hb + j]), dtv);
                for (int a = 0; a < r; ++a) t = z_sub(t, z_scale(z_mul(z_from(P[hr + (size_t)j * r + a]), sol[a]), alpha));
                x = z_mul(dinv[j], t);
            } else {
                x = make_double2(0.0, 0.0);
                for (int z = 0; z < s; ++z)
                    if (sm.zidx[z] == j) x = sol[r + z];
            }
            Bbar[hb + j] = c_from(x);
        }
    }

    // ---- dense Abar = 2 G^{-1} - I, one column per lane ----
    if (Abar) {
        for (int i0 = 0; i0 < N; i0 += kWave) {
            const int i = i0 + lane;
            const bool live = i < N;
            double2 rhs[kMaxOrder], sol[kMaxOrder];
            const bool iJ = live && !z_is_zero(dinv[live ? i : 0]);
            for (int a = 0; a < r; ++a)
                rhs[a] = iJ ? z_mul(z_conj(z_from(Q[hr + (size_t)i * r + a])), dinv[i]) : make_double2(0.0, 0.0);
            for (int z = 0; z < s; ++z) rhs[r + z] = make_double2(live && sm.zidx[z] == i ? 1.0 : 0.0, 0.0);
            for (int a = 0; a < n; ++a) {
                double2 acc = make_double2(0.0, 0.0);
                for (int b = 0; b < n; ++b) acc = z_add(acc, z_mul(sm.Mbinv[a * kMaxOrder + b], rhs[b]));
                sol[a] = acc;
            }
            for (int j = 0; j < N; ++j) {
                const double2 dj = dinv[j];
                double2 x;
                if (!z_is_zero(dj)) {
                    double2 t = make_double2(j == i ? 1.0 : 0.0, 0.0);
                    for (int a = 0; a < r; ++a)
                        t = z_sub(t, z_scale(z_mul(z_from(P[hr + (size_t)j * r + a]), sol[a]), alpha));
                    x = z_mul(dj, t);
                } else {
                    x = make_double2(0.0, 0.0);
                    for (int z = 0; z < s; ++z)
                        if (sm.zidx[z] == j) x = sol[r + z];
                }
                const double2 aij = make_double2(2.0 * x.x - (j == i ? 1.0 : 0.0), 2.0 * x.y);
                if (live) Abar[(size_t)h * N * N + (size_t)j * N + i] = c_from(aij);
            }
        }
    }

    // ---- C~ = C - (Abar^*)^M C by M adjoint steps ----
    if (Ct && N <= 4 * kWave) {
        const int s = sm.s;
        if (N <= kWave)
            ctilde_dispatch<1>(N, r, s, M, alpha, dinv, P, Q, hb, sm, C, Ct, lane);
        else if (N <= 2 * kWave)
            ctilde_dispatch<2>(N, r, s, M, alpha, dinv, P, Q, hb, sm, C, Ct, lane);
        else
            ctilde_dispatch<4>(N, r, s, M, alpha, dinv, P, Q, hb, sm, C, Ct, lane);
    } else if (Ct) {
        for (int j = lane; j < N; j += kWave) cst[j] = z_from(C[hb + j]);
        __syncthreads();
        for (int step = 0; step < M; ++step) {
            double2 rhs[kMaxOrder];
            for (int a = 0; a < r; ++a) {
                double2 acc = make_double2(0.0, 0.0);
                for (int j = lane; j < N; j += kWave) {
                    const double2 p = z_from(P[hr + (size_t)j * r + a]);
                    acc = z_add(acc, z_mul(z_conj(z_mul(p, dinv[j])), cst[j]));
                }
                rhs[a] = wave_sum(acc);
            }
            for (int z = 0; z < s; ++z) rhs[r + z] = cst[sm.zidx[z]];
            double2 sol[kMaxOrder];
            for (int a = 0; a < n; ++a) {
                double2 acc = make_double2(0.0, 0.0);
                for (int b = 0; b < n; ++b) acc = z_add(acc, z_mul(sm.Mainv[a * kMaxOrder + b], rhs[b]));
                sol[a] = acc;
            }
            __syncthreads();  // every lane has read cst[Z] before any update
            for (int j = lane; j < N; j += kWave) {
                const double2 dj = dinv[j];
                const double2 c = cst[j];
                double2 x;
                if (!z_is_zero(dj)) {
                    double2 t = c;
                    for (int a = 0; a < r; ++a)
                        t = z_sub(t, z_scale(z_mul(z_from(Q[hr + (size_t)j * r + a]), sol[a]), alpha));
                    x = z_mul(z_conj(dj), t);
                } else {
                    x = make_double2(0.0, 0.0);
                    for (int z = 0; z < s; ++z)
                        if (sm.zidx[z] == j) x = sol[r + z];
                }
                cst[j] = make_double2(2.0 * x.x - c.x, 2.0 * x.y - c.y);
            }
            __syncthreads();
        }
        for (int j = lane; j < N; j += kWave) Ct[hb + j] = c_from(z_sub(z_from(C[hb + j]), cst[j]));
    }
    if (lane == 0 && status) status[h] = SSM_ST_OK;
}

}  // namespace

size_t discretize_lds_bytes(int64_t N) { return (size_t)N * 2 * sizeof(double2); }

hipError_t launch_discretize(int64_t H, int64_t N, int64_t r, int64_t M, const float2* Lambda, const float2* P,
                             const float2* Q, const float2* Bv, const float2* C, const float* dt, float2* Bbar,
                             float2* Abar, float2* Ct, int32_t* status, hipStream_t stream) {
    const size_t lds = discretize_lds_bytes(N);
    hipError_t e = hipFuncSetAttribute((const void*)discretize_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(discretize_kernel, dim3((unsigned)H), dim3(kWave), lds, stream, (int)N, (int)r, (int)M, Lambda,
                       P, Q, Bv, C, dt, Bbar, Abar, Ct, status);
    return hipGetLastError();
}

}  // namespace ssm
