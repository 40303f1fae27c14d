// Recurrent (step) mode of DPLR channels: the bilinear recurrence run one step
// at a time, with the state kept between calls (streaming inference).
//
// Source: "Recurrent, LSTM, and structured state-space models", DPLR block
// (x_t = Abar x_{t-1} + Bbar u_t, y_t = C^* x_t + D u_t with
// Abar = (I - dt A/2)^{-1}(I + dt A/2), Bbar = (I - dt A/2)^{-1} dt B) and the
// recurrent-solver passage of the Algorithm-1 block (each step solves with
// G = I - alpha A, alpha = dt/2, in O(N r) through the Woodbury core, or the
// bordered system when some d_j = 1 - alpha lambda_j is zero).
//
// Abar is never formed: Abar = G^{-1}(2I - G) = 2 G^{-1} - I, so
//   x_t = 2 G^{-1} x_{t-1} - x_{t-1} + Bbar u_t,
// and with D = diag(d), Z = {j : d_j = 0} (s = |Z| <= r), J its complement,
//   [z; x_Z] = Mb^{-1} [Q_J^* D_J^{-1} v_J; v_Z],   (G^{-1} v)_J = D_J^{-1} v_J - alpha D_J^{-1} P_J z,
//   (G^{-1} v)_Z = x_Z
// where Mb (order r + s) is the matrix of the discretisation kernel.  Per step
// the wave reduces r + 1 complex sums over the states in one pass (the r sums
// Q^* D^{-1} x_{t-1} and C^* x_{t-1}, which gives y_{t-1}), reads x_{t-1} at Z,
// solves with Mb^{-1} and updates its states.
//
// Work split, two layouts.  One 64-lane wave per sequence (batch row b,
// channel h): lane l holds states l + 64 e, e < NPL; the channel's set-up
// (d, Z, Mb^{-1}, Bbar) is computed in float64 by the wave itself; inputs and
// outputs move in blocks of 64 steps (one coalesced load or store per block,
// the next input block fetched one block ahead).  Or, for N <= 64, 16-lane
// groups with four sequences per wave (below).  The recurrence runs in
// float32.  The set-up can also be written once to a buffer (the prepared
// layout) and read by later calls.
#include <float.h>

#include "bilinear.hpp"
#include "common.hpp"

namespace ssm {

namespace {

constexpr int kMaxRank = 4;

struct StepSetup {
    double2 Mb[kMaxOrder * kMaxOrder];
    double2 Mbinv[kMaxOrder * kMaxOrder];
    float2 Mbf[kMaxOrder * kMaxOrder];
    int zidx[kMaxRank];
    int s;
    int ok;
};

// Sum over the 64 lanes, returned to every lane: DPP exchanges within each
// row of 16 lanes (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror: each lane then holds its row's sum), then the rows combined by
// the row broadcasts (lane 15 of rows 0 and 2 added into rows 1 and 3, then
// lane 31 into rows 2 and 3), so lane 63 holds the total, read once.  No LDS
// round trip (the shuffle-based sum takes six).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_get(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
// K values at once, stage by stage, so that the exchanges of different values
// fill each other's wait states
template <int K>
__device__ __forceinline__ void wave_allsum(float (&v)[K]) {
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0xB1>(v[i]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x4E>(v[i]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x141>(v[i]);  // row_half_mirror
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x140>(v[i]);  // row_mirror
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x142, 0xA>(v[i]);  // row_bcast:15 into rows 1 and 3
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x143, 0xC>(v[i]);  // row_bcast:31 into rows 2 and 3
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

// c + a b and c - a b as four fused multiply-adds (a separate product and
// sum would take two multiplies, two FMAs and two adds)
__device__ __forceinline__ float2 c_fma(float2 a, float2 b, float2 c) {
    return make_float2(fmaf(-a.y, b.y, fmaf(a.x, b.x, c.x)), fmaf(a.y, b.x, fmaf(a.x, b.y, c.y)));
}
__device__ __forceinline__ float2 c_fnma(float2 a, float2 b, float2 c) {
    return make_float2(fmaf(a.y, b.y, fmaf(-a.x, b.x, c.x)), fmaf(-a.y, b.x, fmaf(-a.x, b.y, c.y)));
}
// Re(c + a b)
__device__ __forceinline__ float c_fma_re(float2 a, float2 b, float c) { return fmaf(-a.y, b.y, fmaf(a.x, b.x, c)); }

// The first two blocks of a sequence's inputs, lane i holding step i and
// step B + i of blocks of B steps (indexes past the end clamped to the last)
template <int B>
__device__ __forceinline__ void first_inputs(const float* __restrict__ u, size_t ub, int T, int i, float& ucur,
                                             float& unext) {
    ucur = u[ub + min(i, T - 1)];
    unext = u[ub + min(B + i, T - 1)];
}

// The recurrence for one sequence: T steps from the state xs (updated in
// place).  NZ: room for the bordered form's states in Z (0: Woodbury form).
template <int NPL, int RK, int NZ>
__device__ __forceinline__ void recur(int T, int lane, size_t ub, int n, const float2* Mbf, const int (&zl)[kMaxRank],
                                      const int (&ze)[kMaxRank], const float2 (&qd)[NPL][RK],
                                      const float2 (&pa)[NPL][RK], const float2 (&dv)[NPL], const float2 (&cc)[NPL],
                                      const float2 (&bb)[NPL], const int (&zs)[NPL], float Dh, float ucur,
                                      float unext, const float* __restrict__ u, float* __restrict__ y,
                                      float2 (&xs)[NPL]) {
    constexpr int NO = RK + NZ;  // largest order of the small solve
    float2 Mr[NZ == 0 ? RK : 1][NZ == 0 ? RK : 1];
    if constexpr (NZ == 0) {
#pragma unroll
        for (int i = 0; i < RK; ++i)
#pragma unroll
            for (int j = 0; j < RK; ++j) Mr[i][j] = Mbf[i * kMaxOrder + j];
    }
    // ucur, unext: inputs of steps [0, 64) and [64, 128), loaded by the
    // caller (first_inputs) as early as it can; lanes past the end hold the
    // last input instead (never used), so the loads carry no branch
    float yblk = 0.0f;  // outputs of steps [t0, t0 + 64), lane = step - t0
    float uprev = 0.0f;
    for (int t = 0; t <= T; ++t) {
        // sums over x_{t-1}: Q^* D^{-1} x (r of them) and the real part of
        // C^* x (the only part y uses), seeded with the first state's terms
        float2 sq[RK];
        float scr = c_fma_re(cc[0], xs[0], 0.0f);
#pragma unroll
        for (int a = 0; a < RK; ++a) sq[a] = c_mul(qd[0][a], xs[0]);
#pragma unroll
        for (int e = 1; e < NPL; ++e) {
#pragma unroll
            for (int a = 0; a < RK; ++a) sq[a] = c_fma(qd[e][a], xs[e], sq[a]);
            scr = c_fma_re(cc[e], xs[e], scr);
        }
        {
            float v[2 * RK + 1];
#pragma unroll
            for (int a = 0; a < RK; ++a) {
                v[2 * a] = sq[a].x;
                v[2 * a + 1] = sq[a].y;
            }
            v[2 * RK] = scr;
            wave_allsum<2 * RK + 1>(v);
#pragma unroll
            for (int a = 0; a < RK; ++a) sq[a] = make_float2(v[2 * a], v[2 * a + 1]);
            scr = v[2 * RK];
        }
        if (t > 0) {  // y_{t-1} = Re(C^* x_{t-1}) + D u_{t-1}
            const int k = (t - 1) & (kWave - 1);
            if (lane == k) yblk = scr + Dh * uprev;
            if (k == kWave - 1 || t == T) {
                const int t0 = (t - 1) & ~(kWave - 1);
                if (t0 + lane < T) y[ub + t0 + lane] = yblk;
            }
        }
        if (t == T) break;
        const int k = t & (kWave - 1);
        if (k == 0 && t > 0) {  // next block of inputs
            ucur = unext;
            unext = u[ub + min(t + kWave + lane, T - 1)];
        }
        const float ut = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ucur), k));  // k is uniform
        // [z; x_Z] = Mb^{-1} [Q_J^* D_J^{-1} x; x_Z]
        float2 sol[NO];
        if constexpr (NZ == 0) {
#pragma unroll
            for (int i = 0; i < RK; ++i) {
                float2 acc = c_mul(Mr[i][0], sq[0]);
#pragma unroll
                for (int j = 1; j < RK; ++j) acc = c_fma(Mr[i][j], sq[j], acc);
                sol[i] = acc;
            }
        } else {
            float2 rhs[NO];
#pragma unroll
            for (int a = 0; a < RK; ++a) rhs[a] = sq[a];
#pragma unroll
            for (int zz = 0; zz < NZ; ++zz) {
                rhs[RK + zz] = make_float2(0.0f, 0.0f);
                if (RK + zz < n) {
                    float2 v = xs[0];
#pragma unroll
                    for (int e = 1; e < NPL; ++e)
                        if (ze[zz] == e) v = xs[e];
                    rhs[RK + zz] = make_float2(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.x), zl[zz])),
                                               __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.y), zl[zz])));
                }
            }
            // the inverse is read where it is used (an empty asm keeps the
            // compiler from holding all of it in registers across the loop)
            int off = 0;
            asm volatile("" : "+v"(off));
#pragma unroll
            for (int i = 0; i < NO; ++i) {
                float2 acc = make_float2(0.0f, 0.0f);
                if (i < n) {
#pragma unroll
                    for (int j = 0; j < NO; ++j)
                        if (j < n) acc = c_add(acc, c_mul(Mbf[off + i * kMaxOrder + j], rhs[j]));
                }
                sol[i] = acc;
            }
        }
        // x_t = 2 G^{-1} x_{t-1} - x_{t-1} + Bbar u_t
#pragma unroll
        for (int e = 0; e < NPL; ++e) {
            float2 g = c_mul(dv[e], xs[e]);
#pragma unroll
            for (int a = 0; a < RK; ++a) g = c_fnma(pa[e][a], sol[a], g);
            if constexpr (NZ > 0) {
#pragma unroll
                for (int zz = 0; zz < NZ; ++zz)
                    if (zs[e] == zz) g = sol[RK + zz];
            }
            xs[e] = make_float2(2.0f * g.x - xs[e].x + bb[e].x * ut, 2.0f * g.y - xs[e].y + bb[e].y * ut);
        }
        uprev = ut;
    }
}

// The channel set-up in float64: d^{-1}, the zero set Z, Mb^{-1} (into sm, as
// float32 in sm.Mbf) and Bbar = G^{-1} (dt B), then the float32 per-state
// constants of the recurrence in the lane's registers.  Returns the channel's
// status (uniform over the wave); on a failure the constants are not formed.
// States past N get zero constants.
template <int NPL, int RK>
__device__ __forceinline__ int channel_setup(int h, int N, int lane, const float2* __restrict__ Lambda,
                                             const float2* __restrict__ P, const float2* __restrict__ Q,
                                             const float2* __restrict__ Bv, const float2* __restrict__ C,
                                             const float* __restrict__ dt, StepSetup& sm, float2 (&qd)[NPL][RK],
                                             float2 (&pa)[NPL][RK], float2 (&dv)[NPL], float2 (&cc)[NPL],
                                             float2 (&bb)[NPL]) {
    const size_t hb = (size_t)h * N;
    const size_t hr = hb * RK;
    const float dtf = dt[h];
    int st = SSM_ST_OK;
    if (!(dtf > 0.0f) || !(dtf <= FLT_MAX)) st = SSM_ST_INVALID_STEP;
    const double dtv = (double)dtf, alpha = 0.5 * dtv;

    double2 dinv[NPL];
    if (lane == 0) sm.s = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        bool isz = false;
        dinv[e] = make_double2(0.0, 0.0);
        if (j < N && st == SSM_ST_OK) {
            const double2 lam = z_from(Lambda[hb + j]);
            const double2 d = make_double2(1.0 - alpha * lam.x, -alpha * lam.y);
            isz = z_is_zero(d);
            if (!isz) dinv[e] = z_inv(d);
        }
        uint64_t mask = __ballot(isz);
        if (lane == 0) {
            while (mask) {
                const int bit = __ffsll((unsigned long long)mask) - 1;
                if (sm.s < kMaxRank) sm.zidx[sm.s] = kWave * e + bit;
                sm.s++;
                mask &= mask - 1;
            }
        }
    }
    __syncthreads();
    const int s = sm.s;
    if (st == SSM_ST_OK && s > RK) st = SSM_ST_SINGULAR_BILINEAR;
    if (st == SSM_ST_OK) {
        for (int a = 0; a < RK; ++a)
            for (int c = 0; c < RK; ++c) {
                double2 acc = make_double2(0.0, 0.0);
#pragma unroll
                for (int e = 0; e < NPL; ++e) {
                    const int j = lane + kWave * e;
                    if (j < N) {
                        const double2 q = z_from(Q[hr + (size_t)j * RK + a]);
                        const double2 p = z_from(P[hr + (size_t)j * RK + c]);
                        acc = z_add(acc, z_mul(z_mul(z_conj(q), dinv[e]), p));
                    }
                }
                acc = wave_sum(acc);
                if (lane == 0) sm.Mb[a * kMaxOrder + c] = make_double2((a == c ? 1.0 : 0.0) + alpha * acc.x, alpha * acc.y);
            }
        if (lane == 0) {
            for (int zz = 0; zz < s; ++zz) {
                const size_t jz = (size_t)sm.zidx[zz];
                for (int a = 0; a < RK; ++a) {
                    const double2 q = z_from(Q[hr + jz * RK + a]);
                    const double2 p = z_from(P[hr + jz * RK + a]);
                    sm.Mb[a * kMaxOrder + RK + zz] = make_double2(-q.x, q.y);  // -conj(Q_za)
                    sm.Mb[(RK + zz) * kMaxOrder + a] = z_scale(p, alpha);     // alpha P_za
                }
                for (int z2 = 0; z2 < s; ++z2) sm.Mb[(RK + zz) * kMaxOrder + RK + z2] = make_double2(0.0, 0.0);
            }
            sm.ok = small_inverse(sm.Mb, sm.Mbinv, RK + s);
            for (int i = 0; i < kMaxOrder * kMaxOrder; ++i) sm.Mbf[i] = c_from(sm.Mbinv[i]);
        }
        __syncthreads();
        if (!sm.ok) st = SSM_ST_SINGULAR_BILINEAR;
    }
    if (st != SSM_ST_OK) return st;
    const int n = RK + s;

    // Bbar = G^{-1} (dt B) (float64), and the per-state constants
    double2 rhs[kMaxOrder];
    for (int a = 0; a < RK; ++a) {
        double2 acc = make_double2(0.0, 0.0);
#pragma unroll
        for (int e = 0; e < NPL; ++e) {
            const int j = lane + kWave * e;
            if (j < N) {
                const double2 q = z_from(Q[hr + (size_t)j * RK + a]);
                acc = z_add(acc, z_mul(z_mul(z_conj(q), dinv[e]), z_scale(z_from(Bv[hb + j]), dtv)));
            }
        }
        rhs[a] = wave_sum(acc);
    }
    for (int zz = 0; zz < s; ++zz) rhs[RK + zz] = z_scale(z_from(Bv[hb + sm.zidx[zz]]), dtv);
    double2 sol[kMaxOrder];
    for (int i = 0; i < n; ++i) {
        double2 acc = make_double2(0.0, 0.0);
        for (int j = 0; j < n; ++j) acc = z_add(acc, z_mul(sm.Mbinv[i * kMaxOrder + j], rhs[j]));
        sol[i] = acc;
    }
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        int zslot = -1;
        for (int zz = 0; zz < s; ++zz)
            if (sm.zidx[zz] == j) zslot = zz;
        double2 bbar = make_double2(0.0, 0.0);
        dv[e] = c_from(dinv[e]);
        cc[e] = make_float2(0.0f, 0.0f);
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            qd[e][a] = make_float2(0.0f, 0.0f);
            pa[e][a] = make_float2(0.0f, 0.0f);
        }
        if (j < N) {
            cc[e] = c_conj(C[hb + j]);
            if (zslot < 0) {
                double2 tb = z_scale(z_from(Bv[hb + j]), dtv);
#pragma unroll
                for (int a = 0; a < RK; ++a) {
                    const double2 q = z_from(Q[hr + (size_t)j * RK + a]);
                    const double2 p = z_from(P[hr + (size_t)j * RK + a]);
                    qd[e][a] = c_from(z_mul(z_conj(q), dinv[e]));
                    pa[e][a] = c_from(z_scale(z_mul(dinv[e], p), alpha));
                    tb = z_sub(tb, z_scale(z_mul(p, sol[a]), alpha));
                }
                bbar = z_mul(dinv[e], tb);
            } else {
                for (int zz = 0; zz < s; ++zz)
                    if (zslot == zz) bbar = sol[RK + zz];
            }
        }
        bb[e] = c_from(bbar);
    }
    return SSM_ST_OK;
}

// Z's bookkeeping for the recurrence: the slot in Z of each of the lane's
// states (or -1), and the owner lane and register slot of each state in Z
template <int NPL>
__device__ __forceinline__ void z_slots(int lane, int s, const int* zidx, int (&zs)[NPL], int (&zl)[kMaxRank],
                                        int (&ze)[kMaxRank]) {
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        zs[e] = -1;
        for (int zz = 0; zz < s; ++zz)
            if (zidx[zz] == j) zs[e] = zz;
    }
#pragma unroll
    for (int zz = 0; zz < kMaxRank; ++zz) {
        const int j = zz < s ? zidx[zz] : 0;
        zl[zz] = j % kWave;
        ze[zz] = j / kWave;
    }
}

// A failing channel: NaN outputs and state for the sequence
__device__ __forceinline__ void fail_sequence(int lane, int N, int T, size_t ub, size_t xb, float* __restrict__ y,
                                              float2* __restrict__ x) {
    const float nanf = __builtin_nanf("");
    for (int t = lane; t < T; t += kWave) y[ub + t] = nanf;
    for (int j = lane; j < N; j += kWave) x[xb + j] = c_nan();
}

template <int NPL, int RK>
__global__ __launch_bounds__(kWave) void step_kernel(int Bsz, int H, int N, int T, const float2* __restrict__ Lambda,
                                                     const float2* __restrict__ P, const float2* __restrict__ Q,
                                                     const float2* __restrict__ Bv, const float2* __restrict__ C,
                                                     const float* __restrict__ dt, const float* __restrict__ D,
                                                     const float* __restrict__ u, float* __restrict__ y,
                                                     float2* __restrict__ x, int32_t* __restrict__ status) {
    __shared__ StepSetup sm;
    const int seq = blockIdx.x;  // = b * H + h, the row order of u, y and x
    const int h = seq % H;
    const int b = seq / H;
    const int lane = threadIdx.x;
    const size_t xb = (size_t)seq * N;
    const size_t ub = (size_t)seq * T;

    float2 qd[NPL][RK], pa[NPL][RK], dv[NPL], cc[NPL], bb[NPL], xs[NPL];
    const int st = channel_setup<NPL, RK>(h, N, lane, Lambda, P, Q, Bv, C, dt, sm, qd, pa, dv, cc, bb);
    if (st != SSM_ST_OK) {
        fail_sequence(lane, N, T, ub, xb, y, x);
        if (lane == 0 && b == 0 && status) status[h] = st;
        return;
    }
    const int s = sm.s;
    int zs[NPL], zl[kMaxRank], ze[kMaxRank];
    z_slots<NPL>(lane, s, sm.zidx, zs, zl, ze);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        xs[e] = j < N ? x[xb + j] : make_float2(0.0f, 0.0f);
    }
    const float Dh = D ? D[h] : 0.0f;

    // ---- the recurrence (float32) ----
    // channels with no zero d_j (the usual case) take the Woodbury form, whose
    // r x r inverse stays in registers; the bordered form re-reads its order
    // r + s inverse from LDS every step
    float u0, u1;
    first_inputs<kWave>(u, ub, T, lane, u0, u1);
    if (s == 0)
        recur<NPL, RK, 0>(T, lane, ub, RK + s, sm.Mbf, zl, ze, qd, pa, dv, cc, bb, zs, Dh, u0, u1, u, y, xs);
    else
        recur<NPL, RK, kMaxRank>(T, lane, ub, RK + s, sm.Mbf, zl, ze, qd, pa, dv, cc, bb, zs, Dh, u0, u1, u, y, xs);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        if (j < N) x[xb + j] = xs[e];
    }
    if (lane == 0 && b == 0 && status) status[h] = SSM_ST_OK;
}

// ---- prepared constants ----
// One block of step_prepared_channel_bytes(N, r) bytes per channel:
//   int32[16] header: magic, N, r, status, s, zidx[4], zeros;
//   float2[kMaxOrder^2] Mb^{-1} (zero outside the order r + s block);
//   float2 arrays of 64 NPL slots each (state j at slot j, zero past N):
//   d^{-1}, conj(C), Bbar, then Q^* D^{-1} and alpha D^{-1} P column by column.
// The set-up writes them once per parameter set; the recurrence then reads
// the same float32 values its one-call form keeps in registers.
constexpr int32_t kPrepMagic = 0x50534d53;
constexpr int kPrepHeaderWords = 16;
constexpr size_t kPrepConstOffset = kPrepHeaderWords * 4 + kMaxOrder * kMaxOrder * sizeof(float2);

template <int NPL, int RK>
__global__ __launch_bounds__(kWave) void step_prepare_kernel(int N, const float2* __restrict__ Lambda,
                                                             const float2* __restrict__ P,
                                                             const float2* __restrict__ Q,
                                                             const float2* __restrict__ Bv,
                                                             const float2* __restrict__ C,
                                                             const float* __restrict__ dt, uint8_t* __restrict__ prep,
                                                             size_t chan_bytes, int32_t* __restrict__ status) {
    __shared__ StepSetup sm;
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    float2 qd[NPL][RK], pa[NPL][RK], dv[NPL], cc[NPL], bb[NPL];
    const int st = channel_setup<NPL, RK>(h, N, lane, Lambda, P, Q, Bv, C, dt, sm, qd, pa, dv, cc, bb);
    uint8_t* base = prep + (size_t)h * chan_bytes;
    const int s = st == SSM_ST_OK ? sm.s : 0;
    if (lane < kPrepHeaderWords) {
        int32_t w = 0;
        if (lane == 0) w = kPrepMagic;
        if (lane == 1) w = N;
        if (lane == 2) w = RK;
        if (lane == 3) w = st;
        if (lane == 4) w = s;
        if (lane >= 5 && lane < 5 + kMaxRank && lane - 5 < s) w = sm.zidx[lane - 5];
        reinterpret_cast<int32_t*>(base)[lane] = w;
    }
    if (lane == 0 && status) status[h] = st;
    if (st != SSM_ST_OK) return;
    {  // kMaxOrder^2 = 64 entries, one per lane
        const int i = lane / kMaxOrder, j = lane % kMaxOrder, n = RK + s;
        reinterpret_cast<float2*>(base + kPrepHeaderWords * 4)[lane] =
            i < n && j < n ? sm.Mbf[lane] : make_float2(0.0f, 0.0f);
    }
    float2* cst = reinterpret_cast<float2*>(base + kPrepConstOffset);
    constexpr int NS = NPL * kWave;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        cst[j] = dv[e];
        cst[NS + j] = cc[e];
        cst[2 * NS + j] = bb[e];
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            cst[(3 + a) * NS + j] = qd[e][a];
            cst[(3 + RK + a) * NS + j] = pa[e][a];
        }
    }
}

template <int NPL, int RK>
__global__ __launch_bounds__(kWave) void step_prepared_kernel(int Bsz, int H, int N, int T,
                                                              const uint8_t* __restrict__ prep, size_t chan_bytes,
                                                              const float* __restrict__ D,
                                                              const float* __restrict__ u, float* __restrict__ y,
                                                              float2* __restrict__ x, int32_t* __restrict__ status) {
    __shared__ float2 mbf[kMaxOrder * kMaxOrder];
    const int seq = blockIdx.x;  // = b * H + h
    const int h = seq % H;
    const int b = seq / H;
    const int lane = threadIdx.x;
    const size_t xb = (size_t)seq * N;
    const size_t ub = (size_t)seq * T;
    const uint8_t* base = prep + (size_t)h * chan_bytes;
    const int32_t* hd = reinterpret_cast<const int32_t*>(base);
    // every load is issued before the header is looked at (the block, the
    // state and the inputs are in bounds whatever it holds), so that a short
    // call waits for one memory round trip instead of two
    float u0, u1;
    first_inputs<kWave>(u, ub, T, lane, u0, u1);
    const float2 mbv = reinterpret_cast<const float2*>(base + kPrepHeaderWords * 4)[lane];
    const float2* cst = reinterpret_cast<const float2*>(base + kPrepConstOffset);
    constexpr int NS = NPL * kWave;
    float2 qd[NPL][RK], pa[NPL][RK], dv[NPL], cc[NPL], bb[NPL], xs[NPL];
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        dv[e] = cst[j];
        cc[e] = cst[NS + j];
        bb[e] = cst[2 * NS + j];
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            qd[e][a] = cst[(3 + a) * NS + j];
            pa[e][a] = cst[(3 + RK + a) * NS + j];
        }
        xs[e] = j < N ? x[xb + j] : make_float2(0.0f, 0.0f);
    }
    const float Dh = D ? D[h] : 0.0f;
    int st = hd[3];
    if (hd[0] != kPrepMagic || hd[1] != N || hd[2] != RK) st = SSM_ST_UNPREPARED;
    if (st != SSM_ST_OK) {
        fail_sequence(lane, N, T, ub, xb, y, x);
        if (lane == 0 && b == 0 && status) status[h] = st;
        return;
    }
    const int s = min(max(hd[4], 0), RK);
    int zidx[kMaxRank];
#pragma unroll
    for (int zz = 0; zz < kMaxRank; ++zz) zidx[zz] = min(max(hd[5 + zz], 0), NPL * kWave - 1);
    mbf[lane] = mbv;
    int zs[NPL], zl[kMaxRank], ze[kMaxRank];
    z_slots<NPL>(lane, s, zidx, zs, zl, ze);
    __syncthreads();
    if (s == 0)
        recur<NPL, RK, 0>(T, lane, ub, RK + s, mbf, zl, ze, qd, pa, dv, cc, bb, zs, Dh, u0, u1, u, y, xs);
    else
        recur<NPL, RK, kMaxRank>(T, lane, ub, RK + s, mbf, zl, ze, qd, pa, dv, cc, bb, zs, Dh, u0, u1, u, y, xs);
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
        const int j = lane + kWave * e;
        if (j < N) x[xb + j] = xs[e];
    }
    if (lane == 0 && b == 0 && status) status[h] = SSM_ST_OK;
}

// ---- 16-lane groups (N <= 64): four sequences per wave ----
// Lane g of group q holds states g + 16 e (e < S) of sequence 4 w + q.  The
// per-step sums then reduce within a row of 16 lanes (four DPP stages, after
// which every lane of the row holds the sum), with no cross-row combine and
// no scalar round trip; a wave issues about as many instructions per step as
// the one-sequence wave but for four sequences.
constexpr int kGroup = 16;

template <int K>
__device__ __forceinline__ void row_allsum(float (&v)[K]) {
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0xB1>(v[i]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x4E>(v[i]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x141>(v[i]);  // row_half_mirror
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get<0x140>(v[i]);  // row_mirror
}

// value of lane (own group, index k) for every lane
__device__ __forceinline__ float group_read(float v, int lane, int k) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane & ~(kGroup - 1)) | k) << 2, __float_as_int(v)));
}

// T steps of one group's sequence from xs (updated in place).  NZ: room for
// the bordered form's states in Z (0: Woodbury form; the whole wave takes
// the bordered loop when any of its groups needs it).  Mbf: the group's
// order r + s inverse (row stride kMaxOrder); n = r + s of the group.
// store: this group writes its outputs.
template <int S, int RK, int NZ>
__device__ __forceinline__ void recur16(int T, int g, int lane, size_t ub, int n, const float2* Mbf,
                                        const int (&zl)[kMaxRank], const int (&ze)[kMaxRank],
                                        const float2 (&qd)[S][RK], const float2 (&pa)[S][RK], const float2 (&dv)[S],
                                        const float2 (&cc)[S], const float2 (&bb)[S], const int (&zs)[S], float Dh,
                                        bool store, float ucur, float unext, const float* __restrict__ u,
                                        float* __restrict__ y, float2 (&xs)[S]) {
    constexpr int NO = RK + NZ;
    float2 Mr[NZ == 0 ? RK : 1][NZ == 0 ? RK : 1];
    if constexpr (NZ == 0) {
#pragma unroll
        for (int i = 0; i < RK; ++i)
#pragma unroll
            for (int j = 0; j < RK; ++j) Mr[i][j] = Mbf[i * kMaxOrder + j];
    }
    // ucur, unext: inputs of steps [0, 16) and [16, 32) (lane g holds step
    // t0 + g), loaded by the caller; indexes past the end hold the last
    // input (never used)
    float yblk = 0.0f;
    float uprev = 0.0f;
    for (int t = 0; t <= T; ++t) {
        const int k = t & (kGroup - 1);
        const float ut = group_read(ucur, lane, k);  // needed only at the end of the step
        // the lane's partial sums, seeded with its first state's terms
        float2 sq[RK];
        float scr = c_fma_re(cc[0], xs[0], 0.0f);
#pragma unroll
        for (int a = 0; a < RK; ++a) sq[a] = c_mul(qd[0][a], xs[0]);
#pragma unroll
        for (int e = 1; e < S; ++e) {
#pragma unroll
            for (int a = 0; a < RK; ++a) sq[a] = c_fma(qd[e][a], xs[e], sq[a]);
            scr = c_fma_re(cc[e], xs[e], scr);
        }
        {
            float v[2 * RK + 1];
#pragma unroll
            for (int a = 0; a < RK; ++a) {
                v[2 * a] = sq[a].x;
                v[2 * a + 1] = sq[a].y;
            }
            v[2 * RK] = scr;
            row_allsum<2 * RK + 1>(v);
#pragma unroll
            for (int a = 0; a < RK; ++a) sq[a] = make_float2(v[2 * a], v[2 * a + 1]);
            scr = v[2 * RK];
        }
        if (t > 0) {  // y_{t-1} = Re(C^* x_{t-1}) + D u_{t-1}
            const int kp = (t - 1) & (kGroup - 1);
            if (g == kp) yblk = scr + Dh * uprev;
            if (kp == kGroup - 1 || t == T) {
                const int t0 = (t - 1) & ~(kGroup - 1);
                if (store && t0 + g < T) y[ub + t0 + g] = yblk;
            }
        }
        if (t == T) break;
        if (k == kGroup - 1) {  // next block of inputs, for step t + 1
            ucur = unext;
            unext = u[ub + min(t + 1 + kGroup + g, T - 1)];
        }
        float2 sol[NO];
        if constexpr (NZ == 0) {
#pragma unroll
            for (int i = 0; i < RK; ++i) {
                float2 acc = c_mul(Mr[i][0], sq[0]);
#pragma unroll
                for (int j = 1; j < RK; ++j) acc = c_fma(Mr[i][j], sq[j], acc);
                sol[i] = acc;
            }
        } else {
            float2 rhs[NO];
#pragma unroll
            for (int a = 0; a < RK; ++a) rhs[a] = sq[a];
#pragma unroll
            for (int zz = 0; zz < NZ; ++zz) {
                float2 v = xs[0];
#pragma unroll
                for (int e = 1; e < S; ++e)
                    if (ze[zz] == e) v = xs[e];
                v = make_float2(group_read(v.x, lane, zl[zz]), group_read(v.y, lane, zl[zz]));
                rhs[RK + zz] = RK + zz < n ? v : make_float2(0.0f, 0.0f);
            }
            int off = 0;
            asm volatile("" : "+v"(off));
#pragma unroll
            for (int i = 0; i < NO; ++i) {
                float2 acc = make_float2(0.0f, 0.0f);
                if (i < n) {
#pragma unroll
                    for (int j = 0; j < NO; ++j)
                        if (j < n) acc = c_add(acc, c_mul(Mbf[off + i * kMaxOrder + j], rhs[j]));
                }
                sol[i] = acc;
            }
        }
#pragma unroll
        for (int e = 0; e < S; ++e) {
            float2 gv = c_mul(dv[e], xs[e]);
#pragma unroll
            for (int a = 0; a < RK; ++a) gv = c_fnma(pa[e][a], sol[a], gv);
            if constexpr (NZ > 0) {
#pragma unroll
                for (int zz = 0; zz < NZ; ++zz)
                    if (zs[e] == zz) gv = sol[RK + zz];
            }
            xs[e] = make_float2(2.0f * gv.x - xs[e].x + bb[e].x * ut, 2.0f * gv.y - xs[e].y + bb[e].y * ut);
        }
        uprev = ut;
    }
}

// One group's sequence from its channel's constants: cst holds the 64-slot
// arrays of the prepared layout (d^{-1}, conj C, Bbar, Q^* D^{-1}, alpha
// D^{-1} P), mbq the order r + s inverse (in LDS, written by the caller;
// this routine meets the barrier after its own loads), st, s_in and zin the
// channel's status, |Z| and Z.  A group past the end (live false) runs
// along without storing.  Every lane of the wave must call it together (the
// sums are row-wise DPP, the choice of loop wave-uniform).
template <int S, int RK>
__device__ __forceinline__ void group_sequence(int T, int N, int g, int lane, bool live, int st, int s_in,
                                               const int (&zin)[kMaxRank], const float2* mbq, const float2* cst,
                                               float Dh, size_t ub, size_t xb, int32_t* status_slot,
                                               float u0, float u1, const float* __restrict__ u,
                                               float* __restrict__ y, float2* __restrict__ x) {
    const bool ok = st == SSM_ST_OK;
    // constants of states g + 16 e (zero past N), all zero for a failing
    // group so that it runs the loop harmlessly; loaded whatever the status
    // (in bounds either way) and selected after
    constexpr int NS = kWave;
    const float2 zero = make_float2(0.0f, 0.0f);
    float2 qd[S][RK], pa[S][RK], dv[S], cc[S], bb[S], xs[S];
#pragma unroll
    for (int e = 0; e < S; ++e) {
        const int j = g + kGroup * e;
        dv[e] = cst[j];
        cc[e] = cst[NS + j];
        bb[e] = cst[2 * NS + j];
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            qd[e][a] = cst[(3 + a) * NS + j];
            pa[e][a] = cst[(3 + RK + a) * NS + j];
        }
        xs[e] = j < N ? x[xb + j] : zero;
    }
    if (!ok) {
#pragma unroll
        for (int e = 0; e < S; ++e) {
            dv[e] = cc[e] = bb[e] = xs[e] = zero;
#pragma unroll
            for (int a = 0; a < RK; ++a) qd[e][a] = pa[e][a] = zero;
        }
    }
    if (live && !ok) {  // NaN outputs now; the loop below stores nothing for this group
        const float nanf = __builtin_nanf("");
        for (int t = g; t < T; t += kGroup) y[ub + t] = nanf;
        for (int j = g; j < N; j += kGroup) x[xb + j] = c_nan();
    }
    if (g == 0 && status_slot) *status_slot = st;
    const int s = ok ? min(max(s_in, 0), RK) : 0;
    int zidx[kMaxRank];
#pragma unroll
    for (int zz = 0; zz < kMaxRank; ++zz) zidx[zz] = min(max(zin[zz], 0), S * kGroup - 1);
    int zs[S], zl[kMaxRank], ze[kMaxRank];
#pragma unroll
    for (int e = 0; e < S; ++e) {
        const int j = g + kGroup * e;
        zs[e] = -1;
        for (int zz = 0; zz < s; ++zz)
            if (zidx[zz] == j) zs[e] = zz;
    }
#pragma unroll
    for (int zz = 0; zz < kMaxRank; ++zz) {
        const int j = zz < s ? zidx[zz] : 0;
        zl[zz] = j % kGroup;
        ze[zz] = j / kGroup;
    }
    const bool store = live && ok;
    __syncthreads();  // mbq (written by the caller) is complete
    if (__ballot(s > 0) == 0)
        recur16<S, RK, 0>(T, g, lane, ub, RK + s, mbq, zl, ze, qd, pa, dv, cc, bb, zs, Dh, store, u0, u1, u, y,
                          xs);
    else
        recur16<S, RK, kMaxRank>(T, g, lane, ub, RK + s, mbq, zl, ze, qd, pa, dv, cc, bb, zs, Dh, store, u0, u1, u,
                                 y, xs);
    if (store) {
#pragma unroll
        for (int e = 0; e < S; ++e) {
            const int j = g + kGroup * e;
            if (j < N) x[xb + j] = xs[e];
        }
    }
}

// the group's sequence index, clamped to the last one past the end
struct GroupSeq {
    int seq, h, b;
    bool live;
    __device__ GroupSeq(int wave, int q, int nseq, int H) {
        const int raw = wave * (kWave / kGroup) + q;
        live = raw < nseq;
        seq = live ? raw : nseq - 1;
        h = seq % H;
        b = seq / H;
    }
};

template <int S, int RK>
__global__ __launch_bounds__(kWave) void step_prepared16_kernel(int nseq, int H, int N, int T,
                                                                const uint8_t* __restrict__ prep, size_t chan_bytes,
                                                                const float* __restrict__ D,
                                                                const float* __restrict__ u, float* __restrict__ y,
                                                                float2* __restrict__ x,
                                                                int32_t* __restrict__ status) {
    constexpr int kGroups = kWave / kGroup;
    __shared__ float2 mbf[kGroups][kMaxOrder * kMaxOrder];
    const int lane = threadIdx.x;
    const int q = lane / kGroup, g = lane % kGroup;
    const GroupSeq gs(blockIdx.x, q, nseq, H);
    float u0, u1;
    first_inputs<kGroup>(u, (size_t)gs.seq * T, T, g, u0, u1);
    const uint8_t* base = prep + (size_t)gs.h * chan_bytes;
    const int32_t* hd = reinterpret_cast<const int32_t*>(base);
    int st = hd[3];
    if (hd[0] != kPrepMagic || hd[1] != N || hd[2] != RK) st = SSM_ST_UNPREPARED;
    int zin[kMaxRank];
#pragma unroll
    for (int zz = 0; zz < kMaxRank; ++zz) zin[zz] = hd[5 + zz];
    const float2* mb = reinterpret_cast<const float2*>(base + kPrepHeaderWords * 4);
#pragma unroll
    for (int i = 0; i < kMaxOrder * kMaxOrder / kGroup; ++i) {
        const float2 v = mb[g + kGroup * i];
        mbf[q][g + kGroup * i] = st == SSM_ST_OK ? v : make_float2(0.0f, 0.0f);
    }
    group_sequence<S, RK>(T, N, g, lane, gs.live, st, hd[4], zin, mbf[q],
                          reinterpret_cast<const float2*>(base + kPrepConstOffset), D ? D[gs.h] : 0.0f,
                          (size_t)gs.seq * T, (size_t)gs.seq * N,
                          gs.live && gs.b == 0 && status ? status + gs.h : nullptr, u0, u1, u, y, x);
}

// ssm_step in 16-lane groups: the wave runs the float64 set-up of its four
// sequences' channels one after another (the one-wave set-up, N <= 64),
// leaves the constants in LDS in the prepared layout, then each group runs
// its sequence exactly as the prepared kernel does (the same values, bit for
// bit, as ssm_step_prepare + ssm_step_prepared in this layout).
template <int S, int RK>
__global__ __launch_bounds__(kWave) void step16_kernel(int nseq, int H, int N, int T,
                                                       const float2* __restrict__ Lambda,
                                                       const float2* __restrict__ P, const float2* __restrict__ Q,
                                                       const float2* __restrict__ Bv, const float2* __restrict__ C,
                                                       const float* __restrict__ dt, const float* __restrict__ D,
                                                       const float* __restrict__ u, float* __restrict__ y,
                                                       float2* __restrict__ x, int32_t* __restrict__ status) {
    constexpr int kGroups = kWave / kGroup;
    constexpr int NS = kWave;
    __shared__ StepSetup sm;
    __shared__ float2 cstl[kGroups][(3 + 2 * RK) * NS];
    __shared__ float2 mbl[kGroups][kMaxOrder * kMaxOrder];
    __shared__ int hdl[kGroups][2 + kMaxRank];
    const int lane = threadIdx.x;
    const float2 zero = make_float2(0.0f, 0.0f);
    for (int qq = 0; qq < kGroups; ++qq) {
        const GroupSeq gq(blockIdx.x, qq, nseq, H);
        float2 qd[1][RK], pa[1][RK], dv[1], cc[1], bb[1];
        const int stq = channel_setup<1, RK>(gq.h, N, lane, Lambda, P, Q, Bv, C, dt, sm, qd, pa, dv, cc, bb);
        const bool okq = stq == SSM_ST_OK;
        const int sq = okq ? sm.s : 0;
        cstl[qq][lane] = okq ? dv[0] : zero;
        cstl[qq][NS + lane] = okq ? cc[0] : zero;
        cstl[qq][2 * NS + lane] = okq ? bb[0] : zero;
#pragma unroll
        for (int a = 0; a < RK; ++a) {
            cstl[qq][(3 + a) * NS + lane] = okq ? qd[0][a] : zero;
            cstl[qq][(3 + RK + a) * NS + lane] = okq ? pa[0][a] : zero;
        }
        {
            const int i = lane / kMaxOrder, j = lane % kMaxOrder, n = RK + sq;
            mbl[qq][lane] = okq && i < n && j < n ? sm.Mbf[lane] : zero;
        }
        if (lane == 0) {
            hdl[qq][0] = stq;
            hdl[qq][1] = sq;
            for (int zz = 0; zz < kMaxRank; ++zz) hdl[qq][2 + zz] = zz < sq ? sm.zidx[zz] : 0;
        }
        __syncthreads();  // the next set-up reuses sm
    }
    const int q = lane / kGroup, g = lane % kGroup;
    const GroupSeq gs(blockIdx.x, q, nseq, H);
    float u0, u1;
    first_inputs<kGroup>(u, (size_t)gs.seq * T, T, g, u0, u1);
    int zin[kMaxRank];
#pragma unroll
    for (int zz = 0; zz < kMaxRank; ++zz) zin[zz] = hdl[q][2 + zz];
    group_sequence<S, RK>(T, N, g, lane, gs.live, hdl[q][0], hdl[q][1], zin, mbl[q], cstl[q],
                          D ? D[gs.h] : 0.0f, (size_t)gs.seq * T, (size_t)gs.seq * N,
                          gs.live && gs.b == 0 && status ? status + gs.h : nullptr, u0, u1, u, y, x);
}

template <int S>
hipError_t launch_step16(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const float2* Lambda,
                         const float2* P, const float2* Q, const float2* Bv, const float2* C, const float* dt,
                         const float* D, const float* u, float* y, float2* x, int32_t* status, hipStream_t stream) {
    const int64_t nseq = Bsz * H;
    const unsigned waves = (unsigned)((nseq + kWave / kGroup - 1) / (kWave / kGroup));
#define SSM_STEP16(RK)                                                                                           \
    if (r == RK) {                                                                                               \
        hipLaunchKernelGGL((step16_kernel<S, RK>), dim3(waves), dim3(kWave), 0, stream, (int)nseq, (int)H,       \
                           (int)N, (int)T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status);                         \
        return hipGetLastError();                                                                                \
    }
    SSM_STEP16(1) SSM_STEP16(2) SSM_STEP16(3) SSM_STEP16(4)
#undef SSM_STEP16
    return hipErrorInvalidValue;
}

template <int S>
hipError_t launch_prepared16(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const uint8_t* prep,
                             size_t chan_bytes, const float* D, const float* u, float* y, float2* x, int32_t* status,
                             hipStream_t stream) {
    const int64_t nseq = Bsz * H;
    const unsigned waves = (unsigned)((nseq + kWave / kGroup - 1) / (kWave / kGroup));
#define SSM_PREPD16(RK)                                                                                          \
    if (r == RK) {                                                                                               \
        hipLaunchKernelGGL((step_prepared16_kernel<S, RK>), dim3(waves), dim3(kWave), 0, stream, (int)nseq,      \
                           (int)H, (int)N, (int)T, prep, chan_bytes, D, u, y, x, status);                        \
        return hipGetLastError();                                                                                \
    }
    SSM_PREPD16(1) SSM_PREPD16(2) SSM_PREPD16(3) SSM_PREPD16(4)
#undef SSM_PREPD16
    return hipErrorInvalidValue;
}

template <int NPL>
hipError_t launch_npl(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const float2* Lambda,
                      const float2* P, const float2* Q, const float2* Bv, const float2* C, const float* dt,
                      const float* D, const float* u, float* y, float2* x, int32_t* status, hipStream_t stream) {
#define SSM_STEP(RK)                                                                                             \
    if (r == RK) {                                                                                               \
        hipLaunchKernelGGL((step_kernel<NPL, RK>), dim3((unsigned)(Bsz * H)), dim3(kWave), 0, stream, (int)Bsz,   \
                           (int)H, (int)N, (int)T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status);                 \
        return hipGetLastError();                                                                                \
    }
    SSM_STEP(1) SSM_STEP(2) SSM_STEP(3) SSM_STEP(4)
#undef SSM_STEP
    return hipErrorInvalidValue;
}

template <int NPL>
hipError_t launch_prepare_npl(int64_t H, int64_t N, int64_t r, const float2* Lambda, const float2* P, const float2* Q,
                              const float2* Bv, const float2* C, const float* dt, uint8_t* prep, size_t chan_bytes,
                              int32_t* status, hipStream_t stream) {
#define SSM_PREP(RK)                                                                                             \
    if (r == RK) {                                                                                               \
        hipLaunchKernelGGL((step_prepare_kernel<NPL, RK>), dim3((unsigned)H), dim3(kWave), 0, stream, (int)N,    \
                           Lambda, P, Q, Bv, C, dt, prep, chan_bytes, status);                                   \
        return hipGetLastError();                                                                                \
    }
    SSM_PREP(1) SSM_PREP(2) SSM_PREP(3) SSM_PREP(4)
#undef SSM_PREP
    return hipErrorInvalidValue;
}

template <int NPL>
hipError_t launch_prepared_npl(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const uint8_t* prep,
                               size_t chan_bytes, const float* D, const float* u, float* y, float2* x,
                               int32_t* status, hipStream_t stream) {
#define SSM_PREPD(RK)                                                                                            \
    if (r == RK) {                                                                                               \
        hipLaunchKernelGGL((step_prepared_kernel<NPL, RK>), dim3((unsigned)(Bsz * H)), dim3(kWave), 0, stream,   \
                           (int)Bsz, (int)H, (int)N, (int)T, prep, chan_bytes, D, u, y, x, status);              \
        return hipGetLastError();                                                                                \
    }
    SSM_PREPD(1) SSM_PREPD(2) SSM_PREPD(3) SSM_PREPD(4)
#undef SSM_PREPD
    return hipErrorInvalidValue;
}

}  // namespace

constexpr int64_t kStepMaxN = 4 * kWave;

// lanes: 16 (N <= 64: four sequences per wave) or 64 (one per wave)
hipError_t launch_step(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const float2* Lambda,
                       const float2* P, const float2* Q, const float2* Bv, const float2* C, const float* dt,
                       const float* D, const float* u, float* y, float2* x, int32_t* status, int lanes,
                       hipStream_t stream) {
    if (lanes == kGroup) {
        if (N <= kGroup) return launch_step16<1>(Bsz, H, N, r, T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status, stream);
        if (N <= 2 * kGroup)
            return launch_step16<2>(Bsz, H, N, r, T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status, stream);
        if (N <= kWave) return launch_step16<4>(Bsz, H, N, r, T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status, stream);
        return hipErrorInvalidValue;
    }
    if (N <= kWave) return launch_npl<1>(Bsz, H, N, r, T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status, stream);
    if (N <= 2 * kWave) return launch_npl<2>(Bsz, H, N, r, T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status, stream);
    if (N <= kStepMaxN) return launch_npl<4>(Bsz, H, N, r, T, Lambda, P, Q, Bv, C, dt, D, u, y, x, status, stream);
    return hipErrorInvalidValue;
}

// Bytes of one channel's prepared constants (a multiple of 256)
size_t step_prepared_channel_bytes(int64_t N, int64_t r) {
    const int64_t npl = N <= kWave ? 1 : N <= 2 * kWave ? 2 : 4;
    const size_t raw = kPrepConstOffset + sizeof(float2) * (size_t)(npl * kWave) * (size_t)(3 + 2 * r);
    return (raw + 255) / 256 * 256;
}

hipError_t launch_step_prepare(int64_t H, int64_t N, int64_t r, const float2* Lambda, const float2* P,
                               const float2* Q, const float2* Bv, const float2* C, const float* dt, uint8_t* prep,
                               int32_t* status, hipStream_t stream) {
    const size_t cb = step_prepared_channel_bytes(N, r);
    if (N <= kWave) return launch_prepare_npl<1>(H, N, r, Lambda, P, Q, Bv, C, dt, prep, cb, status, stream);
    if (N <= 2 * kWave) return launch_prepare_npl<2>(H, N, r, Lambda, P, Q, Bv, C, dt, prep, cb, status, stream);
    if (N <= kStepMaxN) return launch_prepare_npl<4>(H, N, r, Lambda, P, Q, Bv, C, dt, prep, cb, status, stream);
    return hipErrorInvalidValue;
}

// lanes: 16 (N <= 64: four sequences per wave) or 64 (one per wave)
hipError_t launch_step_prepared(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const uint8_t* prep,
                                const float* D, const float* u, float* y, float2* x, int32_t* status, int lanes,
                                hipStream_t stream) {
    const size_t cb = step_prepared_channel_bytes(N, r);
    if (lanes == kGroup) {
        if (N <= kGroup) return launch_prepared16<1>(Bsz, H, N, r, T, prep, cb, D, u, y, x, status, stream);
        if (N <= 2 * kGroup) return launch_prepared16<2>(Bsz, H, N, r, T, prep, cb, D, u, y, x, status, stream);
        if (N <= kWave) return launch_prepared16<4>(Bsz, H, N, r, T, prep, cb, D, u, y, x, status, stream);
        return hipErrorInvalidValue;
    }
    if (N <= kWave) return launch_prepared_npl<1>(Bsz, H, N, r, T, prep, cb, D, u, y, x, status, stream);
    if (N <= 2 * kWave) return launch_prepared_npl<2>(Bsz, H, N, r, T, prep, cb, D, u, y, x, status, stream);
    if (N <= kStepMaxN) return launch_prepared_npl<4>(Bsz, H, N, r, T, prep, cb, D, u, y, x, status, stream);
    return hipErrorInvalidValue;
}

}  // namespace ssm
