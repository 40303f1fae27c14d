// HiPPO generators to diagonal-plus-low-rank form, in float64 on the device.
//
// [RSS] "Recurrent, LSTM, and structured state-space models", block on the
// HiPPO generators (S4 Theorem 1, App. C.1; HiPPO sec. 2.3, App. D.1-D.3):
// the LegS, LegT and LagT matrices G, the similarity S (identity, or
// diag(sqrt(2n+1)) diag((-1)^n) for LegT), and the split of S^{-1} G S into a
// normal matrix minus a term of rank <= 2.  Block "DPLR structured state-space
// parameterization": a unitary state change V turns the normal part into the
// diagonal Lambda and B, C into V^* B, V^* C.
//
// The transformed matrix is (c I + K) - U U^T with K its skew-symmetric part,
// c = -1/2 (LegS, LagT) or 0 (LegT), and U the closed-form low-rank factor.
// Only K needs a spectral decomposition:
//   A  one workgroup reduces K to a skew tridiagonal T = Q^T K Q with
//      Householder reflections (a skew matrix stays skew, so each trailing
//      update is the rank-2 step A22 += tau (v p^T - p v^T), p = A22 v, and
//      p can be summed down columns: p = -A22^T v);
//   B  one workgroup per eigenvalue: with the unit diagonal d_{k+1} =
//      d_k i sign(T_{k+1,k}), D^* (i T) D is the real symmetric tridiagonal
//      with zero diagonal and off-diagonal |T_{k+1,k}|.  Its eigenvalue mu is
//      bracketed by Sturm counts (a multisection over the workgroup's
//      threads), its eigenvector y found by inverse iteration (LU with row
//      interchanges, in LDS); Q D y is then an eigenvector of K with
//      eigenvalue -i mu, formed with the reflections held across threads.
//      Each vector's phase makes (V^* U)_{j,0} real and non-negative;
//   C  B~ = V^* S^{-1} B and C~ = V^* S C for every input row.
// Eigenvalues come out by ascending imaginary part, Lambda_j = c - i mu_j.
#include <cfloat>

#include "bilinear.hpp"
#include "common.hpp"

namespace ssm {
namespace {

constexpr int kHippoMaxN = 1024;
constexpr int kLegS = 0, kLegT = 1, kLagT = 2;

__device__ __forceinline__ double neg_one_pow(int n) { return (n & 1) ? -1.0 : 1.0; }

// entry (n, k) of S^{-1} G S
__device__ double transformed_entry(int kind, int n, int k, double theta) {
    if (kind == kLegS) {
        if (n > k) return -sqrt((double)(2 * n + 1) * (double)(2 * k + 1));
        return n == k ? -(double)(n + 1) : 0.0;
    }
    if (kind == kLagT) return n >= k ? -1.0 : 0.0;
    // LegT: G_{nk} s_k / s_n with s_n = sqrt(2n+1) (-1)^n
    const double g = n >= k ? -(double)(2 * n + 1) * neg_one_pow(n - k) / theta : -(double)(2 * n + 1) / theta;
    return g * sqrt((double)(2 * k + 1) / (double)(2 * n + 1)) * neg_one_pow(n + k);
}

// column q of the low-rank factor U, entry n
__device__ double low_rank_entry(int kind, int q, int n, double theta) {
    if (kind == kLegS) return sqrt((double)n + 0.5);
    if (kind == kLagT) return sqrt(0.5);
    return (n & 1) == q ? sqrt((double)(2 * n + 1) / theta) : 0.0;
}

__device__ __forceinline__ double similarity_entry(int kind, int n) {
    return kind == kLegT ? sqrt((double)(2 * n + 1)) * neg_one_pow(n) : 1.0;
}

__device__ __forceinline__ double wave_sum(double v) {
    double a[1] = {v};
    wave_allsum_d<1>(a);  // DPP exchanges, no LDS round trip
    return a[0];
}

// sum over the workgroup, returned to every thread (two barriers)
__device__ double block_sum(double v, double* red) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    v = wave_sum(v);
    if (lane == 0) red[wv] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < nw; ++w) s += red[w];
    __syncthreads();
    return s;
}

__device__ double2 block_sum2(double2 v, double2* red) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    double a[2] = {v.x, v.y};
    wave_allsum_d<2>(a);
    v = make_double2(a[0], a[1]);
    if (lane == 0) red[wv] = v;
    __syncthreads();
    double2 s = make_double2(0.0, 0.0);
    for (int w = 0; w < nw; ++w) s = z_add(s, red[w]);
    __syncthreads();
    return s;
}

__device__ double block_max(double v, double* red) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    if (lane == 0) red[wv] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < nw; ++w) s = fmax(s, red[w]);
    __syncthreads();
    return s;
}

// ---- A: skew part and its Householder tridiagonalisation (one workgroup) ----
// K [N,N] row-major (overwritten), Vh [N,N]: row k holds reflection k on
// entries k+1 .. N-1 (entry k+1 is 1), e [N]: T_{k+1,k}, tau [N].
// Step k works on the trailing block of rows and columns k+1 .. N-1 (size m).
// Each thread owns one column c of it and a residue class of its rows, so
// every access to K is a coalesced row segment: the product uses skewness,
// p_c = (A22 v)_c = -sum_i A22[i][c] v_i, from per-class partial sums, and the
// rank-2 update touches the thread's own column.  The reflector is formed
// from row k (= -column k).  For N <= kHippoLdsN the matrix stays in LDS.
constexpr int kHippoLdsN = 64;

template <bool kInLds>
__global__ __launch_bounds__(1024) void hippo_tridiag_kernel(int kind, int N, double theta, double* __restrict__ K,
                                                             double* __restrict__ Vh, double* __restrict__ e,
                                                             double* __restrict__ tau) {
    __shared__ double v[kHippoMaxN];
    __shared__ double p[kHippoMaxN];
    __shared__ double part[1024];
    __shared__ double red[16];
    __shared__ double Kl[kInLds ? kHippoLdsN * kHippoLdsN : 1];
    double* const A = kInLds ? Kl : K;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;

    for (int n = wv; n < N; n += nw)
        for (int k = lane; k < N; k += 64)
            A[(size_t)n * N + k] = 0.5 * (transformed_entry(kind, n, k, theta) - transformed_entry(kind, k, n, theta));
    __syncthreads();

    for (int k = 0; k + 2 < N; ++k) {
        const int c0 = k + 1, m = N - c0;
        const int wc = (m + 63) & ~63, groups = (int)blockDim.x / wc;
        const int cl = tid % wc, g = tid / wc, c = c0 + cl;
        const bool own = g < groups && cl < m;
        // x_i = A[i][k] = -A[k][i], i >= k + 1
        double part_sq = 0.0;
        for (int i = c0 + 1 + tid; i < N; i += blockDim.x) {
            const double x = A[(size_t)k * N + i];
            part_sq += x * x;
        }
        const double sigma = block_sum(part_sq, red);
        const double alpha = -A[(size_t)k * N + c0];
        double beta = alpha, t = 0.0, scal = 0.0;
        if (sigma != 0.0) {
            const double nrm = sqrt(alpha * alpha + sigma);
            beta = alpha >= 0.0 ? -nrm : nrm;
            t = (beta - alpha) / beta;
            scal = -1.0 / (alpha - beta);
        }
        for (int i = c0 + tid; i < N; i += blockDim.x) {
            const double vi = i == c0 ? 1.0 : A[(size_t)k * N + i] * scal;
            v[i] = vi;
            Vh[(size_t)k * N + i] = vi;
        }
        if (tid == 0) {
            e[k] = beta;
            tau[k] = t;
        }
        __syncthreads();
        if (t == 0.0) continue;
        if (own) {  // partial of -(A22^T v)_c over rows i = c0 + g + groups q
            double sacc = 0.0;
            for (int i = c0 + g; i < N; i += groups) sacc += A[(size_t)i * N + c] * v[i];
            part[g * wc + cl] = sacc;
        }
        __syncthreads();
        if (own && g == 0) {
            double sacc = 0.0;
            for (int q = 0; q < groups; ++q) sacc += part[q * wc + cl];
            p[c] = -sacc;
        }
        __syncthreads();
        if (own) {  // A22 += t (v p^T - p v^T), column c
            const double tvc = t * v[c], tpc = t * p[c];
            for (int i = c0 + g; i < N; i += groups) A[(size_t)i * N + c] += v[i] * tpc - p[i] * tvc;
        }
        __syncthreads();
    }
    if (tid == 0 && N >= 2) {
        e[N - 2] = A[(size_t)(N - 1) * N + (N - 2)];
        tau[N - 2] = 0.0;
    }
}

// number of eigenvalues below x of the symmetric tridiagonal with zero
// diagonal and squared off-diagonal b2 (signs of the LDL^T pivots)
__device__ int sturm_count(double x, int N, const double* b2, double pivmin) {
    double q = -x;
    if (fabs(q) < pivmin) q = -pivmin;
    int c = q < 0.0;
    for (int i = 1; i < N; ++i) {
        q = -x - b2[i - 1] / q;
        if (fabs(q) < pivmin) q = -pivmin;
        c += q < 0.0;
    }
    return c;
}

// ---- B: one eigenpair per workgroup ----
__global__ __launch_bounds__(1024) void hippo_eigvec_kernel(int kind, int N, double theta, int rank,
                                                            const double* __restrict__ e,
                                                            const double* __restrict__ tau,
                                                            const double* __restrict__ Vh, double2* __restrict__ Vz,
                                                            float2* __restrict__ Lam, float2* __restrict__ Pout,
                                                            float2* __restrict__ Vout) {
    __shared__ double b2[kHippoMaxN];
    __shared__ double u0[kHippoMaxN], u1[kHippoMaxN], u2[kHippoMaxN], lm[kHippoMaxN], y[kHippoMaxN];
    __shared__ unsigned char piv[kHippoMaxN];
    __shared__ double red[16];
    __shared__ double2 red2[16];
    __shared__ int first;
    const int tid = threadIdx.x, T = blockDim.x;
    const int j = blockIdx.x;              // output index: ascending imaginary part
    const int rnk = N - 1 - j;             // rank of mu among the ascending eigenvalues

    // off-diagonal of the real tridiagonal; Gershgorin bound and pivot floor
    double g = 0.0, bb = 0.0;
    for (int i = tid; i < N; i += T) {
        const double lo_e = i > 0 ? fabs(e[i - 1]) : 0.0, hi_e = i < N - 1 ? fabs(e[i]) : 0.0;
        g = fmax(g, lo_e + hi_e);
        if (i < N - 1) {
            b2[i] = hi_e * hi_e;
            bb = fmax(bb, b2[i]);
        }
    }
    const double tnorm = block_max(g, red);
    const double pivmin = DBL_MIN * fmax(1.0, block_max(bb, red));

    double mu = 0.0;
    if (N > 1 && tnorm > 0.0) {
        double lo = -(tnorm * (1.0 + 4.0 * DBL_EPSILON) + pivmin), hi = -lo;
        for (int it = 0; it < 64; ++it) {
            const double w = hi - lo;
            if (w <= 2.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi)) || w <= DBL_EPSILON * tnorm) break;
            // T interior points; keep the step where the count first exceeds the rank
            const double x = lo + w * (double)(tid + 1) / (double)(T + 1);
            if (tid == 0) first = T;
            __syncthreads();
            if (sturm_count(x, N, b2, pivmin) > rnk) atomicMin(&first, tid);
            __syncthreads();
            const int f = first;
            const double nlo = f == 0 ? lo : lo + w * (double)f / (double)(T + 1);
            const double nhi = f == T ? hi : lo + w * (double)(f + 1) / (double)(T + 1);
            lo = nlo;
            hi = nhi;
            __syncthreads();
        }
        mu = 0.5 * (lo + hi);
    }

    // inverse iteration on (T_r - mu I) y = r, one thread, arrays in LDS
    if (tid == 0) {
        if (N == 1 || tnorm == 0.0) {
            for (int i = 0; i < N; ++i) y[i] = i == rnk ? 1.0 : 0.0;
        } else {
            const double floor_piv = DBL_EPSILON * tnorm;
            double dd = -mu, ee = sqrt(b2[0]);
            for (int i = 0; i + 1 < N; ++i) {
                const double c = sqrt(b2[i]), dn = -mu, en = i + 2 < N ? sqrt(b2[i + 1]) : 0.0;
                if (fabs(dd) >= fabs(c)) {
                    const double l = dd != 0.0 ? c / dd : 0.0;
                    u0[i] = dd; u1[i] = ee; u2[i] = 0.0; lm[i] = l; piv[i] = 0;
                    dd = dn - l * ee;
                    ee = en;
                } else {
                    const double l = dd / c;
                    u0[i] = c; u1[i] = dn; u2[i] = en; lm[i] = l; piv[i] = 1;
                    dd = ee - l * dn;
                    ee = -l * en;
                }
            }
            u0[N - 1] = dd;
            for (int i = 0; i < N; ++i) {  // floored pivots, kept as reciprocals for the solves
                if (fabs(u0[i]) < floor_piv) u0[i] = u0[i] < 0.0 ? -floor_piv : floor_piv;
                u0[i] = 1.0 / u0[i];
            }
            // start vector: a fixed low-discrepancy sequence in (-1, 1)
            for (int i = 0; i < N; ++i) {
                const double f = (double)(i + 1) * 0.6180339887498949 + (double)j * 0.7548776662466927;
                y[i] = 2.0 * (f - floor(f)) - 1.0;
            }
            for (int pass = 0; pass < 3; ++pass) {
                for (int i = 0; i + 1 < N; ++i) {
                    if (piv[i]) {
                        const double tmp = y[i];
                        y[i] = y[i + 1];
                        y[i + 1] = tmp;
                    }
                    y[i + 1] -= lm[i] * y[i];
                }
                y[N - 1] *= u0[N - 1];
                y[N - 2] = (y[N - 2] - u1[N - 2] * y[N - 1]) * u0[N - 2];
                for (int i = N - 3; i >= 0; --i) y[i] = (y[i] - u1[i] * y[i + 1] - u2[i] * y[i + 2]) * u0[i];
                double m = 0.0;
                for (int i = 0; i < N; ++i) m = fmax(m, fabs(y[i]));
                const double s = 1.0 / m;
                for (int i = 0; i < N; ++i) y[i] *= s;
            }
            double nn = 0.0;
            for (int i = 0; i < N; ++i) nn += y[i] * y[i];
            const double s = 1.0 / sqrt(nn);
            for (int i = 0; i < N; ++i) y[i] *= s;
        }
    }
    __syncthreads();

    // z = D y, then the reflections in reverse order: Q D y
    double2 z = make_double2(0.0, 0.0);
    if (tid < N) {
        int q = 0;
        for (int k = 0; k < tid; ++k) q += e[k] > 0.0 ? 1 : (e[k] < 0.0 ? 3 : 0);
        const double yi = y[tid];
        switch (q & 3) {
            case 0: z = make_double2(yi, 0.0); break;
            case 1: z = make_double2(0.0, yi); break;
            case 2: z = make_double2(-yi, 0.0); break;
            default: z = make_double2(0.0, -yi); break;
        }
    }
    // each reflection's entries are fetched one step ahead, so the load is in
    // flight during the previous step's sums
    double vnext = (N >= 3 && tid > N - 3 && tid < N) ? Vh[(size_t)(N - 3) * N + tid] : 0.0;
    for (int k = N - 3; k >= 0; --k) {
        const double t = tau[k];
        const double vi = vnext;
        vnext = (k > 0 && tid > k - 1 && tid < N) ? Vh[(size_t)(k - 1) * N + tid] : 0.0;
        if (t == 0.0) continue;
        const double2 s = block_sum2(z_scale(z, vi), red2);
        z = z_sub(z, z_scale(s, t * vi));
    }

    // phase: (V^* U)_{j,0} real and non-negative
    const double uq0 = tid < N ? low_rank_entry(kind, 0, tid, theta) : 0.0;
    const double2 p0 = block_sum2(z_scale(z_conj(z), uq0), red2);
    const double mag = sqrt(p0.x * p0.x + p0.y * p0.y);
    if (mag > 0.0) z = z_mul(z, z_scale(p0, 1.0 / mag));
    double2 p1 = make_double2(0.0, 0.0);
    if (rank > 1) {
        const double uq1 = tid < N ? low_rank_entry(kind, 1, tid, theta) : 0.0;
        p1 = block_sum2(z_scale(z_conj(z), uq1), red2);
    }
    if (tid < N) {
        Vz[(size_t)tid * N + j] = z;
        if (Vout) Vout[(size_t)tid * N + j] = c_from(z);
    }
    if (tid == 0) {
        const double c = kind == kLegT ? 0.0 : -0.5;
        Lam[j] = make_float2((float)c, (float)(-mu));
        Pout[(size_t)j * rank] = make_float2((float)mag, 0.0f);
        if (rank > 1) Pout[(size_t)j * rank + 1] = c_from(p1);
    }
}

// ---- C: out[v][j] = sum_n conj(V[n][j]) w_n x_v[n] ----
__global__ __launch_bounds__(64) void hippo_project_kernel(int kind, int N, int64_t nb, const float2* __restrict__ B,
                                                           const float2* __restrict__ C,
                                                           const double2* __restrict__ Vz, float2* __restrict__ Bt,
                                                           float2* __restrict__ Ct) {
    const int j = blockIdx.y * 64 + threadIdx.x;
    const int64_t row = blockIdx.x;
    if (j >= N) return;
    const bool is_b = row < nb;
    const float2* x = is_b ? B + row * N : C + (row - nb) * N;
    double2 acc = make_double2(0.0, 0.0);
    for (int n = 0; n < N; ++n) {
        const double s = similarity_entry(kind, n);
        const double2 xv = z_scale(z_from(x[n]), is_b ? 1.0 / s : s);
        acc = z_add(acc, z_mul(z_conj(Vz[(size_t)n * N + j]), xv));
    }
    float2* out = is_b ? Bt + row * N : Ct + (row - nb) * N;
    out[j] = c_from(acc);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct HippoWs {
    size_t K, Vh, e, tau, Vz, total;
};

HippoWs hippo_layout(int64_t N) {
    HippoWs w;
    size_t off = 0;
    w.K = off;
    off = align256(off + (size_t)N * N * sizeof(double));
    w.Vh = off;
    off = align256(off + (size_t)N * N * sizeof(double));
    w.e = off;
    off = align256(off + (size_t)N * sizeof(double));
    w.tau = off;
    off = align256(off + (size_t)N * sizeof(double));
    w.Vz = off;
    off = align256(off + (size_t)N * N * sizeof(double2));
    w.total = off;
    return w;
}

}  // namespace

int64_t hippo_max_n() { return kHippoMaxN; }

size_t hippo_workspace_bytes(int64_t N) { return hippo_layout(N).total; }

hipError_t launch_hippo(int kind, int64_t N, double theta, int64_t nb, const float2* B, int64_t nc, const float2* C,
                        float2* Lam, float2* P, float2* V, float2* Bt, float2* Ct, void* ws, hipStream_t stream) {
    const HippoWs w = hippo_layout(N);
    char* base = (char*)ws;
    double* K = (double*)(base + w.K);
    double* Vh = (double*)(base + w.Vh);
    double* e = (double*)(base + w.e);
    double* tau = (double*)(base + w.tau);
    double2* Vz = (double2*)(base + w.Vz);
    const int n = (int)N, rank = kind == kLegT ? 2 : 1;
    if (n <= kHippoLdsN)
        hipLaunchKernelGGL(hippo_tridiag_kernel<true>, dim3(1), dim3(1024), 0, stream, kind, n, theta, K, Vh, e, tau);
    else
        hipLaunchKernelGGL(hippo_tridiag_kernel<false>, dim3(1), dim3(1024), 0, stream, kind, n, theta, K, Vh, e, tau);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int threads = (int)((N + 63) / 64 * 64);
    hipLaunchKernelGGL(hippo_eigvec_kernel, dim3(n), dim3(threads), 0, stream, kind, n, theta, rank, e, tau, Vh, Vz,
                       Lam, P, V);
    err = hipGetLastError();
    if (err != hipSuccess || nb + nc == 0) return err;
    hipLaunchKernelGGL(hippo_project_kernel, dim3((unsigned)(nb + nc), (unsigned)((N + 63) / 64)), dim3(64), 0,
                       stream, kind, n, nb, B, C, Vz, Bt, Ct);
    return hipGetLastError();
}

}  // namespace ssm
