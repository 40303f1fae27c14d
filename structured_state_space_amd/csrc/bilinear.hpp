// Small float64 pieces of the bilinear discretisation shared by the
// discretisation and step kernels: a wavefront sum and the Gauss-Jordan
// inverse of the order-(r + s) matrix through which every solve with
// G = I - (dt/2) A runs.
//
// Source: "Recurrent, LSTM, and structured state-space models", DPLR block and
// the recurrent-solver passage of the Algorithm-1 block (Woodbury core
// I_r + alpha Q^* D^{-1} P when no d_j = 1 - alpha lambda_j is zero, else the
// bordered system when |Z| <= r).
#pragma once

#include "common.hpp"

namespace ssm {

constexpr int kWave = 64;
constexpr int kMaxOrder = 8;  // r + s <= 2 r <= 8

__device__ __forceinline__ double2 wave_sum(double2 v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        v.x += __shfl_xor(v.x, m, kWave);
        v.y += __shfl_xor(v.y, m, kWave);
    }
    return v;
}

// K float64 sums over the 64 lanes at once, returned to every lane: DPP
// exchanges of both 32-bit halves within each row of 16 lanes (quad_perm
// [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror), then the rows
// combined by the row broadcasts (lane 15 of rows 0 and 2 into rows 1 and 3,
// then lane 31 into rows 2 and 3; rows outside the mask add zero), and the
// total read from lane 63.  Stage by stage over the K values, so their
// exchanges fill each other's wait states.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_get_d(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xF, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}
template <int K>
__device__ __forceinline__ void wave_allsum_d(double (&v)[K]) {
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get_d<0xB1>(v[i]);
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get_d<0x4E>(v[i]);
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get_d<0x141>(v[i]);
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get_d<0x140>(v[i]);
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get_d<0x142, 0xA>(v[i]);  // row_bcast:15 into rows 1 and 3
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] += dpp_get_d<0x143, 0xC>(v[i]);  // row_bcast:31 into rows 2 and 3
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = readlane_d(v[i], 63);
}

__device__ __forceinline__ double z_abs1(double2 a) { return fabs(a.x) + fabs(a.y); }

// In-place Gauss-Jordan inverse of an n x n complex matrix in LDS (row stride
// kMaxOrder), run by one lane; false on an exactly zero pivot.
__device__ inline bool small_inverse(double2* A, double2* Inv, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) Inv[i * kMaxOrder + j] = make_double2(i == j ? 1.0 : 0.0, 0.0);
    for (int c = 0; c < n; ++c) {
        int piv = c;
        for (int r = c + 1; r < n; ++r)
            if (z_abs1(A[r * kMaxOrder + c]) > z_abs1(A[piv * kMaxOrder + c])) piv = r;
        if (z_is_zero(A[piv * kMaxOrder + c])) return false;
        if (piv != c)
            for (int j = 0; j < n; ++j) {
                double2 t = A[c * kMaxOrder + j];
                A[c * kMaxOrder + j] = A[piv * kMaxOrder + j];
                A[piv * kMaxOrder + j] = t;
                t = Inv[c * kMaxOrder + j];
                Inv[c * kMaxOrder + j] = Inv[piv * kMaxOrder + j];
                Inv[piv * kMaxOrder + j] = t;
            }
        const double2 pinv = z_inv(A[c * kMaxOrder + c]);
        for (int j = 0; j < n; ++j) {
            A[c * kMaxOrder + j] = z_mul(A[c * kMaxOrder + j], pinv);
            Inv[c * kMaxOrder + j] = z_mul(Inv[c * kMaxOrder + j], pinv);
        }
        for (int r = 0; r < n; ++r) {
            if (r == c) continue;
            const double2 f = A[r * kMaxOrder + c];
            for (int j = 0; j < n; ++j) {
                A[r * kMaxOrder + j] = z_sub(A[r * kMaxOrder + j], z_mul(f, A[c * kMaxOrder + j]));
                Inv[r * kMaxOrder + j] = z_sub(Inv[r * kMaxOrder + j], z_mul(f, Inv[c * kMaxOrder + j]));
            }
        }
    }
    return true;
}

}  // namespace ssm
