// Kernel spectra and long causal convolution for M = P Q > 16384 (P = 2 or 4,
// Q = 16384): one radix-P step across the whole length, then the
// wave-structured Q-point transforms (wfft.hpp).
//
// Sources: "Recurrent, LSTM, and structured state-space models" -- filter-mode
// block (the kernel is the first L coefficients of the inverse radix-two
// transform of the root values), DPLR block (y_t = C^* x_t + D u_t) and
// radix-two DFT block (an exact polynomial product by zero padding to a
// radix-two length >= 2n - 1; the transform of length P Q factored into P-point
// and Q-point transforms with twiddles).
//
// As for M <= 16384 the zero-padded product is taken modulo z^(2M) + 1 and
// split into the halves with twists psi^c, c = 1 and 3, psi_j = exp(-i pi j/(2M)).
// One half's transform, frequency P k2 + k1, is
//   X[P k2 + k1] = FFT_Q over q of  Y_k1[q] = w_4M^(q m) sum_p x[q + Q p] w_4P^(p m),
// m = c + 4 k1, w_n = exp(-2 pi i/n): the twist and the radix-P step fold into
// one sum of P inputs per output.  The inverse runs the same steps mirrored:
// Z_k1[q] = conj(w_4M^(q m)) IFFT_Q(X_k1 . S_k1)[q], and
//   y[q + Q p] = sum over c and k1 of Z[c][k1][q] conj(w_4P^(p m)).
// The spectrum is stored per channel as [P][Q] (slice k1 in the Q-transform's
// scrambled order) for the half c = 1 only: for a real kernel the other half's
// slice k1 is the conjugate of slice P - 1 - k1 at the complemented positions.
//
// Launches (conv, per chunk of row pairs): wl_conv_a, one workgroup per (row
// pair, k1), the half c = 1 at slice k1 and the half c = 3 at slice P - 1 - k1
// (conjugate radix-P weights: one pass over the inputs serves both), writes Z;
// wl_conv_b combines Z into the output rows.
// Spectrum: wl_spec, one workgroup per (channel, k1), from the real kernel.
#include <type_traits>

#include "common.hpp"
#include "fft.hpp"
#include "wfft.hpp"

namespace ssm {

namespace {

constexpr int kLogQ = 14, kQ = 1 << kLogQ, kT = 1024;  // the inner transform
using GQ = WGeo<kLogQ>;

// w_4P^j = exp(-2 pi i j/(4P)) from the table tw4M[j'] = exp(-i pi j'/(2M)),
// j' < 2M: w_4P^j = tw4M[j M/P], and the upper half by negation
template <int LOGP>
__device__ __forceinline__ float2 root4p(const float2* tw4M, int j) {
    constexpr int P = 1 << LOGP, M = P * kQ;
    j &= 4 * P - 1;
    const float2 w = tw4M[(j & (2 * P - 1)) * (M / P)];
    return j >= 2 * P ? make_float2(-w.x, -w.y) : w;
}

// a i^k, exact (k folds to a constant in unrolled loops): conj(w_P^(p j)) =
// i^(4 p j/P) for P = 2 and 4
__device__ __forceinline__ float2 mul_ipow(float2 a, int k) {
    const float2 r = (k & 1) ? make_float2(-a.y, a.x) : a;
    return (k & 2) ? make_float2(-r.x, -r.y) : r;
}

// The kernel transform from the root values (M = P Q): the root values are
// stored per channel as [P][Q] in the scrambled order (slice k1 holds the
// frequencies P k2 + k1 in the Q-transform's order).  One workgroup per
// (channel, k1): T_k1[q] = conj(w_M^(q k1)) sum_k2 H[P k2 + k1] conj(w_Q^(q k2)),
// natural q, written over the slice it was read from.  The channel status is
// reduced from the root-value kernel's tile statuses; a failing channel's
// slices become NaN (and so do its kernel, spectrum and outputs).
template <int LOGP>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(4))) void wl_kt_kernel(
    int tiles, float2* __restrict__ roots, const int32_t* __restrict__ tile_status, int32_t* __restrict__ status,
    const float2* __restrict__ tw4Q, const float2* __restrict__ tw4M, int remap) {
    constexpr int P = 1 << LOGP, M = P * kQ;
    __shared__ float2 lds[GQ::LDS];
    __shared__ int sst;
    int it = blockIdx.x;
    if (remap) {
        const int x = it & 7, s = it >> 3;
        it = ((s / P) * 8 + x) * P + s % P;
    }
    const int h = it >> LOGP, k1 = it & (P - 1);
    const int t = threadIdx.x;
    if (t == 0) sst = 0;
    __syncthreads();
    int mx = 0;
    for (int i = t; i < tiles; i += kT) mx = max(mx, tile_status[(size_t)h * tiles + i]);
    if (mx) atomicMax(&sst, mx);
    __syncthreads();
    const int st = sst;
    if (k1 == 0 && t == 0 && status) status[h] = st;
    const rsrc_t rr = make_rsrc(roots + (size_t)h * M + (size_t)k1 * kQ, kQ * sizeof(float2));
    const uint32_t vq = (uint32_t)t * sizeof(float2);
    if (st != 0) {  // uniform
#pragma unroll
        for (int e = 0; e < 16; ++e) buf_st_c64(c_nan(), rr, vq, kT * e * sizeof(float2));
        return;
    }
    const uint32_t vp = (uint32_t)wf_pos(t, 0) * sizeof(float2);
    float2 v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = buf_ld_c64(rr, vp, e * 64 * sizeof(float2));
    wf_inverse<kLogQ, 0>(v, lds, tw4Q, t);
    // conj(w_M^(q k1)), q = t + 1024 e: conj(w_4M^(4 t k1)) times conj(w_4M^(4096 k1))^e
    float2 tc = c_conj(tw4M[4 * t * k1]);
    const float2 sc = c_conj(tw4M[4 * kT * k1]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        buf_st_c64(c_mul(v[e], tc), rr, vq, kT * e * sizeof(float2));
        if (e < 15) {
            power_after(tc, v[e]);
            tc = c_mul(tc, sc);
        }
    }
}

// Spectrum of the real kernel k (taps >= L zero, D at tap 0), scaled 1/(2M),
// half c = 1: S[h][k1][pos] for the Q-transform's scrambled positions.
// FROM_T: k = Re K with K[q + Q p] = (1/M) sum_k1' conj(w_P^(p k1')) T_k1'[q] from
// wl_kt (the workgroup with k1 = 0 also writes K_out); otherwise Kin: K [H][L]
// with element stride kstride (1: real; 2: the real part of a complex kernel).
// grid H * P, 1024 threads.
template <int LOGP, bool FROM_T, bool FULL = false>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(4))) void wl_spec_kernel(
    int L, const float* __restrict__ Kin, int64_t kstride, const float2* __restrict__ Tin, const float* __restrict__ D,
    float2* __restrict__ K_out, float2* __restrict__ S, const float2* __restrict__ tw4Q,
    const float2* __restrict__ tw4M, int remap) {
    constexpr int P = 1 << LOGP, M = P * kQ;
    __shared__ float2 lds[GQ::LDS];
    int it = blockIdx.x;
    if (remap) {  // the P workgroups of a channel on one XCD: its kernel is read into that L2 once
        const int x = it & 7, s = it >> 3;
        it = ((s / P) * 8 + x) * P + s % P;
    }
    const int h = it >> LOGP, k1 = it & (P - 1);
    const int t = threadIdx.x;
    const int m = 1 + 4 * k1;
    const float sc = 1.0f / (float)(2 * M);
    float2 wp[P];
#pragma unroll
    for (int p = 0; p < P; ++p) wp[p] = root4p<LOGP>(tw4M, p * m);
    const float2 base = tw4M[t * m], step = tw4M[kT * m];  // w_4M^(t m), w_4M^(1024 m)
    const float dv = D ? D[h] : 0.0f;
    float2 v[16];
    float2 tw = base;
    if constexpr (FROM_T) {
        const rsrc_t rt = make_rsrc(Tin + (size_t)h * M, M * sizeof(float2));
        const uint32_t vq = (uint32_t)t * sizeof(float2);
        const float invM = 1.0f / (float)M;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int q = t + kT * e;
            float2 tk[P];
#pragma unroll
            for (int j = 0; j < P; ++j) tk[j] = buf_ld_c64(rt, vq, (kQ * j + kT * e) * sizeof(float2));
            float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                float2 kv = make_float2(0.0f, 0.0f);
#pragma unroll
                for (int j = 0; j < P; ++j) kv = c_add(kv, mul_ipow(tk[j], (p * j) << (2 - LOGP)));
                kv = c_scale(kv, invM);
                const int n = q + kQ * p;
                if (K_out && k1 == 0 && n < L) K_out[(size_t)h * L + n] = kv;
                float kr = n < L ? kv.x : 0.0f;
                if (n == 0) kr += dv;
                acc = c_add(acc, c_scale(wp[p], kr * sc));
            }
            v[e] = c_mul(acc, tw);
            if (e < 15) {
                power_after(tw, v[e]);
                tw = c_mul(tw, step);
            }
        }
    } else {
        const rsrc_t rk = make_rsrc(Kin + (size_t)h * L * kstride, (uint32_t)(L * kstride) * sizeof(float));
        // all of the thread's taps first, with no branch between the loads (a
        // tap past L reads tap 0 and is replaced by zero), so that they are in
        // flight together; FULL (L = M): every tap exists.  Stride 2 (the real
        // part of a complex kernel) reads every other float of one contiguous
        // run per wave.
        float kv[16][P];
#pragma unroll
        for (int e = 0; e < 16; ++e)
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int n = t + kT * e + kQ * p;
                const bool in = FULL || n < L;
                kv[e][p] = buf_ld_f32(rk, (uint32_t)((in ? n : 0) * kstride) * sizeof(float), 0);
            }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int q = t + kT * e;
            if (!FULL)
#pragma unroll
                for (int p = 0; p < P; ++p) kv[e][p] = q + kQ * p < L ? kv[e][p] : 0.0f;
            if (q == 0) kv[e][0] += dv;
            float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
            for (int p = 0; p < P; ++p) acc = c_add(acc, c_scale(wp[p], kv[e][p] * sc));
            v[e] = c_mul(acc, tw);
            if (e < 15) {
                power_after(tw, v[e]);
                tw = c_mul(tw, step);
            }
        }
    }
    wf_forward<kLogQ, 0>(v, lds, tw4Q, t);
    const rsrc_t rs = make_rsrc(S + (size_t)h * M + (size_t)k1 * kQ, kQ * sizeof(float2));
    const uint32_t vo = (uint32_t)wf_pos(t, 0) * sizeof(float2);
#pragma unroll
    for (int e = 0; e < 16; ++e) buf_st_c64(v[e], rs, vo, e * 64 * sizeof(float2));
}

// One workgroup per (row pair, k1) of the chunk [p0, p0 + np): the half c = 1
// at slice k1 and the half c = 3 at slice P - 1 - k1, whose radix-P weights are
// conjugates (3 + 4 (P - 1 - k1) = 4 P - (1 + 4 k1)), so one pass over the
// pair's inputs gives both: with the rows a (real part) and b (imaginary part),
// A = sum_p a_p W_p and B = sum_p b_p W_p, W_p = w_4P^(p (1 + 4 k1)), the c = 1
// sum is A + i B and the c = 3 sum conj(A) + i conj(B).  Both halves take the
// spectrum slice k1 (the c = 3 slice P - 1 - k1 is the conjugate of slice k1 at
// the complemented positions).  Each half is transformed, multiplied by its
// spectrum, inverse transformed and untwisted into Z[pl][half][slice][q]
// (natural q).  Items are renumbered so that the P workgroups of one pair share
// an XCD (their inputs are read into its L2 once).  FULL: L = M, every input
// position exists (no per-element test).
template <int LOGP, bool FULL>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(4))) void wl_conv_a_kernel(
    int Bsz, int H, int L, int npb, int64_t p0, int64_t nitems, int remap, const float* __restrict__ u,
    const float2* __restrict__ S, float2* __restrict__ Z, const float2* __restrict__ tw4Q,
    const float2* __restrict__ tw4M) {
    constexpr int P = 1 << LOGP, M = P * kQ;
    __shared__ float2 lds[GQ::LDS];
    const int t = threadIdx.x;
    int64_t it = blockIdx.x;
    if (remap) {
        const int64_t x = it & 7, s = it >> 3;
        it = ((s / P) * 8 + x) * P + s % P;
    }
    if (it >= nitems) return;  // uniform
    const int64_t pl = it >> LOGP;
    const int k1 = (int)(it & (P - 1));
    const int64_t pair = p0 + pl;
    const int h = (int)(pair / npb);
    const int b1 = 2 * (int)(pair - (int64_t)h * npb);
    const bool has2 = b1 + 1 < Bsz;
    const size_t row1 = ((size_t)b1 * H + h) * (size_t)L;
    const rsrc_t r1 = make_rsrc(u + row1, (uint32_t)L * sizeof(float));
    const rsrc_t r2 = make_rsrc(u + row1 + (has2 ? (size_t)H * L : 0), (uint32_t)L * sizeof(float));
    const uint32_t vt = (uint32_t)t * sizeof(float);

    float2 ya[16], yb[16];
    {
        const int ma = 1 + 4 * k1, mb = 4 * P - ma;
        float2 wa[P];
#pragma unroll
        for (int p = 0; p < P; ++p) wa[p] = root4p<LOGP>(tw4M, p * ma);
        float2 ta = tw4M[t * ma], tb = tw4M[t * mb];
        const float2 sa = tw4M[kT * ma], sb = tw4M[kT * mb];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int q = t + kT * e;
            float2 A = make_float2(0.0f, 0.0f), B = make_float2(0.0f, 0.0f);
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const uint32_t so = (uint32_t)(kT * e + kQ * p) * sizeof(float);
                float av = 0.0f, bv = 0.0f;
                if (FULL || q + kQ * p < L) {
                    av = buf_ld_f32(r1, vt, so);
                    bv = buf_ld_f32(r2, vt, so);  // row 1 again without a second row: dropped below
                }
                A.x = fmaf(av, wa[p].x, A.x);
                A.y = fmaf(av, wa[p].y, A.y);
                B.x = fmaf(bv, wa[p].x, B.x);
                B.y = fmaf(bv, wa[p].y, B.y);
            }
            if (!has2) B = make_float2(0.0f, 0.0f);
            ya[e] = c_mul(make_float2(A.x - B.y, A.y + B.x), ta);
            yb[e] = c_mul(make_float2(A.x + B.y, B.x - A.y), tb);
            if (e < 15) {
                power_after(ta, ya[e]);
                power_after(tb, yb[e]);
                ta = c_mul(ta, sa);
                tb = c_mul(tb, sb);
            }
        }
    }
    const uint32_t vq = (uint32_t)t * sizeof(float2);
    const int wv = t >> 6, lane = t & 63;
    // one half: transform, product with its spectrum slice, inverse, conjugate
    // twiddle, store (HALF 0: c = 1 at slice k1; HALF 1: c = 3 at slice P - 1 - k1)
    auto half = [&](float2(&v)[16], auto half_tag) {
        constexpr int HALF = decltype(half_tag)::value;
        const int ks = HALF ? P - 1 - k1 : k1;
        const int m = (HALF ? 3 : 1) + 4 * ks;
        wf_forward<kLogQ, 0>(v, lds, tw4Q, t);
        const rsrc_t rs = make_rsrc(S + (size_t)h * M + (size_t)k1 * kQ, kQ * sizeof(float2));
        if constexpr (HALF == 0) {
            const uint32_t vk = (uint32_t)wf_pos(t, 0) * sizeof(float2);
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = c_mul(v[e], buf_ld_c64(rs, vk, e * 64 * sizeof(float2)));
        } else {
            const uint32_t vkm = (uint32_t)((GQ::W - 1 - wv) * 16 * 64 + 63 - lane) * sizeof(float2);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                v[e] = c_mul(v[e], c_conj(buf_ld_c64(rs, vkm, (15 - e) * 64 * sizeof(float2))));
        }
        wf_inverse<kLogQ, 0>(v, lds, tw4Q, t);
        float2 tc = c_conj(tw4M[t * m]);
        const float2 sc = c_conj(tw4M[kT * m]);
        const rsrc_t rz = make_rsrc(Z + ((size_t)pl * 2 + HALF) * M + (size_t)ks * kQ, kQ * sizeof(float2));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            buf_st_c64(c_mul(v[e], tc), rz, vq, kT * e * sizeof(float2));
            if (e < 15) {
                power_after(tc, v[e]);
                tc = c_mul(tc, sc);
            }
        }
    };
    half(ya, std::integral_constant<int, 0>{});
    half(yb, std::integral_constant<int, 1>{});
}

// y[q + Q p] = sum over half, k1 of Z[pl][half][k1][q] conj(w_4P^(p m)); one
// thread per q.  grid np * (Q / 256), 256 threads.
template <int LOGP>
__global__ __launch_bounds__(256) void wl_conv_b_kernel(int Bsz, int H, int L, int npb, int64_t p0,
                                                        float* __restrict__ y, const float2* __restrict__ Z,
                                                        const float2* __restrict__ tw4M) {
    constexpr int P = 1 << LOGP, M = P * kQ;
    constexpr int QB = kQ / 256;
    const int64_t pl = blockIdx.x / QB;
    const int q = (int)(blockIdx.x % QB) * 256 + threadIdx.x;
    const int64_t pair = p0 + pl;
    const int h = (int)(pair / npb);
    const int b1 = 2 * (int)(pair - (int64_t)h * npb);
    const bool has2 = b1 + 1 < Bsz;
    float2 zc[2][P];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int k1 = 0; k1 < P; ++k1) zc[half][k1] = Z[((size_t)pl * 2 + half) * M + (size_t)k1 * kQ + q];
    float* y1 = y + ((size_t)b1 * H + h) * (size_t)L;
    float* y2 = y1 + (size_t)H * L;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float2 o = make_float2(0.0f, 0.0f);
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int k1 = 0; k1 < P; ++k1)
                o = c_add(o, c_mul(zc[half][k1], c_conj(root4p<LOGP>(tw4M, p * ((half ? 3 : 1) + 4 * k1)))));
        const int n = q + kQ * p;
        if (n < L) {
            __builtin_nontemporal_store(o.x, &y1[n]);
            if (has2) __builtin_nontemporal_store(o.y, &y2[n]);
        }
    }
}

// tab[j] = exp(-i pi j/(2n)), j < 2n, in float64, rounded
__global__ __launch_bounds__(256) void wl_twiddle_kernel(int n, float2* __restrict__ tab) {
    for (int j = blockIdx.x * 256 + threadIdx.x; j < 2 * n; j += gridDim.x * 256) {
        double sn, cs;
        sincospi((double)j / (double)(2 * n), &sn, &cs);
        tab[j] = make_float2((float)cs, (float)-sn);
    }
}

template <int LOGP>
hipError_t wl_spec_t(int64_t H, int64_t L, int64_t tiles, float2* roots, const int32_t* tstat, int32_t* status,
                     const float* Kin, int64_t kstride, const float* D, float2* K_out, float2* S, float2* tw4Q,
                     float2* tw4M, hipStream_t s) {
    constexpr int P = 1 << LOGP, M = P * kQ;
    hipLaunchKernelGGL(wl_twiddle_kernel, dim3((2 * kQ + 255) / 256), dim3(256), 0, s, kQ, tw4Q);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL(wl_twiddle_kernel, dim3((2 * M + 255) / 256), dim3(256), 0, s, M, tw4M);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    const int remap = H % 8 == 0 ? 1 : 0;  // whole rounds of 8 XCDs x P
    if (roots) {
        hipLaunchKernelGGL((wl_kt_kernel<LOGP>), dim3((unsigned)(H * P)), dim3(kT), 0, s, (int)tiles, roots, tstat,
                           status, (const float2*)tw4Q, (const float2*)tw4M, remap);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((wl_spec_kernel<LOGP, true>), dim3((unsigned)(H * P)), dim3(kT), 0, s, (int)L, nullptr,
                           (int64_t)1, (const float2*)roots, D, K_out, S, (const float2*)tw4Q, (const float2*)tw4M,
                           remap);
    } else {
        if (L == (int64_t)M)
            hipLaunchKernelGGL((wl_spec_kernel<LOGP, false, true>), dim3((unsigned)(H * P)), dim3(kT), 0, s, (int)L,
                               Kin, kstride, nullptr, D, nullptr, S, (const float2*)tw4Q, (const float2*)tw4M, remap);
        else
            hipLaunchKernelGGL((wl_spec_kernel<LOGP, false, false>), dim3((unsigned)(H * P)), dim3(kT), 0, s, (int)L,
                               Kin, kstride, nullptr, D, nullptr, S, (const float2*)tw4Q, (const float2*)tw4M, remap);
    }
    return hipGetLastError();
}

template <int LOGP>
hipError_t wl_conv_t(int64_t Bsz, int64_t H, int64_t L, const float* u, float* y, const float2* S, float2* Z,
                     const float2* tw4Q, const float2* tw4M, hipStream_t s) {
    constexpr int P = 1 << LOGP;
    const int64_t npb = (Bsz + 1) / 2, npairs = npb * H;
    // chunks of row pairs, each through both launches before the next, so the
    // intermediate of one chunk stays in the caches
    for (int64_t p0 = 0; p0 < npairs; p0 += kConvChunkPairs) {
        const int64_t np = npairs - p0 < kConvChunkPairs ? npairs - p0 : kConvChunkPairs;
        const int64_t items = np * P;
        // the renumbering is a bijection when the items fill whole rounds of 8 XCDs x P
        const int remap = items % (8 * P) == 0 ? 1 : 0;
        if (L == (int64_t)P * kQ)
            hipLaunchKernelGGL((wl_conv_a_kernel<LOGP, true>), dim3((unsigned)items), dim3(kT), 0, s, (int)Bsz, (int)H,
                               (int)L, (int)npb, p0, items, remap, u, S, Z, tw4Q, tw4M);
        else
            hipLaunchKernelGGL((wl_conv_a_kernel<LOGP, false>), dim3((unsigned)items), dim3(kT), 0, s, (int)Bsz,
                               (int)H, (int)L, (int)npb, p0, items, remap, u, S, Z, tw4Q, tw4M);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((wl_conv_b_kernel<LOGP>), dim3((unsigned)(np * (kQ / 256))), dim3(256), 0, s, (int)Bsz,
                           (int)H, (int)L, (int)npb, p0, y, (const float2*)Z, tw4M);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    return hipSuccess;
}

}  // namespace

// Spectrum for M = 32768 or 65536, of Re K + D delta_0 with K from the
// scrambled root values (roots non-null: they are overwritten; status, K_out
// nullable), or of a caller's real kernel (Kin with stride kstride); also fills
// the two twiddle tables (tw4Q: 2 x 16384 entries, tw4M: 2 M entries)
hipError_t launch_wl_spectrum(int64_t H, int64_t L, int64_t M, int64_t tiles, float2* roots, const int32_t* tstat,
                              int32_t* status, const float* Kin, int64_t kstride, const float* D, float2* K_out,
                              float2* S, float2* tw4Q, float2* tw4M, hipStream_t stream) {
    if (M == 2 * kQ)
        return wl_spec_t<1>(H, L, tiles, roots, tstat, status, Kin, kstride, D, K_out, S, tw4Q, tw4M, stream);
    if (M == 4 * kQ)
        return wl_spec_t<2>(H, L, tiles, roots, tstat, status, Kin, kstride, D, K_out, S, tw4Q, tw4M, stream);
    return hipErrorInvalidValue;
}

// convolution with a spectrum from launch_wl_spectrum; Z: the intermediate of
// one chunk of row pairs (kConvChunkPairs x 2 M complex)
hipError_t launch_wl_conv(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y, const float2* S,
                          float2* Z, const float2* tw4Q, const float2* tw4M, hipStream_t stream) {
    if (M == 2 * kQ) return wl_conv_t<1>(Bsz, H, L, u, y, S, Z, tw4Q, tw4M, stream);
    if (M == 4 * kQ) return wl_conv_t<2>(Bsz, H, L, u, y, S, Z, tw4Q, tw4M, stream);
    return hipErrorInvalidValue;
}

}  // namespace ssm
