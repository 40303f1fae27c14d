// Kernel transform and convolution for M = R*C > 16384 (four-step FFT through
// the workspace).
//
// Sources as for the LDS-resident path ("Recurrent, LSTM, and structured
// state-space models": filter-mode block, DPLR block, radix-two DFT block).
// When one M-point transform no longer fits a workgroup's LDS, the length
// M = R*C (R = 256 rows, C = M/256 columns) is split into column transforms of
// length R or C, a twiddle exp(-+2 pi i a b/M), and row transforms, with the
// intermediate matrix in global memory:
//
//   spectrum of one channel (roots H in natural order):
//     SP1  X[r][c] = H[r*C + c]: inverse FFT over r, times conj w^(c*kr)
//     SP2  inverse FFT over each row c -> T[jr][jc] = K[jr + R*jc] (scaled 1/M);
//          writes K_out; forms the real kernel k (taps >= L zero, D at j = 0)
//          and its twisted copy; since X'[r'][c'] = k[r'*R + c'] = T[c'][r'],
//          the column FFT of X' is an FFT along a row of T; times w^(c'*kr');
//          stores Y[kr'][c'] (transposed through LDS)
//     SP3  FFT over each row of Y -> spectrum at [kr'][kc'] for frequency
//          kr' + C*kc' (in place)
//   convolution of one row pair z = u_b + i u_{b+1} (and its twisted copy):
//     C1   X'[r'][c'] = z[r'*R + c']: FFT over r' (length C), times w^(c'*kr')
//     C2   FFT over each row, times the spectrum (same order), inverse FFT,
//          times conj w^(c'*kr')                                   (in place)
//     C3   inverse FFT over kr' -> natural position r'*R + c'; untwist,
//          add the halves, store the two rows
//
// Every transform is a register/LDS Stockham FFT of 16 points per thread;
// each workgroup runs 16 transforms (256 threads) side by side, so global
// accesses are 128-byte rows of 16 neighbouring columns.
#include "common.hpp"
#include "fft.hpp"

namespace ssm {

namespace {

constexpr int kR = 256, kLogR = 8;   // rows of the four-step split
constexpr int kThreads = 256;
constexpr int kE = 16, kLogE = 4;    // points per thread
constexpr int kPad = lds_padded_size(256);

// w_M^e = exp(-2 pi i e/M) from the table tab[j] = exp(-i pi j/M)
__device__ __forceinline__ float2 wM(const float2* tab, int logm, int e) {
    return table_root(tab, logm, e & ((1 << logm) - 1), logm);
}

// SP1: column inverse transforms of the root values, in place.
// grid: H * (C/16) blocks; group g = column c0+g, thread t runs rows t + 16 e.
template <int LOGC>
__global__ __launch_bounds__(kThreads) void sp1_kernel(const float2* roots, float2* B1, const float2* __restrict__ twtab) {
    constexpr int C = 1 << LOGC, M = kR * C, LOGM = kLogR + LOGC, CB = 16;
    __shared__ float2 lds[CB * kPad];
    const int nb = C / CB;
    const int h = blockIdx.x / nb, c0 = (blockIdx.x % nb) * CB;
    const int g = threadIdx.x % CB, t = threadIdx.x / CB;  // T = R/16 = 16 threads per column
    const int c = c0 + g;
    const float2* X = roots + (size_t)h * M;
    float2* Xo = B1 + (size_t)h * M;  // may equal X: every element is read before it is written
    const TwiddleRegs<kLogR, kLogE> tw(twtab, LOGM, t);
    float2 v[1][kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) v[0][e] = X[(t + 16 * e) * C + c];
    float2* const b[1] = {lds + g * kPad};
    fft_multi<1, kLogR, kLogE, true>(v, b, t, tw);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int kr = t + 16 * e;
        Xo[kr * C + c] = c_mul(v[0][e], c_conj(wM(twtab, LOGM, c * kr)));
    }
}

// SP2: row inverse transforms -> K (natural order out), the real kernel and its
// twisted copy, their column transforms, Y = [2][C][R] into khat.
// FROM_ROOTS = false: the real kernel comes from Kin instead.
// grid: H * (R / RB) blocks, RB = 256 / (C/16) rows per block.
template <int LOGC, bool FROM_ROOTS>
__global__ __launch_bounds__(kThreads) void sp2_kernel(int L, int tiles, const float2* __restrict__ B1,
                                                       const int32_t* __restrict__ tile_status,
                                                       const float* __restrict__ Kin, int64_t kstride,
                                                       const float* __restrict__ D, float2* __restrict__ K_out,
                                                       int32_t* __restrict__ status, float2* __restrict__ khat,
                                                       const float2* __restrict__ twtab) {
    constexpr int C = 1 << LOGC, M = kR * C, LOGM = kLogR + LOGC, TC = C / kE, RB = kThreads / TC;
    constexpr int PAD = lds_padded_size(C);
    __shared__ float2 lds[2 * RB * PAD];
    __shared__ int sst;
    const int nb = kR / RB;
    const int h = blockIdx.x / nb, jr0 = (blockIdx.x % nb) * RB;
    const int g = threadIdx.x / TC, t = threadIdx.x % TC;  // row jr0+g, columns t + TC e
    const int jr = jr0 + g;
    float2* Y0 = khat ? khat + (size_t)h * 2 * M : nullptr;
    float2* Y1 = khat ? Y0 + M : nullptr;

    int st = 0;
    if constexpr (FROM_ROOTS) {
        if (threadIdx.x == 0) sst = 0;
        __syncthreads();
        int mx = 0;
        for (int i = threadIdx.x; i < tiles; i += kThreads) mx = max(mx, tile_status[(size_t)h * tiles + i]);
        if (mx) atomicMax(&sst, mx);
        __syncthreads();
        st = sst;
        if (blockIdx.x % nb == 0 && threadIdx.x == 0 && status) status[h] = st;
    }
    const TwiddleRegs<LOGC, kLogE> tw(twtab, LOGM, t);
    float kr[kE];
    if (st != 0) {  // uniform over the block: NaN-fill this block's outputs
        for (int i = threadIdx.x; i < RB * C; i += kThreads) {
            const int ri = i % RB, jc = i / RB;
            const int n = jr0 + ri + kR * jc;
            if (K_out && n < L) K_out[(size_t)h * L + n] = c_nan();
            if (khat) {
                Y0[jc * kR + jr0 + ri] = c_nan();
                Y1[jc * kR + jr0 + ri] = c_nan();
            }
        }
        return;
    }
    float2* tp = lds;  // staging for transposed global access: [RB][C + 1]
    if constexpr (FROM_ROOTS) {
        float2 v[1][kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) v[0][e] = B1[(size_t)h * M + jr * C + t + TC * e];
        float2* const b[1] = {lds + g * PAD};
        fft_multi<1, LOGC, kLogE, true>(v, b, t, tw);
        const float invM = 1.0f / (float)M;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const int n = jr + kR * (t + TC * e);
            v[0][e] = c_scale(v[0][e], invM);
            kr[e] = n < L ? v[0][e].x : 0.0f;
        }
        if (K_out) {  // K[jr + R jc]: stage [g][jc], store runs of RB neighbouring jr
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kE; ++e) tp[g * (C + 1) + t + TC * e] = v[0][e];
            __syncthreads();
            for (int i = threadIdx.x; i < RB * C; i += kThreads) {
                const int ri = i % RB, jc = i / RB;
                const int n = jr0 + ri + kR * jc;
                if (n < L) K_out[(size_t)h * L + n] = tp[ri * (C + 1) + jc];
            }
        }
        if (!khat) return;  // kernel transform only (uniform)
    } else {
        // stage Kin[jr + R jc] as [g][jc] with runs of RB neighbouring jr
        __syncthreads();
        for (int i = threadIdx.x; i < RB * C; i += kThreads) {
            const int ri = i % RB, jc = i / RB;
            const int n = jr0 + ri + kR * jc;
            tp[ri * (C + 1) + jc] = make_float2(n < L ? Kin[((size_t)h * L + n) * kstride] : 0.0f, 0.0f);
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kE; ++e) kr[e] = tp[g * (C + 1) + t + TC * e].x;
    }
    if (jr == 0 && t == 0 && D) kr[0] += D[h];  // n = 0 is (jr, jc) = (0, 0)

    const float sc = 1.0f / (float)(2 * M);
    float2 w[2][kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int n = jr + kR * (t + TC * e);
        w[0][e] = make_float2(kr[e] * sc, 0.0f);
        w[1][e] = c_scale(twtab[n], kr[e] * sc);
    }
    __syncthreads();  // staging buffer reused as FFT exchange space
    float2* const b2[2] = {lds + g * PAD, lds + (RB + g) * PAD};
    fft_multi<2, LOGC, kLogE, false>(w, b2, t, tw);
    // times w^(c' kr'), c' = jr, kr' = t + TC e; store Y[kr'][c'] through LDS
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int krp = t + TC * e;
        const float2 f = wM(twtab, LOGM, jr * krp);
        lds[g * (C + 1) + krp] = c_mul(w[0][e], f);
        lds[RB * (C + 1) + g * (C + 1) + krp] = c_mul(w[1][e], f);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < RB * C; i += kThreads) {
        const int ri = i % RB, krp = i / RB;
        Y0[krp * kR + jr0 + ri] = lds[ri * (C + 1) + krp];
        Y1[krp * kR + jr0 + ri] = lds[RB * (C + 1) + ri * (C + 1) + krp];
    }
}

// SP3: row transforms of Y (length R), in place -> spectra.
// grid: H * 2 * (C/16) blocks; group g = row, 16 threads per row.
template <int LOGC>
__global__ __launch_bounds__(kThreads) void sp3_kernel(float2* __restrict__ khat, const float2* __restrict__ twtab) {
    constexpr int C = 1 << LOGC, M = kR * C, LOGM = kLogR + LOGC, RB = 16;
    __shared__ float2 lds[RB * kPad];
    const int nb = C / RB;
    const int hs = blockIdx.x / nb, row0 = (blockIdx.x % nb) * RB;  // hs = 2h + half
    const int g = threadIdx.x / 16, t = threadIdx.x % 16;
    float2* Y = khat + (size_t)hs * M + (size_t)(row0 + g) * kR;
    const TwiddleRegs<kLogR, kLogE> tw(twtab, LOGM, t);
    float2 v[1][kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) v[0][e] = Y[t + 16 * e];
    float2* const b[1] = {lds + g * kPad};
    fft_multi<1, kLogR, kLogE, false>(v, b, t, tw);
#pragma unroll
    for (int e = 0; e < kE; ++e) Y[t + 16 * e] = v[0][e];
}

// C1: column transforms (length C) of a row pair and its twisted copy.
// grid: npairs * (R / CB) blocks, CB = 256 / (C/16) columns per block.
template <int LOGC>
__global__ __launch_bounds__(kThreads) void c1_kernel(int Bsz, int H, int L, int npb, int p0,
                                                      const float* __restrict__ u, float2* __restrict__ Z,
                                                      const float2* __restrict__ twtab) {
    constexpr int C = 1 << LOGC, M = kR * C, LOGM = kLogR + LOGC, TC = C / kE, CB = kThreads / TC;
    constexpr int PAD = lds_padded_size(C);
    __shared__ float2 lds[2 * CB * PAD];
    const int nb = kR / CB;
    const int pl = blockIdx.x / nb, c0 = (blockIdx.x % nb) * CB;  // pair pl of the chunk from p0
    const int p = p0 + pl;
    const int g = threadIdx.x % CB, t = threadIdx.x / CB;
    const int cp = c0 + g;  // column c'
    const int h = p / npb, b1 = 2 * (p % npb);
    const bool has2 = b1 + 1 < Bsz;
    const float* u1 = u + ((size_t)b1 * H + h) * (size_t)L;
    const float* u2 = u1 + (size_t)H * L;
    const TwiddleRegs<LOGC, kLogE> tw(twtab, LOGM, t);
    float2 v[2][kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int n = (t + TC * e) * kR + cp;
        const float2 z = make_float2(n < L ? u1[n] : 0.0f, (n < L && has2) ? u2[n] : 0.0f);
        v[0][e] = z;
        v[1][e] = c_mul(z, twtab[n]);
    }
    float2* const b[2] = {lds + g * PAD, lds + (CB + g) * PAD};
    fft_multi<2, LOGC, kLogE, false>(v, b, t, tw);
    float2* Z0 = Z + (size_t)pl * 2 * M;
    float2* Z1 = Z0 + M;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int krp = t + TC * e;
        const float2 f = wM(twtab, LOGM, cp * krp);
        Z0[krp * kR + cp] = c_mul(v[0][e], f);
        Z1[krp * kR + cp] = c_mul(v[1][e], f);
    }
}

// C2: row transform, times the spectrum, inverse row transform, conj twiddle.
// grid: npairs * (C / 16) blocks; both halves of 16 rows per block.
template <int LOGC>
__global__ __launch_bounds__(kThreads) void c2_kernel(int npb, int p0, float2* __restrict__ Z,
                                                      const float2* __restrict__ khat,
                                                      const float2* __restrict__ twtab) {
    constexpr int C = 1 << LOGC, M = kR * C, LOGM = kLogR + LOGC, RB = 16;
    __shared__ float2 lds[2 * RB * kPad];
    const int nb = C / RB;
    const int pl = blockIdx.x / nb, row0 = (blockIdx.x % nb) * RB;  // pair pl of the chunk from p0
    const int g = threadIdx.x / 16, t = threadIdx.x % 16;
    const int krp = row0 + g;
    const int h = (p0 + pl) / npb;
    float2* Z0 = Z + (size_t)pl * 2 * M + (size_t)krp * kR;
    float2* Z1 = Z0 + M;
    const float2* K0 = khat + (size_t)h * 2 * M + (size_t)krp * kR;
    const float2* K1 = K0 + M;
    const TwiddleRegs<kLogR, kLogE> tw(twtab, LOGM, t);
    float2 v[2][kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        v[0][e] = Z0[t + 16 * e];
        v[1][e] = Z1[t + 16 * e];
    }
    float2* const b[2] = {lds + g * kPad, lds + (RB + g) * kPad};
    fft_multi<2, kLogR, kLogE, false>(v, b, t, tw);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        v[0][e] = c_mul(v[0][e], K0[t + 16 * e]);
        v[1][e] = c_mul(v[1][e], K1[t + 16 * e]);
    }
    fft_multi<2, kLogR, kLogE, true>(v, b, t, tw);
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int cp = t + 16 * e;
        const float2 f = c_conj(wM(twtab, LOGM, cp * krp));
        Z0[cp] = c_mul(v[0][e], f);
        Z1[cp] = c_mul(v[1][e], f);
    }
}

// C3: inverse column transforms, untwist, add the halves, store both rows.
template <int LOGC>
__global__ __launch_bounds__(kThreads) void c3_kernel(int Bsz, int H, int L, int npb, int p0, float* __restrict__ y,
                                                      const float2* __restrict__ Z, const float2* __restrict__ twtab) {
    constexpr int C = 1 << LOGC, M = kR * C, LOGM = kLogR + LOGC, TC = C / kE, CB = kThreads / TC;
    constexpr int PAD = lds_padded_size(C);
    __shared__ float2 lds[2 * CB * PAD];
    const int nb = kR / CB;
    const int pl = blockIdx.x / nb, c0 = (blockIdx.x % nb) * CB;  // pair pl of the chunk from p0
    const int p = p0 + pl;
    const int g = threadIdx.x % CB, t = threadIdx.x / CB;
    const int cp = c0 + g;
    const int h = p / npb, b1 = 2 * (p % npb);
    const bool has2 = b1 + 1 < Bsz;
    const float2* Z0 = Z + (size_t)pl * 2 * M;
    const float2* Z1 = Z0 + M;
    const TwiddleRegs<LOGC, kLogE> tw(twtab, LOGM, t);
    float2 v[2][kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        v[0][e] = Z0[(t + TC * e) * kR + cp];
        v[1][e] = Z1[(t + TC * e) * kR + cp];
    }
    float2* const b[2] = {lds + g * PAD, lds + (CB + g) * PAD};
    fft_multi<2, LOGC, kLogE, true>(v, b, t, tw);
    float* y1 = y + ((size_t)b1 * H + h) * (size_t)L;
    float* y2 = y1 + (size_t)H * L;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int n = (t + TC * e) * kR + cp;
        if (n < L) {
            const float2 o = c_add(v[0][e], c_mul(v[1][e], c_conj(twtab[n])));
            y1[n] = o.x;
            if (has2) y2[n] = o.y;
        }
    }
}

__global__ __launch_bounds__(kThreads) void twiddle_table_kernel(int M, float2* __restrict__ twtab) {
    for (int j = blockIdx.x * kThreads + threadIdx.x; j < M; j += gridDim.x * kThreads) {
        double sn, cs;
        sincospi((double)j / (double)M, &sn, &cs);
        twtab[j] = make_float2((float)cs, (float)-sn);
    }
}

template <int LOGC>
hipError_t spectrum_large_t(bool from_roots, int64_t H, int64_t L, int64_t tiles, const float2* roots, float2* B1,
                            const int32_t* tstat, const float* Kin, int64_t kstride, const float* D, float2* K_out,
                            int32_t* status, float2* khat, float2* twtab, hipStream_t s) {
    constexpr int C = 1 << LOGC, TC = C / kE, RB = kThreads / TC;
    if (from_roots) {
        hipLaunchKernelGGL(sp1_kernel<LOGC>, dim3((unsigned)(H * (C / 16))), dim3(kThreads), 0, s, roots, B1, twtab);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((sp2_kernel<LOGC, true>), dim3((unsigned)(H * (kR / RB))), dim3(kThreads), 0, s, (int)L,
                           (int)tiles, B1, tstat, Kin, kstride, D, K_out, status, khat, twtab);
    } else {
        hipLaunchKernelGGL(twiddle_table_kernel, dim3(64), dim3(kThreads), 0, s, (int)(kR * C), twtab);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((sp2_kernel<LOGC, false>), dim3((unsigned)(H * (kR / RB))), dim3(kThreads), 0, s, (int)L,
                           (int)tiles, B1, tstat, Kin, kstride, D, K_out, status, khat, twtab);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    if (!khat) return hipSuccess;
    hipLaunchKernelGGL(sp3_kernel<LOGC>, dim3((unsigned)(H * 2 * (C / 16))), dim3(kThreads), 0, s, khat, twtab);
    return hipGetLastError();
}

template <int LOGC>
hipError_t conv_large_t(int64_t Bsz, int64_t H, int64_t L, const float* u, float* y, const float2* khat, float2* Z,
                        const float2* twtab, hipStream_t s) {
    constexpr int C = 1 << LOGC, TC = C / kE, CB = kThreads / TC;
    const int64_t npb = (Bsz + 1) / 2, npairs = npb * H;
    // chunks of row pairs, each through the three passes before the next, so
    // the intermediate of one chunk stays in the caches
    for (int64_t p0 = 0; p0 < npairs; p0 += kConvChunkPairs) {
        const int64_t np = npairs - p0 < kConvChunkPairs ? npairs - p0 : kConvChunkPairs;
        hipLaunchKernelGGL(c1_kernel<LOGC>, dim3((unsigned)(np * (kR / CB))), dim3(kThreads), 0, s, (int)Bsz,
                           (int)H, (int)L, (int)npb, (int)p0, u, Z, twtab);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL(c2_kernel<LOGC>, dim3((unsigned)(np * (C / 16))), dim3(kThreads), 0, s, (int)npb,
                           (int)p0, Z, khat, twtab);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL(c3_kernel<LOGC>, dim3((unsigned)(np * (kR / CB))), dim3(kThreads), 0, s, (int)Bsz,
                           (int)H, (int)L, (int)npb, (int)p0, y, Z, twtab);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    return hipSuccess;
}

}  // namespace

// M = 32768 or 65536.  from_roots: roots [H,M] -> B1 [H,M] (may alias roots),
// else the real kernel Kin (and twtab is filled here first).  khat may be
// null (kernel transform only).
hipError_t launch_spectrum_large(bool from_roots, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                                 float2* B1, const int32_t* tstat, const float* Kin, int64_t kstride, const float* D,
                                 float2* K_out, int32_t* status, float2* khat, float2* twtab, hipStream_t stream) {
    if (M == 32768)
        return spectrum_large_t<7>(from_roots, H, L, tiles, roots, B1, tstat, Kin, kstride, D, K_out, status, khat,
                                   twtab, stream);
    if (M == 65536)
        return spectrum_large_t<8>(from_roots, H, L, tiles, roots, B1, tstat, Kin, kstride, D, K_out, status, khat,
                                   twtab, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_conv_large(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y,
                             const float2* khat, float2* Z, const float2* twtab, hipStream_t stream) {
    if (M == 32768) return conv_large_t<7>(Bsz, H, L, u, y, khat, Z, twtab, stream);
    if (M == 65536) return conv_large_t<8>(Bsz, H, L, u, y, khat, Z, twtab, stream);
    return hipErrorInvalidValue;
}

}  // namespace ssm
