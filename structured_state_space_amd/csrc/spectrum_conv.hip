// Kernel transform and long causal convolution, LDS-resident (M <= 16384).
//
// Sources: "Recurrent, LSTM, and structured state-space models" -- filter-mode
// block (the kernel is the first L coefficients of the inverse radix-two
// transform of the root values), DPLR block (y_t = C^* x_t + D u_t, the skip term
// is separate) and radix-two DFT block (an exact polynomial product by zero
// padding to a radix-two length >= 2n - 1).
//
// Convolution by the zero-padded length-2M product, split into its even and odd
// frequencies.  With k the length-M real kernel (taps j >= L zero, D added at
// j = 0) and z a zero-padded input row, let tw_j = exp(-i pi j/M):
//   cyclic:   c = IFFT_M(FFT_M(z) . FFT_M(k))
//   twisted:  n = conj(tw) . IFFT_M(FFT_M(tw . z) . FFT_M(tw . k))
// (the even and odd bins of the 2M-point transform), and the linear product is
// (c + n)/2 on j < M.  Both inverse transforms are left unscaled; the spectra
// carry the factor 1/(2M).  Two batch rows of one channel are convolved at once
// as z = u_b + i u_{b+1}: the kernel is real, so the real and imaginary parts of
// the result are the two rows' outputs.
#include "common.hpp"
#include "fft.hpp"

namespace ssm {

namespace {

// points per thread: 8 up to M = 1024 (more waves per row for the small
// transforms), 16 above (M = 16384 takes 1024 threads)
__host__ __device__ constexpr int conv_loge(int logm) { return logm <= 3 ? logm : logm <= 10 ? 3 : 4; }

template <int LOGM>
struct Geo {
    static constexpr int M = 1 << LOGM;
    static constexpr int LOGE = conv_loge(LOGM);
    static constexpr int E = 1 << LOGE;
    static constexpr int T = M >> LOGE;  // threads per transform
    static constexpr int LDS = lds_padded_size(M);
    // conv: the cyclic and twisted halves are transformed together (sharing
    // twiddles and barriers).  Groups of T threads (one row pair each) per
    // workgroup: one wave holds several small transforms.  The halves have an
    // LDS buffer each for multi-wave groups up to M = 4096; otherwise they take
    // turns in one buffer.
    static constexpr bool ONE_WAVE = T <= 64;
    static constexpr int G = ONE_WAVE ? 64 / T : 1;
    static constexpr int THREADS = G * T;
    static constexpr int NBUF = (!ONE_WAVE && LOGM <= 12) ? 2 : 1;
    // spectrum kernel: its two forward transforms share one buffer above M = 4096
    static constexpr int SPEC_NBUF = LOGM <= 12 ? 2 : 1;
    static constexpr int WAVES = LOGM >= 14 ? 4 : 2;  // register budget: 128 / 256 VGPRs
    static constexpr bool PREFETCH = LOGM <= 13;
    // M = 16384 (1024 threads, 128 registers): the cyclic and twisted halves
    // one after the other, one vector in registers
    static constexpr bool SEQ = LOGM >= 14;
    static constexpr int LRMAX = LOGE < 4 ? LOGE : 4;  // largest butterfly radix (log2)
};

// Spectra of the kernel: khat[h][0] = FFT_M(k)/(2M), khat[h][1] = FFT_M(tw k)/(2M),
// tw_j = exp(-i pi j/M).  FROM_ROOTS: k comes from the inverse transform of the
// root values (and is also written to K_out), and the twiddles come from the
// table tab[j] = exp(-i pi j/M) that the root-value kernel wrote; otherwise k
// is read from a caller's real kernel, the twiddles are computed here, and
// block 0 writes the table for the convolution.
template <int LOGM, bool FROM_ROOTS>
__global__ __launch_bounds__(Geo<LOGM>::T) __attribute__((amdgpu_waves_per_eu(Geo<LOGM>::WAVES))) void spectrum_kernel(
    int L, int tiles, const float2* __restrict__ roots, const int32_t* __restrict__ tile_status,
    const float* __restrict__ Kin, int64_t kstride, const float* __restrict__ D, float2* __restrict__ K_out,
    int32_t* __restrict__ status, float2* __restrict__ khat, float2* __restrict__ twtab) {
    using Gm = Geo<LOGM>;
    constexpr int M = Gm::M, E = Gm::E, T = Gm::T, LOGE = Gm::LOGE;
    __shared__ float2 lds[Gm::SPEC_NBUF * Gm::LDS];
    __shared__ int sst;
    const int h = blockIdx.x;
    const int t = threadIdx.x;
    float2* kh0 = khat ? khat + (size_t)h * 2 * M : nullptr;  // null: kernel transform only
    float2* kh1 = khat ? kh0 + M : nullptr;
    float kr[E];
    float2* const one[1] = {lds};
    float2* const two[2] = {lds, lds + (Gm::SPEC_NBUF - 1) * Gm::LDS};

    if constexpr (FROM_ROOTS) {
        if (t == 0) sst = 0;
        __syncthreads();
        int mx = 0;
        for (int i = t; i < tiles; i += T) mx = max(mx, tile_status[(size_t)h * tiles + i]);
        if (mx) atomicMax(&sst, mx);
        __syncthreads();
        const int st = sst;
        if (t == 0 && status) status[h] = st;
        if (st != 0) {  // uniform: NaN-fill this channel's outputs
            for (int j = t; j < L; j += T)
                if (K_out) K_out[(size_t)h * L + j] = c_nan();
            if (khat)
                for (int j = t; j < M; j += T) {
                    kh0[j] = c_nan();
                    kh1[j] = c_nan();
                }
            return;
        }
        const TwiddleRegs<LOGM, LOGE> tw(twtab, LOGM, t);
        float2 v[1][E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[0][e] = roots[(size_t)h * M + t + T * e];
        fft_multi<1, LOGM, LOGE, true>(v, one, t, tw);
        const float invM = 1.0f / (float)M;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = t + T * e;
            v[0][e] = c_scale(v[0][e], invM);
            if (K_out && j < L) K_out[(size_t)h * L + j] = v[0][e];
            kr[e] = j < L ? v[0][e].x : 0.0f;
        }
        if (!khat) return;  // uniform
        if (t == 0 && D) kr[0] += D[h];
        const float sc = 1.0f / (float)(2 * M);
        float2 w[2][E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            w[0][e] = make_float2(kr[e] * sc, 0.0f);
            w[1][e] = c_scale(twtab[t + T * e], kr[e] * sc);
        }
        fft_multi<2, LOGM, LOGE, false, Gm::SPEC_NBUF == 1>(w, two, t, tw);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            kh0[t + T * e] = w[0][e];
            kh1[t + T * e] = w[1][e];
        }
    } else {
        if (h == 0)
            for (int j = t; j < M; j += T) {
                double sn, cs;
                sincospi((double)j / (double)M, &sn, &cs);
                twtab[j] = make_float2((float)cs, (float)-sn);
            }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = t + T * e;
            kr[e] = j < L ? Kin[((size_t)h * L + j) * kstride] : 0.0f;
        }
        if (t == 0 && D) kr[0] += D[h];
        const float sc = 1.0f / (float)(2 * M);
        float2 w[2][E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            w[0][e] = make_float2(kr[e] * sc, 0.0f);
            w[1][e] = c_scale(root_of_unity<false>(t + T * e, 2 * M), kr[e] * sc);
        }
        fft_multi<2, LOGM, LOGE, false, Gm::SPEC_NBUF == 1>(w, two, t, TwiddleSincos{});
#pragma unroll
        for (int e = 0; e < E; ++e) {
            kh0[t + T * e] = w[0][e];
            kh1[t + T * e] = w[1][e];
        }
    }
}

// Inputs of the fused form: the spectra are formed from the root values inside
// the convolution (no separate kernel-transform launch, no spectra in HBM).
struct FusedSpec {
    const float2* roots;         // [H][M] root values
    const int32_t* tile_status;  // [H][tiles] root-value kernel status
    int tiles;
    const float* D;   // [H] or null
    float2* K_out;    // [H][L] or null
    int32_t* status;  // [H] or null
};

// One group of T threads per pair of batch rows (b, b+1) of one channel:
// z = u_b + i u_{b+1};  y = IFFT(FFT(z) khat0) + conj(tw) IFFT(FFT(tw z) khat1).
// FUSED: each group computes its channel's khat0/khat1 from the root values
// itself (inverse transform, truncation to L taps, D at tap 0, two forward
// transforms), the inverse transform alongside the input's forward transforms;
// the group of the channel's first row pair also writes K_out and the channel
// status.  This repeats the kernel transform once per row pair, which pays only
// where the grid is small and latency-bound.
// CPLX: a complex kernel K = K_r + i K_i given by two spectra sets (khat for
// K_r + D delta_0, khat_im for K_i).  The input's forward transforms are shared:
// Z.khat gives (K_r * u_b, K_r * u_{b+1}) into y, Z.khat_im gives
// (K_i * u_b, K_i * u_{b+1}) into y_im.
template <int LOGM, bool FUSED, bool CPLX = false>
__global__ __launch_bounds__(Geo<LOGM>::THREADS) __attribute__((amdgpu_waves_per_eu(Geo<LOGM>::WAVES))) void conv_kernel(
    int Bsz, int H, int L, int npb, int64_t npairs, int remap_bpc, const float* __restrict__ u,
    float* __restrict__ y, const float2* __restrict__ khat, const float2* __restrict__ twtab, FusedSpec fs,
    const float2* __restrict__ khat_im = nullptr, float* __restrict__ y_im = nullptr) {
    using Gm = Geo<LOGM>;
    static_assert(!(CPLX && (FUSED || Gm::SEQ)), "complex kernels take the form with both halves in registers (M <= 8192)");
    constexpr int M = Gm::M, E = Gm::E, T = Gm::T, LOGE = Gm::LOGE, G = Gm::G;
    // fused: three transforms at once (one buffer each, or one shared buffer)
    constexpr int FNBUF = Gm::NBUF == 1 ? 1 : 3;
    constexpr int NB = FUSED ? FNBUF : Gm::NBUF;
    __shared__ float2 lds[G * NB * Gm::LDS];
    // one group per workgroup: the row pair is uniform (scalar registers and
    // scalar-based addressing)
    const int grp = G == 1 ? 0 : threadIdx.x / T;
    const int t = threadIdx.x - grp * T;

    int64_t wg = blockIdx.x;
    if (remap_bpc > 0) {  // keep the blocks of one channel on one XCD (dispatch is round-robin over 8)
        const int64_t x = wg & 7, s = wg >> 3;
        wg = ((s / remap_bpc) * 8 + x) * remap_bpc + s % remap_bpc;
    }
    const int64_t pair = wg * G + grp;
    const bool active = pair < npairs;
    int h = active ? (int)(pair / npb) : 0;
    int b1 = active ? 2 * (int)(pair - (int64_t)h * npb) : 0;
    if constexpr (G == 1) {  // uniform: keep in scalar registers
        h = __builtin_amdgcn_readfirstlane(h);
        b1 = __builtin_amdgcn_readfirstlane(b1);
    }
    const bool has2 = active && (b1 + 1 < Bsz);
    const size_t row1 = ((size_t)b1 * H + h) * (size_t)L;
    const size_t row2 = row1 + (size_t)H * L;
    float2* my = lds + grp * NB * Gm::LDS;
    const float2* kh0 = khat + (size_t)h * 2 * M;
    const float2* kh1 = kh0 + M;
    const TwiddleRegs<LOGM, LOGE, Gm::LRMAX> tw(twtab, LOGM, t);

    auto load = [&](int e) {
        const int j = t + T * e;
        const bool in = active && j < L;
        return make_float2(in ? u[row1 + j] : 0.0f, (in && has2) ? u[row2 + j] : 0.0f);
    };

    float2 out[E];
    float2 outi[CPLX ? E : 1];
    int chst = 0;
    if constexpr (Gm::SEQ && !FUSED) {
        float2* const one[1] = {my};
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {
            // the thread index passes through an empty asm in each half, so the
            // inputs, spectra and twist factors are read where they are used
            // rather than hoisted out of the loop (their registers would spill)
            int tl = t;
            asm volatile("" : "+v"(tl));
            float2 v[1][E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int j = tl + T * e;
                const bool in = active && j < L;
                const float2 z = make_float2(in ? u[row1 + j] : 0.0f, (in && has2) ? u[row2 + j] : 0.0f);
                v[0][e] = half ? c_mul(z, twtab[j]) : z;
            }
            fft_multi<1, LOGM, LOGE, false, false, Gm::LRMAX>(v, one, t, tw);
            const float2* kh = half ? kh1 : kh0;
#pragma unroll
            for (int e = 0; e < E; ++e) v[0][e] = c_mul(v[0][e], kh[tl + T * e]);
            fft_multi<1, LOGM, LOGE, true, false, Gm::LRMAX>(v, one, t, tw);
#pragma unroll
            for (int e = 0; e < E; ++e)
                out[e] = half ? c_add(out[e], c_mul(v[0][e], c_conj(twtab[tl + T * e]))) : v[0][e];
        }
    } else {
        // spectra and twist factors are fetched up front (and held) unless registers are short
        constexpr bool PRE = Gm::PREFETCH || FUSED;
        float2 v[2][E], tws[PRE ? E : 1], k0[PRE ? E : 1], k1[PRE ? E : 1];
        float2* const bufs[2] = {my, my + (Gm::NBUF - 1) * Gm::LDS};
        if constexpr (FUSED) {
            // The root values' inverse transform is run as a forward transform of
            // their conjugates, together with the input's two forward transforms
            // (they are independent): three vectors in one pass sequence.
            float2 x3[3][E];
#pragma unroll
            for (int e = 0; e < E; ++e) x3[0][e] = c_conj(fs.roots[(size_t)h * M + t + T * e]);
#pragma unroll
            for (int e = 0; e < E; ++e) tws[e] = twtab[t + T * e];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float2 z = load(e);
                x3[1][e] = z;
                x3[2][e] = c_mul(z, tws[e]);
            }
            for (int i = 0; i < fs.tiles; ++i) chst = max(chst, fs.tile_status[(size_t)h * fs.tiles + i]);
            const bool lead = active && b1 == 0;
            if (lead && t == 0 && fs.status) fs.status[h] = chst;
            constexpr int STEP = FNBUF == 1 ? 0 : Gm::LDS;  // FNBUF == 1: one shared buffer
            float2* const three[3] = {my, my + STEP, my + 2 * STEP};
            fft_multi<3, LOGM, LOGE, false, FNBUF == 1, Gm::LRMAX>(x3, three, t, tw);
            const float invM = 1.0f / (float)M, sc = 1.0f / (float)(2 * M);
            float2 w[2][E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int j = t + T * e;
                const float2 kv = c_scale(c_conj(x3[0][e]), invM);
                if (lead && fs.K_out && j < L) fs.K_out[(size_t)h * L + j] = chst ? c_nan() : kv;
                float kr = j < L ? kv.x : 0.0f;
                if (j == 0 && fs.D) kr += fs.D[h];
                w[0][e] = make_float2(kr * sc, 0.0f);
                w[1][e] = c_scale(tws[e], kr * sc);
                v[0][e] = x3[1][e];
                v[1][e] = x3[2][e];
            }
            fft_multi<2, LOGM, LOGE, false, Gm::NBUF == 1, Gm::LRMAX>(w, bufs, t, tw);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                k0[e] = w[0][e];
                k1[e] = w[1][e];
            }
        } else {
            if constexpr (PRE) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    tws[e] = twtab[t + T * e];
                    k0[e] = kh0[t + T * e];
                    k1[e] = kh1[t + T * e];
                }
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float2 z = load(e);
                v[0][e] = z;
                v[1][e] = c_mul(z, PRE ? tws[PRE ? e : 0] : twtab[t + T * e]);
            }
            fft_multi<2, LOGM, LOGE, false, Gm::NBUF == 1, Gm::LRMAX>(v, bufs, t, tw);
        }
        float2 wi[CPLX ? 2 : 1][E];
        if constexpr (CPLX) {  // products with the imaginary part's spectra (read on use)
            const float2* ki0 = khat_im + (size_t)h * 2 * M;
            const float2* ki1 = ki0 + M;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                wi[0][e] = c_mul(v[0][e], ki0[t + T * e]);
                wi[1][e] = c_mul(v[1][e], ki1[t + T * e]);
            }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            v[0][e] = c_mul(v[0][e], PRE ? k0[PRE ? e : 0] : kh0[t + T * e]);
            v[1][e] = c_mul(v[1][e], PRE ? k1[PRE ? e : 0] : kh1[t + T * e]);
        }
        fft_multi<2, LOGM, LOGE, true, Gm::NBUF == 1, Gm::LRMAX>(v, bufs, t, tw);
#pragma unroll
        for (int e = 0; e < E; ++e)
            out[e] = c_add(v[0][e], c_mul(v[1][e], c_conj(PRE ? tws[PRE ? e : 0] : twtab[t + T * e])));
        if constexpr (CPLX) {
            fft_multi<2, LOGM, LOGE, true, Gm::NBUF == 1, Gm::LRMAX>(wi, bufs, t, tw);
#pragma unroll
            for (int e = 0; e < E; ++e)
                outi[e] = c_add(wi[0][e], c_mul(wi[1][e], c_conj(PRE ? tws[PRE ? e : 0] : twtab[t + T * e])));
        }
    }

    if (active) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = t + T * e;
            if (j < L) {
                if (FUSED && chst) out[e] = c_nan();
                // streaming stores (not read again; less end-of-kernel write-back)
                __builtin_nontemporal_store(out[e].x, &y[row1 + j]);
                if (has2) __builtin_nontemporal_store(out[e].y, &y[row2 + j]);
                if constexpr (CPLX) {
                    __builtin_nontemporal_store(outi[e].x, &y_im[row1 + j]);
                    if (has2) __builtin_nontemporal_store(outi[e].y, &y_im[row2 + j]);
                }
            }
        }
    }
}

template <int LOGM>
hipError_t spectrum_launch(bool from_roots, int64_t H, int64_t L, int64_t tiles, const float2* roots,
                           const int32_t* tstat, const float* Kin, int64_t kstride, const float* D, float2* K_out,
                           int32_t* status, float2* khat, float2* twtab, hipStream_t stream) {
    using Gm = Geo<LOGM>;
    if (from_roots)
        hipLaunchKernelGGL((spectrum_kernel<LOGM, true>), dim3((unsigned)H), dim3(Gm::T), 0, stream, (int)L,
                           (int)tiles, roots, tstat, Kin, kstride, D, K_out, status, khat, twtab);
    else
        hipLaunchKernelGGL((spectrum_kernel<LOGM, false>), dim3((unsigned)H), dim3(Gm::T), 0, stream, (int)L,
                           (int)tiles, roots, tstat, Kin, kstride, D, K_out, status, khat, twtab);
    return hipGetLastError();
}

template <int LOGM>
hipError_t conv_launch(int64_t Bsz, int64_t H, int64_t L, const float* u, float* y, const float2* khat,
                       const float2* twtab, hipStream_t stream) {
    using Gm = Geo<LOGM>;
    const int64_t npb = (Bsz + 1) / 2;
    const int64_t npairs = npb * H;
    const int64_t blocks = (npairs + Gm::G - 1) / Gm::G;
    int remap = 0;
    if (npb % Gm::G == 0 && H % 8 == 0) remap = (int)(npb / Gm::G);
    hipLaunchKernelGGL((conv_kernel<LOGM, false>), dim3((unsigned)blocks), dim3(Gm::THREADS), 0, stream, (int)Bsz,
                       (int)H, (int)L, (int)npb, npairs, remap, u, y, khat, twtab, FusedSpec{});
    return hipGetLastError();
}

template <int LOGM>
hipError_t conv_complex_launch(int64_t Bsz, int64_t H, int64_t L, const float* u, float* y_re, float* y_im,
                               const float2* khat_re, const float2* khat_im, const float2* twtab,
                               hipStream_t stream) {
    using Gm = Geo<LOGM>;
    const int64_t npb = (Bsz + 1) / 2;
    const int64_t npairs = npb * H;
    const int64_t blocks = (npairs + Gm::G - 1) / Gm::G;
    int remap = 0;
    if (npb % Gm::G == 0 && H % 8 == 0) remap = (int)(npb / Gm::G);
    hipLaunchKernelGGL((conv_kernel<LOGM, false, true>), dim3((unsigned)blocks), dim3(Gm::THREADS), 0, stream,
                       (int)Bsz, (int)H, (int)L, (int)npb, npairs, remap, u, y_re, khat_re, twtab, FusedSpec{},
                       khat_im, y_im);
    return hipGetLastError();
}

template <int LOGM>
hipError_t conv_fused_launch(int64_t Bsz, int64_t H, int64_t L, const float* u, float* y, const float2* twtab,
                             const FusedSpec& fs, hipStream_t stream) {
    using Gm = Geo<LOGM>;
    const int64_t npb = (Bsz + 1) / 2;
    const int64_t npairs = npb * H;
    const int64_t blocks = (npairs + Gm::G - 1) / Gm::G;
    int remap = 0;
    if (npb % Gm::G == 0 && H % 8 == 0) remap = (int)(npb / Gm::G);
    hipLaunchKernelGGL((conv_kernel<LOGM, true>), dim3((unsigned)blocks), dim3(Gm::THREADS), 0, stream, (int)Bsz,
                       (int)H, (int)L, (int)npb, npairs, remap, u, y, nullptr, twtab, fs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_spectrum(bool from_roots, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                           const int32_t* tstat, const float* Kin, int64_t kstride, const float* D,
                           float2* K_out, int32_t* status, float2* khat, float2* twtab, hipStream_t stream) {
    switch (ilog2_exact(M)) {
#define SSM_SPEC_CASE(LG)                                                                                       \
    case LG:                                                                                                    \
        return spectrum_launch<LG>(from_roots, H, L, tiles, roots, tstat, Kin, kstride, D, K_out, status, khat, \
                                   twtab, stream);
        SSM_SPEC_CASE(0) SSM_SPEC_CASE(1) SSM_SPEC_CASE(2) SSM_SPEC_CASE(3) SSM_SPEC_CASE(4)
        SSM_SPEC_CASE(5) SSM_SPEC_CASE(6) SSM_SPEC_CASE(7) SSM_SPEC_CASE(8) SSM_SPEC_CASE(9)
        SSM_SPEC_CASE(10) SSM_SPEC_CASE(11) SSM_SPEC_CASE(12) SSM_SPEC_CASE(13) SSM_SPEC_CASE(14)
#undef SSM_SPEC_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_conv(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y, const float2* khat,
                       const float2* twtab, hipStream_t stream) {
    switch (ilog2_exact(M)) {
#define SSM_CONV_CASE(LG) \
    case LG: return conv_launch<LG>(Bsz, H, L, u, y, khat, twtab, stream);
        SSM_CONV_CASE(0) SSM_CONV_CASE(1) SSM_CONV_CASE(2) SSM_CONV_CASE(3) SSM_CONV_CASE(4)
        SSM_CONV_CASE(5) SSM_CONV_CASE(6) SSM_CONV_CASE(7) SSM_CONV_CASE(8) SSM_CONV_CASE(9)
        SSM_CONV_CASE(10) SSM_CONV_CASE(11) SSM_CONV_CASE(12) SSM_CONV_CASE(13) SSM_CONV_CASE(14)
#undef SSM_CONV_CASE
        default: return hipErrorInvalidValue;
    }
}

// Both parts of a complex kernel in one convolution (shared input transforms),
// where that measured faster than two convolutions: up to M = 1024 (no spill)
// and at M = 4096 (a small spill; 10% less added time than a second spectrum
// and convolution).  At M = 2048 the larger spill made it slower, and from
// M = 8192 on the two halves do not fit the registers at all.
bool conv_complex_fits(int64_t M) { return M <= 1024 || M == 4096; }

hipError_t launch_conv_complex(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y_re,
                               float* y_im, const float2* khat_re, const float2* khat_im, const float2* twtab,
                               hipStream_t stream) {
    switch (ilog2_exact(M)) {
#define SSM_CPLX_CASE(LG) \
    case LG: return conv_complex_launch<LG>(Bsz, H, L, u, y_re, y_im, khat_re, khat_im, twtab, stream);
        SSM_CPLX_CASE(0) SSM_CPLX_CASE(1) SSM_CPLX_CASE(2) SSM_CPLX_CASE(3) SSM_CPLX_CASE(4)
        SSM_CPLX_CASE(5) SSM_CPLX_CASE(6) SSM_CPLX_CASE(7) SSM_CPLX_CASE(8) SSM_CPLX_CASE(9)
        SSM_CPLX_CASE(10) SSM_CPLX_CASE(11) SSM_CPLX_CASE(12) SSM_CPLX_CASE(13)
#undef SSM_CPLX_CASE
        default: return hipErrorInvalidValue;
    }
}

// The kernel transform runs inside the convolution for transforms of at most
// 1024 points and at most four row pairs per channel (the repeated transform
// then costs less than a separate launch and the spectra's HBM round trip).
bool conv_fuses_spectrum(int64_t Bsz, int64_t M) { return M >= 16 && M <= 1024 && (Bsz + 1) / 2 <= 4; }

hipError_t launch_conv_fused(int64_t Bsz, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                             const int32_t* tstat, const float* D, float2* K_out, int32_t* status, const float* u,
                             float* y, const float2* twtab, hipStream_t stream) {
    const FusedSpec fs{roots, tstat, (int)tiles, D, K_out, status};
    switch (ilog2_exact(M)) {
#define SSM_FUSED_CASE(LG) \
    case LG: return conv_fused_launch<LG>(Bsz, H, L, u, y, twtab, fs, stream);
        SSM_FUSED_CASE(4) SSM_FUSED_CASE(5) SSM_FUSED_CASE(6) SSM_FUSED_CASE(7) SSM_FUSED_CASE(8)
        SSM_FUSED_CASE(9) SSM_FUSED_CASE(10)
#undef SSM_FUSED_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
