// Kernel spectra and long causal convolution on the wave-structured transforms
// (1024 <= M <= 16384).
//
// Sources: "Recurrent, LSTM, and structured state-space models" -- filter-mode
// block (the kernel is the first L coefficients of the inverse radix-two
// transform of the root values), DPLR block (y_t = C^* x_t + D u_t) and
// radix-two DFT block (an exact polynomial product by zero padding to a
// radix-two length >= 2n - 1).
//
// The zero-padded length-2M product is split into its even and odd frequencies
// (cyclic and twisted halves, tw_j = exp(-i pi j/M)):
//   y = IFFT_M(FFT_M(z) . FFT_M(k)) + conj(tw) . IFFT_M(FFT_M(tw . z) . FFT_M(tw . k))
// on j < M, with both spectra scaled by 1/(2M).  Two batch rows of one channel
// go through at once as z = u_b + i u_{b+1} (the kernel is real, so the real
// and imaginary parts of y are the two rows).  The spectra are stored in the
// transform's scrambled order (wfft.hpp), so the convolution multiplies and
// transforms back without ever unscrambling, and each lane's spectrum loads
// are coalesced.
#include "common.hpp"
#include "fft.hpp"
#include "wfft.hpp"

namespace ssm {

namespace {

// Spectra of one channel's real kernel k (taps >= L zero, D at tap 0), scaled
// 1/(2M), into khat[h][0] (cyclic) and khat[h][1] (twisted), scrambled order.
// FROM_ROOTS: k = Re K, K the first L taps of the inverse transform of the root
// values (also written to K_out); the per-channel status is reduced from the
// root-value kernel's tile statuses, and a failing channel gets NaN spectra
// and kernel.  Otherwise k is read from a caller's kernel (stride kstride).
template <int LOGM, bool FROM_ROOTS>
__global__ __launch_bounds__(WGeo<LOGM>::T) __attribute__((amdgpu_waves_per_eu(4))) void wspec_kernel(
    int L, int tiles, const float2* __restrict__ roots, const int32_t* __restrict__ tile_status,
    const float* __restrict__ Kin, int64_t kstride, const float* __restrict__ D, float2* __restrict__ K_out,
    int32_t* __restrict__ status, float2* __restrict__ khat, const float2* __restrict__ twtab) {
    using G = WGeo<LOGM>;
    constexpr int M = G::M, T = G::T;
    __shared__ float2 lds[G::LDS > lds_padded_size(M) ? G::LDS : lds_padded_size(M)];
    __shared__ int sst;
    const int h = blockIdx.x;
    const int t = threadIdx.x;
    float2* kh0 = khat + (size_t)h * 2 * M;
    float2* kh1 = kh0 + M;
    float kr[16];
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
            for (int j = t; j < M; j += T) {
                kh0[j] = c_nan();
                kh1[j] = c_nan();
            }
            return;
        }
        // the inverse transform of the root values in natural order (Stockham,
        // 16 points per thread: the same thread count as the wave layout)
        const TwiddleRegs<LOGM, 4> tw(twtab, LOGM, t);
        float2 v[1][16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[0][e] = roots[(size_t)h * M + t + T * e];
        float2* const one[1] = {lds};
        fft_multi<1, LOGM, 4, true>(v, one, t, tw);
        const float invM = 1.0f / (float)M;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = t + T * e;
            const float2 kv = c_scale(v[0][e], invM);
            if (K_out && j < L) K_out[(size_t)h * L + j] = kv;
            kr[e] = j < L ? kv.x : 0.0f;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = t + T * e;
            kr[e] = j < L ? Kin[((size_t)h * L + j) * kstride] : 0.0f;
        }
    }
    if (t == 0 && D) kr[0] += D[h];
    const float sc = 1.0f / (float)(2 * M);
    const rsrc_t rk = make_rsrc(kh0, 2 * M * sizeof(float2));
    const uint32_t vo = (uint32_t)wf_pos(t, 0) * sizeof(float2);
    float2 w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = make_float2(kr[e] * sc, 0.0f);
    wf_forward<LOGM, false>(w, lds, twtab, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) buf_st_c64(w[e], rk, vo, e * 64 * sizeof(float2));
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = make_float2(kr[e] * sc, 0.0f);
    wf_forward<LOGM, true>(w, lds, twtab, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) buf_st_c64(w[e], rk, vo, (M + e * 64) * sizeof(float2));
}

// One workgroup (T = M/16 threads) per pair of batch rows (b, b+1) of one
// channel.  The input pair is read once and kept in registers for both halves;
// the cyclic half's result is kept in registers while the twisted half runs.
template <int LOGM>
__global__ __launch_bounds__(WGeo<LOGM>::T) __attribute__((amdgpu_waves_per_eu(4))) void wconv_kernel(
    int Bsz, int H, int L, int npb, int64_t npairs, int remap_bpc, const float* __restrict__ u,
    float* __restrict__ y, const float2* __restrict__ khat, const float2* __restrict__ twtab) {
    using G = WGeo<LOGM>;
    constexpr int M = G::M, T = G::T;
    __shared__ float2 lds[G::LDS];
    const int t = threadIdx.x;

    int64_t wg = blockIdx.x;
    if (remap_bpc > 0) {  // keep the blocks of one channel on one XCD (dispatch is round-robin over 8)
        const int64_t x = wg & 7, s = wg >> 3;
        wg = ((s / remap_bpc) * 8 + x) * remap_bpc + s % remap_bpc;
    }
    const int64_t pair = wg;
    if (pair >= npairs) return;  // uniform over the workgroup
    const int h = (int)(pair / npb);
    const int b1 = 2 * (int)(pair - (int64_t)h * npb);
    const bool has2 = b1 + 1 < Bsz;
    const size_t row1 = ((size_t)b1 * H + h) * (size_t)L;
    // buffer views: each row, and the channel's two spectra; lane offset t
    // (rows) or its scrambled position (spectra), register e as a uniform offset
    const rsrc_t r1 = make_rsrc(u + row1, (uint32_t)L * sizeof(float));
    const rsrc_t r2 = make_rsrc(u + row1 + (has2 ? (size_t)H * L : 0), (uint32_t)L * sizeof(float));
    const rsrc_t o1 = make_rsrc(y + row1, (uint32_t)L * sizeof(float));
    const rsrc_t o2 = make_rsrc(y + row1 + (has2 ? (size_t)H * L : 0), (uint32_t)L * sizeof(float));
    const rsrc_t rk = make_rsrc(khat + (size_t)h * 2 * M, 2 * M * sizeof(float2));
    const uint32_t vt = (uint32_t)t * sizeof(float);
    const uint32_t vk = (uint32_t)wf_pos(t, 0) * sizeof(float2);

    float2 z[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        z[e] = make_float2(0.0f, 0.0f);
        if (t + T * e < L) {
            z[e].x = buf_ld_f32(r1, vt, T * e * sizeof(float));
            if (has2) z[e].y = buf_ld_f32(r2, vt, T * e * sizeof(float));
        }
    }
    float2 v[16], out[16];
    // cyclic half
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = z[e];
    wf_forward<LOGM, false>(v, lds, twtab, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = c_mul(v[e], buf_ld_c64(rk, vk, e * 64 * sizeof(float2)));
    wf_inverse<LOGM, false>(v, lds, twtab, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = v[e];
    // twisted half (the twist and untwist are inside the transforms)
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = z[e];
    wf_forward<LOGM, true>(v, lds, twtab, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = c_mul(v[e], buf_ld_c64(rk, vk, (M + e * 64) * sizeof(float2)));
    wf_inverse<LOGM, true>(v, lds, twtab, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (t + T * e < L) {
            const float2 o = c_add(out[e], v[e]);
            buf_st_f32_nt(o.x, o1, vt, T * e * sizeof(float));
            if (has2) buf_st_f32_nt(o.y, o2, vt, T * e * sizeof(float));
        }
    }
}

// tab[j] = exp(-i pi j/M) in float64, rounded (the given-kernel path, where no
// root-value kernel writes it)
__global__ __launch_bounds__(256) void wtwiddle_kernel(int M, float2* __restrict__ twtab) {
    for (int j = blockIdx.x * 256 + threadIdx.x; j < M; j += gridDim.x * 256) {
        double sn, cs;
        sincospi((double)j / (double)M, &sn, &cs);
        twtab[j] = make_float2((float)cs, (float)-sn);
    }
}

template <int LOGM>
hipError_t wspec_launch(bool from_roots, int64_t H, int64_t L, int64_t tiles, const float2* roots,
                        const int32_t* tstat, const float* Kin, int64_t kstride, const float* D, float2* K_out,
                        int32_t* status, float2* khat, float2* twtab, hipStream_t stream) {
    using G = WGeo<LOGM>;
    if (from_roots) {
        hipLaunchKernelGGL((wspec_kernel<LOGM, true>), dim3((unsigned)H), dim3(G::T), 0, stream, (int)L, (int)tiles,
                           roots, tstat, Kin, kstride, D, K_out, status, khat, twtab);
    } else {
        hipLaunchKernelGGL(wtwiddle_kernel, dim3((unsigned)((G::M + 255) / 256)), dim3(256), 0, stream, G::M, twtab);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((wspec_kernel<LOGM, false>), dim3((unsigned)H), dim3(G::T), 0, stream, (int)L, (int)tiles,
                           roots, tstat, Kin, kstride, D, K_out, status, khat, twtab);
    }
    return hipGetLastError();
}

template <int LOGM>
hipError_t wconv_launch(int64_t Bsz, int64_t H, int64_t L, const float* u, float* y, const float2* khat,
                        const float2* twtab, hipStream_t stream) {
    using G = WGeo<LOGM>;
    const int64_t npb = (Bsz + 1) / 2;
    const int64_t npairs = npb * H;
    int remap = 0;
    if (H % 8 == 0) remap = (int)npb;
    hipLaunchKernelGGL((wconv_kernel<LOGM>), dim3((unsigned)npairs), dim3(G::T), 0, stream, (int)Bsz, (int)H, (int)L,
                       (int)npb, npairs, remap, u, y, khat, twtab);
    return hipGetLastError();
}

}  // namespace

// the wave-structured path covers these transform lengths
bool wave_path_fits(int64_t M) { return M >= 1024 && M <= 16384; }

hipError_t launch_wspectrum(bool from_roots, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                            const int32_t* tstat, const float* Kin, int64_t kstride, const float* D,
                            float2* K_out, int32_t* status, float2* khat, float2* twtab, hipStream_t stream) {
    switch (ilog2_exact(M)) {
#define SSM_WSPEC_CASE(LG)                                                                                       \
    case LG:                                                                                                     \
        return wspec_launch<LG>(from_roots, H, L, tiles, roots, tstat, Kin, kstride, D, K_out, status, khat,    \
                                twtab, stream);
        SSM_WSPEC_CASE(10) SSM_WSPEC_CASE(11) SSM_WSPEC_CASE(12) SSM_WSPEC_CASE(13) SSM_WSPEC_CASE(14)
#undef SSM_WSPEC_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_wconv(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y, const float2* khat,
                        const float2* twtab, hipStream_t stream) {
    switch (ilog2_exact(M)) {
#define SSM_WCONV_CASE(LG) \
    case LG: return wconv_launch<LG>(Bsz, H, L, u, y, khat, twtab, stream);
        SSM_WCONV_CASE(10) SSM_WCONV_CASE(11) SSM_WCONV_CASE(12) SSM_WCONV_CASE(13) SSM_WCONV_CASE(14)
#undef SSM_WCONV_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
