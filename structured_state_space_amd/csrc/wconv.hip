// Kernel spectra and long causal convolution on the wave-structured transforms
// (1024 <= M <= 16384).
//
// Sources: "Recurrent, LSTM, and structured state-space models" -- filter-mode
// block (the kernel is the first L coefficients of the inverse radix-two
// transform of the root values), DPLR block (y_t = C^* x_t + D u_t) and
// radix-two DFT block (an exact polynomial product by zero padding to a
// radix-two length >= 2n - 1).
//
// The zero-padded product is taken modulo z^(2M) + 1 (negacyclic; the linear
// product has degree < 2M - 1, so nothing wraps), split by z^(2M) + 1 =
// (z^M - i)(z^M + i) into two M-point halves with the twists psi^1 and psi^3,
// psi_j = exp(-i pi j/(2M)):
//   y = conj(psi) . IFFT_M(FFT_M(psi . z) . S_A) + conj(psi^3) . IFFT_M(FFT_M(psi^3 . z) . S_B)
// on j < M, with S_A = FFT_M(psi . k)/(2M) and S_B = FFT_M(psi^3 . k)/(2M).
// For a real kernel k, S_B[j] = conj(S_A[M - 1 - j]), so only S_A is formed
// and stored (M complex per channel): in the transform's scrambled order the
// partner M - 1 - j of a position is the position with every index complemented
// (wfft.hpp), and a lane's reads of S_B are S_A read backwards, conjugated.
// Two batch rows of one channel go through at once as z = u_b + i u_{b+1}
// (the kernel is real, so the real and imaginary parts of y are the two rows).
// The convolution multiplies in the scrambled order and transforms back
// without ever unscrambling; each lane's spectrum loads are coalesced.
#include "common.hpp"
#include "fft.hpp"
#include "wfft.hpp"

namespace ssm {

namespace {

// Spectrum S_A of one channel's real kernel k (taps >= L zero, D at tap 0),
// scaled 1/(2M), into khat[h] (M complex, scrambled order).  FROM_ROOTS:
// k = Re K, K the first L taps of the inverse transform of the root values
// (stored in the transform's scrambled order; K is also written to K_out);
// the per-channel status is reduced from the root-value kernel's tile
// statuses, and a failing channel gets a NaN spectrum and kernel.  Otherwise k
// is read from a caller's kernel (stride kstride).  tw4: exp(-i pi j/(2M)),
// j < 2M.
template <int LOGM, bool FROM_ROOTS>
__global__ __launch_bounds__(WGeo<LOGM>::T) __attribute__((amdgpu_waves_per_eu(4))) void wspec_kernel(
    int L, int tiles, const float2* __restrict__ roots, const int32_t* __restrict__ tile_status,
    const float* __restrict__ Kin, int64_t kstride, const float* __restrict__ D, float2* __restrict__ K_out,
    int32_t* __restrict__ status, float2* __restrict__ khat, const float2* __restrict__ tw4) {
    using G = WGeo<LOGM>;
    constexpr int M = G::M, T = G::T;
    __shared__ float2 lds[G::LDS];
    __shared__ int sst;
    const int h = blockIdx.x;
    const int t = threadIdx.x;
    float2* kh = khat + (size_t)h * M;
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
            for (int j = t; j < M; j += T) kh[j] = c_nan();
            return;
        }
        // the root values are stored in the transform's scrambled order: the
        // mirrored steps give the inverse transform in natural order
        const rsrc_t rr = make_rsrc(roots + (size_t)h * M, M * sizeof(float2));
        const uint32_t vp = (uint32_t)wf_pos(t, 0) * sizeof(float2);
        float2 v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = buf_ld_c64(rr, vp, e * 64 * sizeof(float2));
        wf_inverse<LOGM, 0>(v, lds, tw4, t);
        const float invM = 1.0f / (float)M;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = t + T * e;
            const float2 kv = c_scale(v[e], invM);
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
    const rsrc_t rk = make_rsrc(kh, M * sizeof(float2));
    const uint32_t vo = (uint32_t)wf_pos(t, 0) * sizeof(float2);
    float2 w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = make_float2(kr[e] * sc, 0.0f);
    wf_forward<LOGM, 1>(w, lds, tw4, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) buf_st_c64(w[e], rk, vo, e * 64 * sizeof(float2));
}

// One workgroup (T = M/16 threads) per pair of batch rows (b, b+1) of one
// channel.  The input pair is read once and kept in registers for both halves;
// the cyclic half's result is kept in registers while the twisted half runs.
// At its register limit: the transforms load each stage's table entries right
// before the stage.
template <int LOGM>
__global__ __launch_bounds__(WGeo<LOGM>::T) __attribute__((amdgpu_waves_per_eu(4))) void wconv_kernel(
    int Bsz, int H, int L, int npb, int64_t npairs, int remap_bpc, const float* __restrict__ u,
    float* __restrict__ y, const float2* __restrict__ khat, const float2* __restrict__ tw4) {
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
    const rsrc_t rk = make_rsrc(khat + (size_t)h * M, M * sizeof(float2));
    const uint32_t vt = (uint32_t)t * sizeof(float);
    const int wv = t >> 6, lane = t & 63;
    const uint32_t vk = (uint32_t)wf_pos(t, 0) * sizeof(float2);
    // the complemented position (G::W - 1 - wv, 15 - e, 63 - lane), register e at uniform offset (15 - e) 64
    const uint32_t vkm = (uint32_t)((G::W - 1 - wv) * 16 * 64 + 63 - lane) * sizeof(float2);

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
    // half A: twist psi
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = z[e];
    wf_forward<LOGM, 1, false>(v, lds, tw4, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = c_mul(v[e], buf_ld_c64(rk, vk, e * 64 * sizeof(float2)));
    wf_inverse<LOGM, 1, false>(v, lds, tw4, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = v[e];
    // half B: twist psi^3, spectrum S_B = conj(S_A) at the complemented position
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = z[e];
    wf_forward<LOGM, 3, false>(v, lds, tw4, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = c_mul(v[e], c_conj(buf_ld_c64(rk, vkm, (15 - e) * 64 * sizeof(float2))));
    wf_inverse<LOGM, 3, false>(v, lds, tw4, t);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (t + T * e < L) {
            const float2 o = c_add(out[e], v[e]);
            buf_st_f32_nt(o.x, o1, vt, T * e * sizeof(float));
            if (has2) buf_st_f32_nt(o.y, o2, vt, T * e * sizeof(float));
        }
    }
}

// tab[j] = exp(-i pi j/(2M)), j < 2M, in float64, rounded
__global__ __launch_bounds__(256) void wtwiddle4_kernel(int M, float2* __restrict__ tw4) {
    for (int j = blockIdx.x * 256 + threadIdx.x; j < 2 * M; j += gridDim.x * 256) {
        double sn, cs;
        sincospi((double)j / (double)(2 * M), &sn, &cs);
        tw4[j] = make_float2((float)cs, (float)-sn);
    }
}

template <int LOGM>
hipError_t wspec_launch(bool from_roots, int64_t H, int64_t L, int64_t tiles, const float2* roots,
                        const int32_t* tstat, const float* Kin, int64_t kstride, const float* D, float2* K_out,
                        int32_t* status, float2* khat, float2* tw4, hipStream_t stream, bool tw4_ready) {
    using G = WGeo<LOGM>;
    if (!tw4_ready) {
        hipLaunchKernelGGL(wtwiddle4_kernel, dim3((unsigned)((2 * G::M + 255) / 256)), dim3(256), 0, stream, G::M,
                           tw4);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    if (from_roots)
        hipLaunchKernelGGL((wspec_kernel<LOGM, true>), dim3((unsigned)H), dim3(G::T), 0, stream, (int)L, (int)tiles,
                           roots, tstat, Kin, kstride, D, K_out, status, khat, (const float2*)tw4);
    else
        hipLaunchKernelGGL((wspec_kernel<LOGM, false>), dim3((unsigned)H), dim3(G::T), 0, stream, (int)L, (int)tiles,
                           roots, tstat, Kin, kstride, D, K_out, status, khat, (const float2*)tw4);
    return hipGetLastError();
}

template <int LOGM>
hipError_t wconv_launch(int64_t Bsz, int64_t H, int64_t L, const float* u, float* y, const float2* khat,
                        const float2* tw4, hipStream_t stream) {
    using G = WGeo<LOGM>;
    const int64_t npb = (Bsz + 1) / 2;
    const int64_t npairs = npb * H;
    int remap = 0;
    if (H % 8 == 0) remap = (int)npb;
    hipLaunchKernelGGL((wconv_kernel<LOGM>), dim3((unsigned)npairs), dim3(G::T), 0, stream, (int)Bsz, (int)H, (int)L,
                       (int)npb, npairs, remap, u, y, khat, tw4);
    return hipGetLastError();
}

}  // namespace

// the wave-structured path covers these transform lengths
bool wave_path_fits(int64_t M) { return M >= 1024 && M <= 16384; }

// tw4_ready: the table was written earlier on this stream (by the root-value launch)
hipError_t launch_wspectrum(bool from_roots, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                            const int32_t* tstat, const float* Kin, int64_t kstride, const float* D,
                            float2* K_out, int32_t* status, float2* khat, float2* tw4, hipStream_t stream,
                            bool tw4_ready) {
    switch (ilog2_exact(M)) {
#define SSM_WSPEC_CASE(LG)                                                                                       \
    case LG:                                                                                                     \
        return wspec_launch<LG>(from_roots, H, L, tiles, roots, tstat, Kin, kstride, D, K_out, status, khat,    \
                                tw4, stream, tw4_ready);
        SSM_WSPEC_CASE(10) SSM_WSPEC_CASE(11) SSM_WSPEC_CASE(12) SSM_WSPEC_CASE(13) SSM_WSPEC_CASE(14)
#undef SSM_WSPEC_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_wconv(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y, const float2* khat,
                        const float2* tw4, hipStream_t stream) {
    switch (ilog2_exact(M)) {
#define SSM_WCONV_CASE(LG) \
    case LG: return wconv_launch<LG>(Bsz, H, L, u, y, khat, tw4, stream);
        SSM_WCONV_CASE(10) SSM_WCONV_CASE(11) SSM_WCONV_CASE(12) SSM_WCONV_CASE(13) SSM_WCONV_CASE(14)
#undef SSM_WCONV_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
