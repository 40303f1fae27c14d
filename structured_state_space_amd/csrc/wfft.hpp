// Wave-structured FFT for gfx950: an M = 2^LOGM point transform (1024 <= M <=
// 16384) held by W = M/1024 wavefronts of 64 lanes, 16 points per lane.
//
// The transform is the radix-two DFT of the pages' definition block ("Radix-two
// discrete Fourier transform": forward root exp(-2 pi i/M), the inverse the
// conjugate root, unscaled), factored as DFT_16 (register index) x DFT_W (wave
// index) x DFT_64 (lane index, itself DFT_4 x DFT_16), decimation in frequency:
//
//   A  registers: thread t = lane + 64 wave holds x[t + T e] in v[e] (T = 64 W,
//      the natural, coalesced order).  DFT_16 over e in registers, then the
//      twiddle exp(-2 pi i t k/M).
//   B  wave bits (W > 1): one exchange through LDS brings the wave index into
//      log2(W) register bits (the workgroup's only barriers); DFT_W over them
//      in registers; twiddle exp(-2 pi i lane k/T).
//   C1 lane bits 4, 5: swapped with register bits 0, 1 by gfx950's
//      v_permlane16_swap / v_permlane32_swap (no LDS); DFT_4; twiddle
//      exp(-2 pi i (lane mod 16) k/64).
//   C2 lane bits 0-3: swapped with register bits 0-3 through the wave's own
//      slice of LDS (wave-level synchronisation only; padded so that neither
//      side has bank conflicts); DFT_16.
//
// The output is every frequency exactly once, in a fixed scrambled order that
// depends only on M: thread (wave, lane) register e holds one frequency, and
// "position" (16 wave + e) 64 + lane is where a spectrum stored in that order
// keeps it, so a lane's loads of a stored spectrum are coalesced.  A
// convolution needs no unscrambling: the product of two spectra in the same
// order, run through the exact mirror of the forward steps with conjugate
// constants (wf_inverse), gives the unscaled inverse transform in natural order.
//
// TW folds a twist x_n exp(-2 pi i TW n/(4M)) (TW = 1 or 3) into stage A: the
// constant exp(-2 pi i TW e/64) per register and exp(-2 pi i t (TW + 4k)/(4M))
// as the stage twiddle.  So wf_forward<.., TW> is FFT_M(x . psi^TW) with
// psi_n = exp(-i pi n/(2M)), and wf_inverse<.., TW> is conj(psi^TW) . IFFT_M
// (unscaled): the two halves (bins 4j+1 and 4j+3 of the 4M-point transform)
// of a zero-padded negacyclic product of length 2M.
//
// Twiddles come from the table tab[j] = exp(-i pi j/(2M)), j < 2M (float64-
// accurate), one entry per stage and thread; the powers are formed by products.
#pragma once

#include "common.hpp"
#include "fft.hpp"

namespace ssm {

template <int LOGM>
struct WGeo {
    static_assert(LOGM >= 10 && LOGM <= 14, "wave-structured transforms cover 1024..16384 points");
    static constexpr int M = 1 << LOGM;
    static constexpr int LOGW = LOGM - 10;
    static constexpr int W = 1 << LOGW;   // waves per transform
    static constexpr int T = 64 * W;      // threads per transform
    static constexpr int S = 16 / W;      // register stride of the wave-index DFT
    // LDS of one transform (complex): the stage-B exchange uses M of them,
    // stage C2 one slice of kSlice per wave
    static constexpr int LDS = 1040 * W;
};

// per-wave LDS slice of stage C2: element (lane, e) at lane + 65 e (< 1039)
constexpr int kSlice = 1040;

// (cos, sin) of 2 pi K/64, K < 64
constexpr float kCos64[17] = {1.0f,
                              0.99518472667219688624f,
                              0.98078528040323044913f,
                              0.95694033573220886494f,
                              0.92387953251128675613f,
                              0.88192126434835502971f,
                              0.83146961230254523708f,
                              0.77301045336273696081f,
                              0.70710678118654752440f,
                              0.63439328416364549822f,
                              0.55557023301960222474f,
                              0.47139673682599764856f,
                              0.38268343236508977173f,
                              0.29028467725446236764f,
                              0.19509032201612826785f,
                              0.09801714032956060199f,
                              0.0f};
constexpr float cos64(int k) {
    k &= 63;
    return k <= 16 ? kCos64[k] : k <= 32 ? -kCos64[32 - k] : k <= 48 ? -kCos64[k - 32] : kCos64[64 - k];
}
constexpr float sin64(int k) { return cos64(k - 16); }

// a * exp(-+2 pi i K/64) for a compile-time K
template <int K, bool INV>
__device__ __forceinline__ float2 mul_root64(float2 a) {
    constexpr int k = K & 63;
    if constexpr (k == 0) {
        return a;
    } else if constexpr (k == 16) {
        return c_mul_mi<INV>(a);
    } else if constexpr (k == 32) {
        return make_float2(-a.x, -a.y);
    } else if constexpr (k == 48) {
        return c_mul_mi<!INV>(a);
    } else {
        return c_mul(a, make_float2(cos64(k), INV ? sin64(k) : -sin64(k)));
    }
}

// v[e] *= exp(-+2 pi i TW e/64)
template <int TW, bool INV, int K = 0>
__device__ __forceinline__ void pretwist64(float2 (&v)[16]) {
    if constexpr (K < 16) {
        v[K] = mul_root64<TW * K, INV>(v[K]);
        pretwist64<TW, INV, K + 1>(v);
    }
}

// The next power of a twiddle is formed only after the current one has been
// applied to `used`: an empty asm that takes `used` and passes p through.
// Otherwise the compiler computes the whole chain of powers first (for
// instruction-level parallelism) and holds all of them in registers.
__device__ __forceinline__ void power_after(float2& p, const float2& used) {
    asm volatile("" : "+v"(p.x), "+v"(p.y) : "v"(used.x), "v"(used.y));
}

// ---- stage A: DFT_16 over the register index, twiddle exp(-2 pi i t k/M)
//      (TW: exp(-2 pi i t (TW + 4k)/(4M)), the per-register constant first) ----
// The four table entries a transform's stage twiddles start from.  PRE
// transforms load them together when they start, so that only the first
// stage's wait is exposed; the others load each right before its stage (fewer
// registers held, for kernels at their register limit).
struct WTw {
    float2 a;   // exp(-2 pi i t/M)
    float2 u;   // exp(-2 pi i t/(4M)) (twisted transforms)
    float2 b;   // exp(-2 pi i lane/T), T = 64 W = 4M/64
    float2 c1;  // exp(-2 pi i (lane mod 16)/64), 4M/64 = 64 W
};
template <int LOGM, int TW>
__device__ __forceinline__ void wf_tw_load_a(WTw& w, const float2* __restrict__ tab, int t) {
    w.a = tab[4 * t];
    w.u = TW != 0 ? tab[t] : make_float2(1.0f, 0.0f);
}
template <int LOGM>
__device__ __forceinline__ void wf_tw_load_b(WTw& w, const float2* __restrict__ tab, int lane) {
    w.b = WGeo<LOGM>::W > 1 ? tab[lane * 64] : make_float2(1.0f, 0.0f);
}
template <int LOGM>
__device__ __forceinline__ void wf_tw_load_c1(WTw& w, const float2* __restrict__ tab, int lane) {
    w.c1 = tab[(lane & 15) * 64 * WGeo<LOGM>::W];
}

template <int LOGM, int TW, bool INV>
__device__ __forceinline__ void wf_twiddle_a(float2 (&v)[16], const WTw& tw) {
    float2 step = tw.a;
    if (INV) step.y = -step.y;
    // keep the powers per call (not hoisted and kept live across stages)
    asm volatile("" : "+v"(step.x), "+v"(step.y));
    if constexpr (TW != 0) {
        float2 u = tw.u;
        if (INV) u.y = -u.y;
        float2 p = TW == 1 ? u : c_mul(c_mul(u, u), u);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            v[k] = c_mul(v[k], p);
            if (k < 15) {
                power_after(p, v[k]);
                p = c_mul(p, step);
            }
        }
    } else {
        float2 p = step;
#pragma unroll
        for (int k = 1; k < 16; ++k) {
            v[k] = c_mul(v[k], p);
            if (k < 15) {
                power_after(p, v[k]);
                p = c_mul(p, step);
            }
        }
    }
}

// ---- stage B helpers: DFT_W over the register groups {e_lo + S j} ----
template <int LOGM, bool INV>
__device__ __forceinline__ void wf_dft_waves(float2 (&v)[16]) {
    using G = WGeo<LOGM>;
#pragma unroll
    for (int elo = 0; elo < G::S; ++elo) {
        float2 x[G::W];
#pragma unroll
        for (int j = 0; j < G::W; ++j) x[j] = v[elo + G::S * j];
        dft_reg<G::W, INV>(x);
#pragma unroll
        for (int j = 0; j < G::W; ++j) v[elo + G::S * j] = x[j];
    }
}

template <int LOGM, bool INV>
__device__ __forceinline__ void wf_twiddle_b(float2 (&v)[16], const WTw& tw) {
    using G = WGeo<LOGM>;
    float2 base = tw.b;
    if (INV) base.y = -base.y;
    asm volatile("" : "+v"(base.x), "+v"(base.y));
    float2 p = base;
#pragma unroll
    for (int k = 1; k < G::W; ++k) {
#pragma unroll
        for (int elo = 0; elo < G::S; ++elo) v[elo + G::S * k] = c_mul(v[elo + G::S * k], p);
        if (k + 1 < G::W) {
            power_after(p, v[G::S * k]);
            p = c_mul(p, base);
        }
    }
}

// ---- stage C1: register bits 0, 1 <-> lane bits 4, 5 ----
__device__ __forceinline__ void swap_bits_lane45(float2 (&v)[16]) {
#pragma unroll
    for (int e = 0; e < 16; e += 2) {  // register bit 0 <-> lane bit 4
        const auto rx = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[e].x), __float_as_uint(v[e + 1].x), false,
                                                         false);
        const auto ry = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[e].y), __float_as_uint(v[e + 1].y), false,
                                                         false);
        v[e] = make_float2(__uint_as_float(rx[0]), __uint_as_float(ry[0]));
        v[e + 1] = make_float2(__uint_as_float(rx[1]), __uint_as_float(ry[1]));
    }
#pragma unroll
    for (int g = 0; g < 16; g += 4) {  // register bit 1 <-> lane bit 5
#pragma unroll
        for (int e = g; e < g + 2; ++e) {
            const auto rx = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[e].x), __float_as_uint(v[e + 2].x),
                                                             false, false);
            const auto ry = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[e].y), __float_as_uint(v[e + 2].y),
                                                             false, false);
            v[e] = make_float2(__uint_as_float(rx[0]), __uint_as_float(ry[0]));
            v[e + 2] = make_float2(__uint_as_float(rx[1]), __uint_as_float(ry[1]));
        }
    }
}

template <bool INV>
__device__ __forceinline__ void wf_dft4_groups(float2 (&v)[16]) {
#pragma unroll
    for (int g = 0; g < 16; g += 4) {
        float2 x[4] = {v[g], v[g + 1], v[g + 2], v[g + 3]};
        dft_reg<4, INV>(x);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[g + j] = x[j];
    }
}

template <int LOGM, bool INV>
__device__ __forceinline__ void wf_twiddle_c1(float2 (&v)[16], const WTw& tw) {
    float2 base = tw.c1;
    if (INV) base.y = -base.y;
    asm volatile("" : "+v"(base.x), "+v"(base.y));
    const float2 b2 = c_mul(base, base), b3 = c_mul(b2, base);
#pragma unroll
    for (int g = 0; g < 16; g += 4) {
        v[g + 1] = c_mul(v[g + 1], base);
        v[g + 2] = c_mul(v[g + 2], b2);
        v[g + 3] = c_mul(v[g + 3], b3);
    }
}

// ---- stage C2: register bits 0-3 <-> lane bits 0-3 through the wave's LDS slice.
//      Element (lane, e) sits at lane + 65 e: the writes of one register are 64
//      consecutive slots, and the reads of one register, (lane & 48) + e' +
//      65 (lane & 15), fall on 16 distinct bank pairs within each 16-lane group;
//      each side takes one address register plus immediate offsets. ----
template <bool BACK>
__device__ __forceinline__ void swap_bits_lane0123(float2 (&v)[16], float2* __restrict__ slice, int lane) {
    float2* const pw = slice + lane;                              // + 65 e
    float2* const pr = slice + (lane & 48) + 65 * (lane & 15);    // + e
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (!BACK)
            pw[65 * e] = v[e];
        else
            pr[e] = v[e];
    }
    lds_sync<true>();
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = BACK ? pw[65 * e] : pr[e];
    lds_sync<true>();
}

// ---- the exchange of stage B (W > 1): every wave of the transform takes part ----
// forward: element (wave j, register e_lo + S wv) moves to (wave wv, register e_lo + S j)
template <int LOGM, bool BACK>
__device__ __forceinline__ void exchange_waves(float2 (&v)[16], float2* __restrict__ lds, int lane, int wv) {
    using G = WGeo<LOGM>;
    __syncthreads();  // the buffer's previous readers (and other waves' slices) are done
#pragma unroll
    for (int j = 0; j < G::W; ++j)
#pragma unroll
        for (int elo = 0; elo < G::S; ++elo) {
            const int natural = lane + 64 * (elo + G::S * j + 16 * wv);       // written by (wv, register e)
            const int swapped = lane + 64 * (elo + G::S * wv + 16 * j);       // read into (wv, register e_lo + S j)
            if (!BACK)
                lds[natural] = v[elo + G::S * j];
            else
                lds[swapped] = v[elo + G::S * j];
        }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G::W; ++j)
#pragma unroll
        for (int elo = 0; elo < G::S; ++elo) {
            const int natural = lane + 64 * (elo + G::S * j + 16 * wv);
            const int swapped = lane + 64 * (elo + G::S * wv + 16 * j);
            v[elo + G::S * j] = BACK ? lds[natural] : lds[swapped];
        }
    if (!BACK) __syncthreads();  // before the wave slices of stage C2 reuse the buffer
}

// Forward transform (see the header comment).  lds: WGeo::LDS complex, shared by the
// T = 64 W threads of the transform (threadIdx.x < T), every one of which
// must call it.  t = threadIdx.x.
template <int LOGM, int TW, bool PRE = true>
__device__ __forceinline__ void wf_forward(float2 (&v)[16], float2* __restrict__ lds, const float2* __restrict__ tab,
                                           int t) {
    using G = WGeo<LOGM>;
    const int lane = t & 63, wv = t >> 6;
    WTw tw;
    if constexpr (PRE) {
        wf_tw_load_a<LOGM, TW>(tw, tab, t);
        wf_tw_load_b<LOGM>(tw, tab, lane);
        wf_tw_load_c1<LOGM>(tw, tab, lane);
    }
    if constexpr (TW != 0) pretwist64<TW, false>(v);
    dft_reg<16, false>(v);
    if constexpr (!PRE) wf_tw_load_a<LOGM, TW>(tw, tab, t);
    wf_twiddle_a<LOGM, TW, false>(v, tw);
    if constexpr (G::W > 1) {
        exchange_waves<LOGM, false>(v, lds, lane, wv);
        wf_dft_waves<LOGM, false>(v);
        if constexpr (!PRE) wf_tw_load_b<LOGM>(tw, tab, lane);
        wf_twiddle_b<LOGM, false>(v, tw);
    }
    swap_bits_lane45(v);
    wf_dft4_groups<false>(v);
    if constexpr (!PRE) wf_tw_load_c1<LOGM>(tw, tab, lane);
    wf_twiddle_c1<LOGM, false>(v, tw);
    swap_bits_lane0123<false>(v, lds + kSlice * wv, lane);
    dft_reg<16, false>(v);
}

// The exact mirror of wf_forward with conjugate constants: from the scrambled
// order back to natural order, unscaled (M x the inverse transform).
template <int LOGM, int TW, bool PRE = true>
__device__ __forceinline__ void wf_inverse(float2 (&v)[16], float2* __restrict__ lds, const float2* __restrict__ tab,
                                           int t) {
    using G = WGeo<LOGM>;
    const int lane = t & 63, wv = t >> 6;
    WTw tw;
    if constexpr (PRE) {
        wf_tw_load_c1<LOGM>(tw, tab, lane);
        wf_tw_load_b<LOGM>(tw, tab, lane);
        wf_tw_load_a<LOGM, TW>(tw, tab, t);
    }
    dft_reg<16, true>(v);
    swap_bits_lane0123<true>(v, lds + kSlice * wv, lane);
    if constexpr (!PRE) wf_tw_load_c1<LOGM>(tw, tab, lane);
    wf_twiddle_c1<LOGM, true>(v, tw);
    wf_dft4_groups<true>(v);
    swap_bits_lane45(v);
    if constexpr (G::W > 1) {
        if constexpr (!PRE) wf_tw_load_b<LOGM>(tw, tab, lane);
        wf_twiddle_b<LOGM, true>(v, tw);
        wf_dft_waves<LOGM, true>(v);
        exchange_waves<LOGM, true>(v, lds, lane, wv);
    }
    if constexpr (!PRE) wf_tw_load_a<LOGM, TW>(tw, tab, t);
    wf_twiddle_a<LOGM, TW, true>(v, tw);
    dft_reg<16, true>(v);
    if constexpr (TW != 0) pretwist64<TW, true>(v);
}

// position of register e of thread t in a spectrum stored in the scrambled order
__device__ __forceinline__ int wf_pos(int t, int e) { return ((t >> 6) * 16 + e) * 64 + (t & 63); }

// The frequency index held at position ((16 wave + e) 64 + lane): stage A leaves
// the DFT_16 output k1 in the registers; the exchange moves its top log2(W)
// bits to the wave index and the stage-B output k2a into the top register
// bits; stage C1 moves register bits 0-1 to lane bits 4-5 and leaves k2b_a in
// register bits 0-1; stage C2 moves register bits 0-3 to lane bits 0-3 and
// leaves k2b_b in the registers.  k = k1 + 16 (k2a + W (k2b_a + 4 k2b_b)).
// Complementing every digit (k -> M - 1 - k) complements the wave, register and
// lane indices.
template <int LOGM>
__host__ __device__ constexpr int wf_freq(int wave, int e, int lane) {
    constexpr int LOGW = LOGM - 10, W = 1 << LOGW, SB = 4 - LOGW;  // register bits of k1 left after the exchange
    const int rb = ((lane >> 4) & 3) | (((lane >> 2) & 3) << 2);  // register index before stage C1
    const int k1 = (rb & ((1 << SB) - 1)) | (wave << SB);
    const int k2a = rb >> SB;
    const int k2b_a = lane & 3, k2b_b = e;
    return k1 + 16 * (k2a + W * (k2b_a + 4 * k2b_b));
}

// Run-time form for the root-value kernel: the frequency stored at position pos
// of a channel's scrambled root values.  M <= 16384: the transform's own order;
// M = P 16384 (P = 2, 4): slice k1 = pos / 16384 holds the frequencies P k2 + k1,
// k2 in the order of the 16384-point transform.
__host__ __device__ inline int wf_freq_rt(int logm, int pos) {
    const int lq = logm < 14 ? logm : 14;
    const int q = pos & ((1 << lq) - 1);
    const int logw = lq - 10, sb = 4 - logw;
    const int wave = q >> 10, e = (q >> 6) & 15, lane = q & 63;
    const int rb = ((lane >> 4) & 3) | (((lane >> 2) & 3) << 2);
    const int k1 = (rb & ((1 << sb) - 1)) | (wave << sb);
    const int k2a = rb >> sb;
    const int k = k1 + 16 * (k2a + (1 << logw) * ((lane & 3) + 4 * e));
    if (logm <= 14) return k;
    return (k << (logm - 14)) + (pos >> 14);
}

// ---- raw buffer access: the base and size in scalar registers, one 32-bit
//      lane offset, and a uniform offset per register (so a thread's 16
//      strided accesses need no per-access address registers) ----
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float2 buf_ld_c64(rsrc_t r, uint32_t voff, uint32_t soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
}
__device__ __forceinline__ float buf_ld_f32(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void buf_st_c64(float2 x, rsrc_t r, uint32_t voff, uint32_t soff) {
    using u2 = __attribute__((ext_vector_type(2))) unsigned int;
    const u2 d = {__float_as_uint(x.x), __float_as_uint(x.y)};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)voff, (int)soff, 0);
}
// streaming store (nt: not read again)
__device__ __forceinline__ void buf_st_f32_nt(float x, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)voff, (int)soff, 2);
}

}  // namespace ssm
