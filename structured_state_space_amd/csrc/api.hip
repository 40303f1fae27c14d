// C ABI entry points: argument checks, workspace layout, kernel launches.
// Everything data-dependent happens on the device; the host only validates
// sizes and pointers and enqueues work on the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.hpp"

namespace ssm {
int64_t cauchy_tiles(int64_t H, int64_t N, int64_t r, int64_t M);
int64_t cauchy_prep_bytes(int64_t H, int64_t N, int64_t r, int64_t M);
hipError_t launch_cauchy(int64_t H, int64_t N, int64_t r, int64_t M, const float2* Lambda, const float2* P,
                         const float2* Q, const float2* Bv, const float2* Ct, const float* dt, float2* roots,
                         int32_t* tile_status, float2* twtab, double* tant, void* prep, hipStream_t stream,
                         bool scrambled, float2* tw4 = nullptr, bool* tw4_done = nullptr);
hipError_t launch_spectrum(bool from_roots, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                           const int32_t* tstat, const float* Kin, int64_t kstride, const float* D,
                           float2* K_out, int32_t* status, float2* khat, float2* twtab, hipStream_t stream);
hipError_t launch_conv(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y, const float2* khat,
                       const float2* twtab, hipStream_t stream);
bool conv_fuses_spectrum(int64_t Bsz, int64_t M);
bool conv_complex_fits(int64_t M);
hipError_t launch_conv_complex(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y_re,
                               float* y_im, const float2* khat_re, const float2* khat_im, const float2* twtab,
                               hipStream_t stream);
bool single_launch_fits(int64_t Bsz, int64_t H, int64_t M);
hipError_t launch_single(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, const float2* Lambda,
                         const float2* P, const float2* Q, const float2* Bv, const float2* Ct, const float* dt,
                         const float* D, const float* u, float* y, float2* K_out, int32_t* status,
                         hipStream_t stream, float2* roots_out = nullptr);
hipError_t launch_conv_fused(int64_t Bsz, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                             const int32_t* tstat, const float* D, float2* K_out, int32_t* status, const float* u,
                             float* y, const float2* twtab, hipStream_t stream);
hipError_t launch_spectrum_large(bool from_roots, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                                 float2* B1, const int32_t* tstat, const float* Kin, int64_t kstride, const float* D,
                                 float2* K_out, int32_t* status, float2* khat, float2* twtab, hipStream_t stream);
bool wave_path_fits(int64_t M);
hipError_t launch_wspectrum(bool from_roots, int64_t H, int64_t L, int64_t M, int64_t tiles, const float2* roots,
                            const int32_t* tstat, const float* Kin, int64_t kstride, const float* D,
                            float2* K_out, int32_t* status, float2* khat, float2* tw4, hipStream_t stream,
                            bool tw4_ready = false);
hipError_t launch_wconv(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y, const float2* khat,
                        const float2* tw4, hipStream_t stream);
hipError_t launch_wl_spectrum(int64_t H, int64_t L, int64_t M, int64_t tiles, float2* roots, const int32_t* tstat,
                              int32_t* status, const float* Kin, int64_t kstride, const float* D, float2* K_out,
                              float2* S, float2* tw4Q, float2* tw4M, hipStream_t stream);
hipError_t launch_wl_conv(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y, const float2* S,
                          float2* Z, const float2* tw4Q, const float2* tw4M, hipStream_t stream);
hipError_t launch_conv_large(int64_t Bsz, int64_t H, int64_t L, int64_t M, const float* u, float* y,
                             const float2* khat, float2* Z, const float2* twtab, hipStream_t stream);
hipError_t launch_discretize(int64_t H, int64_t N, int64_t r, int64_t M, const float2* Lambda, const float2* P,
                             const float2* Q, const float2* Bv, const float2* C, const float* dt, float2* Bbar,
                             float2* Abar, float2* Ct, int32_t* status, hipStream_t stream);
hipError_t launch_step(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const float2* Lambda,
                       const float2* P, const float2* Q, const float2* Bv, const float2* C, const float* dt,
                       const float* D, const float* u, float* y, float2* x, int32_t* status, int lanes,
                       hipStream_t stream);
size_t step_prepared_channel_bytes(int64_t N, int64_t r);
hipError_t launch_step_prepare(int64_t H, int64_t N, int64_t r, const float2* Lambda, const float2* P,
                               const float2* Q, const float2* Bv, const float2* C, const float* dt, uint8_t* prep,
                               int32_t* status, hipStream_t stream);
hipError_t launch_step_prepared(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const uint8_t* prep,
                                const float* D, const float* u, float* y, float2* x, int32_t* status, int lanes,
                                hipStream_t stream);
int64_t hippo_max_n();
size_t hippo_workspace_bytes(int64_t N);
hipError_t launch_hippo(int kind, int64_t N, double theta, int64_t nb, const float2* B, int64_t nc, const float2* C,
                        float2* Lam, float2* P, float2* V, float2* Bt, float2* Ct, void* ws, hipStream_t stream);
}  // namespace ssm

using namespace ssm;

namespace {

constexpr int64_t kMaxL = 65536;
constexpr int64_t kMaxR = 4;
constexpr int64_t kMaxNDisc = 4096;
constexpr int64_t kMaxNStep = 256;
constexpr int64_t kMaxDim = (int64_t)1 << 31;

int64_t pow2_at_least(int64_t v) {
    int64_t m = 1;
    while (m < v) m <<= 1;
    return m;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// size rules shared by all entry points; returns SSM_OK or an error code
int check_sizes(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, bool needs_state, bool needs_batch) {
    if (H < 1 || L < 1) return SSM_ERR_INVALID_ARGUMENT;
    if (needs_state && (N < 1 || r < 1)) return SSM_ERR_INVALID_ARGUMENT;
    if (needs_batch && Bsz < 1) return SSM_ERR_INVALID_ARGUMENT;
    if (L > kMaxL) return SSM_ERR_UNSUPPORTED;
    if (needs_state && r > kMaxR) return SSM_ERR_UNSUPPORTED;
    if (H >= kMaxDim || (needs_state && N >= kMaxDim) || (needs_batch && Bsz >= kMaxDim))
        return SSM_ERR_UNSUPPORTED;
    if (needs_batch && (Bsz * H >= kMaxDim || Bsz * H > ((int64_t)1 << 62) / L)) return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

WsLayout layout(int op, int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L) {
    WsLayout w;
    const int64_t M = pow2_at_least(L);
    size_t off = 0;
    const bool fwd = op == SSM_OP_FORWARD || op == SSM_OP_FORWARD_COMPLEX;
    if (op == SSM_OP_KERNEL_GEN || fwd) {
        w.roots = off;
        w.roots_bytes = (size_t)H * M * sizeof(float2);
        off = align256(off + w.roots_bytes);
        w.tstat = off;
        w.tstat_bytes = (size_t)H * cauchy_tiles(H, N, r, M) * sizeof(int32_t);
        off = align256(off + w.tstat_bytes);
        w.tant = off;
        w.tant_bytes = (size_t)M * sizeof(double);
        off = align256(off + w.tant_bytes);
        w.cprep = off;
        w.cprep_bytes = (size_t)cauchy_prep_bytes(H, N, r, M);
        off = align256(off + w.cprep_bytes);
    }
    if (op == SSM_OP_FFTCONV || fwd) {
        w.khat = off;
        w.khat_bytes = (size_t)H * 2 * M * sizeof(float2);
        off = align256(off + w.khat_bytes);
    }
    w.tw = off;  // every op but the discretisation keeps the twiddle table
    w.tw_bytes = (size_t)M * sizeof(float2);
    off = align256(off + w.tw_bytes);
    if (M > ((int64_t)1 << kMaxLdsLogM)) {  // multi-pass transforms
        w.big = off;
        if (op == SSM_OP_KERNEL_GEN) w.big_bytes = (size_t)H * M * sizeof(float2);  // first-pass output
        if (op == SSM_OP_FFTCONV || fwd) {  // conv intermediate: one chunk of row pairs
            const int64_t npairs = ((Bsz + 1) / 2) * H;
            w.big_bytes = (size_t)(npairs < kConvChunkPairs ? npairs : kConvChunkPairs) * 2 * M * sizeof(float2);
        }
        off = align256(off + w.big_bytes);
    }
    if ((op == SSM_OP_FFTCONV || op == SSM_OP_FORWARD) && wave_path_fits(M)) {
        w.tw4 = off;
        w.tw4_bytes = (size_t)2 * M * sizeof(float2);
        off = align256(off + w.tw4_bytes);
    }
    if ((op == SSM_OP_FFTCONV || op == SSM_OP_FORWARD) && M > ((int64_t)1 << kMaxLdsLogM)) {
        // the inner transforms' table (2 x 16384 entries), then the whole length's (2M)
        w.tw4 = off;
        w.tw4_bytes = (size_t)(2 * ((int64_t)1 << kMaxLdsLogM) + 2 * M) * sizeof(float2);
        off = align256(off + w.tw4_bytes);
    }
    if (op == SSM_OP_FORWARD_COMPLEX) {
        w.kbuf = off;
        w.kbuf_bytes = (size_t)H * L * sizeof(float2);
        off = align256(off + w.kbuf_bytes);
        if (conv_complex_fits(M)) {  // both spectra sets live at once for the shared-transform convolution
            w.khat2 = off;
            w.khat2_bytes = (size_t)H * 2 * M * sizeof(float2);
            off = align256(off + w.khat2_bytes);
        }
    }
    w.total = off;
    return w;
}

int device_status(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_DEVICE; }

// M > 16384 in the forward path: the kernel transform from the scrambled root
// values (in place on them; K written to K_out when given), then the spectrum
// of Re K + D delta_0
hipError_t launch_spectrum_wl(int64_t H, int64_t L, int64_t M, int64_t tiles, float2* roots, const int32_t* tstat,
                              const float* D, float2* K_out, int32_t* status, float2* khat, float2* tw4,
                              hipStream_t s) {
    return launch_wl_spectrum(H, L, M, tiles, roots, tstat, status, nullptr, 1, D, K_out, khat, tw4,
                              tw4 + 2 * ((int64_t)1 << kMaxLdsLogM), s);
}

}  // namespace

extern "C" {

int ssm_transform_lengths(int64_t L, int64_t* M, int64_t* n_fft) {
    if (L < 1 || L > ((int64_t)1 << 61) || !M || !n_fft) return SSM_ERR_INVALID_ARGUMENT;
    *M = pow2_at_least(L);
    *n_fft = pow2_at_least(2 * L - 1);
    return SSM_OK;
}

namespace {
int forward_form(int64_t Bsz, int64_t H, int64_t M) {
    if (M > ((int64_t)1 << kMaxLdsLogM)) return 3;
    if (single_launch_fits(Bsz, H, M)) return 1;
    return conv_fuses_spectrum(Bsz, M) ? 2 : 3;
}
}  // namespace

int ssm_forward_form(int64_t Bsz, int64_t H, int64_t L, int32_t* form) {
    if (Bsz < 1 || H < 1 || L < 1 || L > ((int64_t)1 << 61) || !form) return SSM_ERR_INVALID_ARGUMENT;
    *form = forward_form(Bsz, H, pow2_at_least(L));
    return SSM_OK;
}

const char* ssm_status_string(int code) {
    switch (code) {
        case SSM_OK: return "ok";
        case SSM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SSM_ERR_WORKSPACE: return "workspace too small";
        case SSM_ERR_DEVICE: return "device error";
        case SSM_ERR_UNSUPPORTED: return "unsupported size";
        case SSM_ERR_SCRATCH_LIMIT: return "shape needs more than the fixed no-allocation scratch";
        case SSM_ST_RESONANT_CORRECTION: return "resonant-correction";
        case SSM_ST_RESONANT_DIAGONAL: return "resonant-diagonal";
        case SSM_ST_SINGULAR_BILINEAR: return "singular-bilinear-matrix";
        case SSM_ST_INVALID_STEP: return "invalid-step";
        case SSM_ST_UNPREPARED: return "unprepared";
        default: return "unknown code";
    }
}

int ssm_workspace_bytes(int op, int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, size_t* bytes) {
    if (!bytes) return SSM_ERR_INVALID_ARGUMENT;
    if (op == SSM_OP_HIPPO) {
        if (N < 1) return SSM_ERR_INVALID_ARGUMENT;
        if (N > hippo_max_n()) return SSM_ERR_UNSUPPORTED;
        *bytes = hippo_workspace_bytes(N);
        return SSM_OK;
    }
    if (op == SSM_OP_STEP_PREPARED) {
        if (H < 1 || N < 1 || r < 1) return SSM_ERR_INVALID_ARGUMENT;
        if (r > kMaxR || N > kMaxNStep || H >= kMaxDim) return SSM_ERR_UNSUPPORTED;
        *bytes = (size_t)H * step_prepared_channel_bytes(N, r);
        return SSM_OK;
    }
    int rc;
    switch (op) {
        case SSM_OP_DISCRETIZE: rc = check_sizes(1, H, N, r, L, true, false); break;
        case SSM_OP_KERNEL_GEN: rc = check_sizes(1, H, N, r, L, true, false); break;
        case SSM_OP_FFTCONV: rc = check_sizes(Bsz, H, 1, 1, L, false, true); break;
        case SSM_OP_FORWARD:
        case SSM_OP_FORWARD_COMPLEX: rc = check_sizes(Bsz, H, N, r, L, true, true); break;
        default: return SSM_ERR_INVALID_ARGUMENT;
    }
    if (rc != SSM_OK) return rc;
    if (op == SSM_OP_DISCRETIZE && N > kMaxNDisc) return SSM_ERR_UNSUPPORTED;
    *bytes = op == SSM_OP_DISCRETIZE ? 0 : layout(op, Bsz, H, N, r, L).total;
    return SSM_OK;
}

int ssm_discretize(int64_t H, int64_t N, int64_t r, int64_t L, const ssm_c64* Lambda, const ssm_c64* P,
                   const ssm_c64* Q, const ssm_c64* B, const ssm_c64* C, const float* dt, ssm_c64* Bbar,
                   ssm_c64* Abar, ssm_c64* Ctilde, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    int rc = check_sizes(1, H, N, r, L, true, false);
    if (rc != SSM_OK) return rc;
    if (N > kMaxNDisc) return SSM_ERR_UNSUPPORTED;
    if (!Lambda || !P || !Q || !B || !dt || (Ctilde && !C)) return SSM_ERR_INVALID_ARGUMENT;
    const void* c64s[] = {Lambda, P, Q, B, C, Bbar, Abar, Ctilde};
    for (const void* p : c64s)
        if (!aligned(p, 8)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(dt, 4) || !aligned(status, 4)) return SSM_ERR_INVALID_ARGUMENT;
    const int64_t M = pow2_at_least(L);
    return device_status(launch_discretize(H, N, r, M, (const float2*)Lambda, (const float2*)P, (const float2*)Q,
                                           (const float2*)B, (const float2*)C, dt, (float2*)Bbar, (float2*)Abar,
                                           (float2*)Ctilde, status, (hipStream_t)stream));
}

int ssm_kernel_gen(int64_t H, int64_t N, int64_t r, int64_t L, const ssm_c64* Lambda, const ssm_c64* P,
                   const ssm_c64* Q, const ssm_c64* B, const ssm_c64* Ctilde, const float* dt, ssm_c64* K,
                   ssm_c64* roots_out, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sizes(1, H, N, r, L, true, false);
    if (rc != SSM_OK) return rc;
    const int64_t M = pow2_at_least(L);
    if (!Lambda || !P || !Q || !B || !Ctilde || !dt) return SSM_ERR_INVALID_ARGUMENT;
    const void* c64s[] = {Lambda, P, Q, B, Ctilde, K, roots_out};
    for (const void* p : c64s)
        if (!aligned(p, 8)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(dt, 4) || !aligned(status, 4) || !aligned(ws, 256)) return SSM_ERR_INVALID_ARGUMENT;
    const WsLayout w = layout(SSM_OP_KERNEL_GEN, 1, H, N, r, L);
    if (ws_bytes < w.total || !ws) return SSM_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (single_launch_fits(0, H, M))  // one launch: root values and kernel transform per channel workgroup
        return device_status(launch_single(0, H, N, r, L, (const float2*)Lambda, (const float2*)P,
                                           (const float2*)Q, (const float2*)B, (const float2*)Ctilde, dt, nullptr,
                                           nullptr, nullptr, (float2*)K, status, s, (float2*)roots_out));
    char* base = (char*)ws;
    float2* roots = roots_out ? (float2*)roots_out : (float2*)(base + w.roots);
    int32_t* tstat = (int32_t*)(base + w.tstat);
    float2* twtab = (float2*)(base + w.tw);
    hipError_t e = launch_cauchy(H, N, r, M, (const float2*)Lambda, (const float2*)P, (const float2*)Q,
                                 (const float2*)B, (const float2*)Ctilde, dt, roots, tstat, twtab, (double*)(base + w.tant), base + w.cprep, s,
                                 false);
    if (e != hipSuccess) return SSM_ERR_DEVICE;
    if (K || status) {  // kernel transform only: no spectra
        if (M > ((int64_t)1 << kMaxLdsLogM))
            e = launch_spectrum_large(true, H, L, M, cauchy_tiles(H, N, r, M), roots, (float2*)(base + w.big), tstat,
                                      nullptr, 1, nullptr, (float2*)K, status, nullptr, twtab, s);
        else
            e = launch_spectrum(true, H, L, M, cauchy_tiles(H, N, r, M), roots, tstat, nullptr, 1, nullptr, (float2*)K,
                                status, nullptr, twtab, s);
        if (e != hipSuccess) return SSM_ERR_DEVICE;
    }
    return SSM_OK;
}

int ssm_fftconv(int64_t Bsz, int64_t H, int64_t L, const float* K, int64_t k_stride, const float* D, const float* u,
                float* y, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sizes(Bsz, H, 1, 1, L, false, true);
    if (rc != SSM_OK) return rc;
    const int64_t M = pow2_at_least(L);
    if (!K || !u || !y || (k_stride != 1 && k_stride != 2)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(K, 4) || !aligned(D, 4) || !aligned(u, 4) || !aligned(y, 4) || !aligned(ws, 256))
        return SSM_ERR_INVALID_ARGUMENT;
    const WsLayout w = layout(SSM_OP_FFTCONV, Bsz, H, 1, 1, L);
    if (ws_bytes < w.total || !ws) return SSM_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    float2* khat = (float2*)((char*)ws + w.khat);
    float2* twtab = (float2*)((char*)ws + w.tw);
    if (M > ((int64_t)1 << kMaxLdsLogM)) {
        float2* tw4Q = (float2*)((char*)ws + w.tw4);
        float2* tw4M = tw4Q + 2 * ((int64_t)1 << kMaxLdsLogM);
        hipError_t e = launch_wl_spectrum(H, L, M, 0, nullptr, nullptr, nullptr, K, k_stride, D, nullptr, khat, tw4Q,
                                          tw4M, s);
        if (e != hipSuccess) return SSM_ERR_DEVICE;
        return device_status(
            launch_wl_conv(Bsz, H, L, M, u, y, khat, (float2*)((char*)ws + w.big), tw4Q, tw4M, s));
    }
    if (wave_path_fits(M)) {
        float2* tw4 = (float2*)((char*)ws + w.tw4);
        hipError_t e = launch_wspectrum(false, H, L, M, 0, nullptr, nullptr, K, k_stride, D, nullptr, nullptr, khat,
                                        tw4, s);
        if (e != hipSuccess) return SSM_ERR_DEVICE;
        return device_status(launch_wconv(Bsz, H, L, M, u, y, khat, tw4, s));
    }
    hipError_t e =
        launch_spectrum(false, H, L, M, 0, nullptr, nullptr, K, k_stride, D, nullptr, nullptr, khat, twtab, s);
    if (e != hipSuccess) return SSM_ERR_DEVICE;
    return device_status(launch_conv(Bsz, H, L, M, u, y, khat, twtab, s));
}

int ssm_hippo_dplr(int kind, int64_t N, double theta, int64_t nb, const ssm_c64* B, int64_t nc, const ssm_c64* C,
                   ssm_c64* Lambda, ssm_c64* P, ssm_c64* V, ssm_c64* Bt, ssm_c64* Ct, void* ws, size_t ws_bytes,
                   void* stream) {
    if (kind != SSM_HIPPO_LEGS && kind != SSM_HIPPO_LEGT && kind != SSM_HIPPO_LAGT) return SSM_ERR_INVALID_ARGUMENT;
    if (N < 1 || nb < 0 || nc < 0) return SSM_ERR_INVALID_ARGUMENT;
    if (kind == SSM_HIPPO_LEGT && !(theta > 0.0 && theta < HUGE_VAL)) return SSM_ERR_INVALID_ARGUMENT;
    if (N > hippo_max_n() || nb >= kMaxDim || nc >= kMaxDim || nb + nc >= kMaxDim) return SSM_ERR_UNSUPPORTED;
    if (!Lambda || !P || !ws || (nb > 0 && (!B || !Bt)) || (nc > 0 && (!C || !Ct))) return SSM_ERR_INVALID_ARGUMENT;
    const void* c64s[] = {B, C, Lambda, P, V, Bt, Ct};
    for (const void* p : c64s)
        if (!aligned(p, 8)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(ws, 256)) return SSM_ERR_INVALID_ARGUMENT;
    if (ws_bytes < hippo_workspace_bytes(N)) return SSM_ERR_WORKSPACE;
    return device_status(launch_hippo(kind, N, theta, nb, (const float2*)B, nc, (const float2*)C, (float2*)Lambda,
                                      (float2*)P, (float2*)V, (float2*)Bt, (float2*)Ct, ws, (hipStream_t)stream));
}

}  // extern "C"

namespace {

int forward_impl(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, const ssm_c64* Lambda, const ssm_c64* P,
                 const ssm_c64* Q, const ssm_c64* B, const ssm_c64* Ctilde, const float* dt, const float* D,
                 const float* u, float* y, ssm_c64* K_out, int32_t* status, void* ws, size_t ws_bytes, void* stream,
                 void* const* ev, int repeat) {
    int rc = check_sizes(Bsz, H, N, r, L, true, true);
    if (rc != SSM_OK) return rc;
    const int64_t M = pow2_at_least(L);
    if (!Lambda || !P || !Q || !B || !Ctilde || !dt || !u || !y) return SSM_ERR_INVALID_ARGUMENT;
    const void* c64s[] = {Lambda, P, Q, B, Ctilde, K_out};
    for (const void* p : c64s)
        if (!aligned(p, 8)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(dt, 4) || !aligned(D, 4) || !aligned(u, 4) || !aligned(y, 4) || !aligned(status, 4) ||
        !aligned(ws, 256))
        return SSM_ERR_INVALID_ARGUMENT;
    const WsLayout w = layout(SSM_OP_FORWARD, Bsz, H, N, r, L);
    if (ws_bytes < w.total || !ws) return SSM_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)ws;
    float2* roots = (float2*)(base + w.roots);
    int32_t* tstat = (int32_t*)(base + w.tstat);
    float2* khat = (float2*)(base + w.khat);
    float2* twtab = (float2*)(base + w.tw);
    auto mark = [&](int i) { return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess; };
    if (mark(0) != hipSuccess) return SSM_ERR_DEVICE;
    hipError_t e = hipSuccess;
    const int form = forward_form(Bsz, H, M);
    if (form == 1) {  // one launch: stages 2 and 3 are empty
        for (int i = 0; i < repeat && e == hipSuccess; ++i)
            e = launch_single(Bsz, H, N, r, L, (const float2*)Lambda, (const float2*)P, (const float2*)Q,
                              (const float2*)B, (const float2*)Ctilde, dt, D, u, y, (float2*)K_out, status, s);
        if (e != hipSuccess || mark(1) != hipSuccess || mark(2) != hipSuccess || mark(3) != hipSuccess)
            return SSM_ERR_DEVICE;
        return SSM_OK;
    }
    const bool large = M > ((int64_t)1 << kMaxLdsLogM);
    const bool fused = form == 2;
    const bool wave = !large && !fused && wave_path_fits(M);
    // the wave-structured transforms take the root values in their own order
    const bool scrambled = large || wave;
    // on the wave-structured path the root-value launch also writes the
    // transforms' table when it can (one launch fewer)
    bool tw4_done = false;
    for (int i = 0; i < repeat && e == hipSuccess; ++i)
        e = launch_cauchy(H, N, r, M, (const float2*)Lambda, (const float2*)P, (const float2*)Q, (const float2*)B,
                          (const float2*)Ctilde, dt, roots, tstat, twtab, (double*)(base + w.tant), base + w.cprep, s,
                          scrambled, wave ? (float2*)(base + w.tw4) : nullptr, &tw4_done);
    if (e != hipSuccess || mark(1) != hipSuccess) return SSM_ERR_DEVICE;
    // the multi-pass kernel transform works in place on the root values, so a
    // repeated stage first regenerates them (the repeat count is a timing aid)
    for (int i = 0; i < repeat && e == hipSuccess && !fused; ++i) {
        if (large && i > 0)
            e = launch_cauchy(H, N, r, M, (const float2*)Lambda, (const float2*)P, (const float2*)Q,
                              (const float2*)B, (const float2*)Ctilde, dt, roots, tstat, twtab, (double*)(base + w.tant), base + w.cprep, s,
                              scrambled);
        if (e != hipSuccess) break;
        e = large  ? launch_spectrum_wl(H, L, M, cauchy_tiles(H, N, r, M), roots, tstat, D, (float2*)K_out, status,
                                        khat, (float2*)(base + w.tw4), s)
            : wave ? launch_wspectrum(true, H, L, M, cauchy_tiles(H, N, r, M), roots, tstat, nullptr, 1, D,
                                      (float2*)K_out, status, khat, (float2*)(base + w.tw4), s, tw4_done)
                   : launch_spectrum(true, H, L, M, cauchy_tiles(H, N, r, M), roots, tstat, nullptr, 1, D,
                                     (float2*)K_out, status, khat, twtab, s);
    }
    if (e != hipSuccess || mark(2) != hipSuccess) return SSM_ERR_DEVICE;
    for (int i = 0; i < repeat && e == hipSuccess; ++i)
        e = large   ? launch_wl_conv(Bsz, H, L, M, u, y, khat, (float2*)(base + w.big), (const float2*)(base + w.tw4),
                                     (const float2*)(base + w.tw4) + 2 * ((int64_t)1 << kMaxLdsLogM), s)
            : fused ? launch_conv_fused(Bsz, H, L, M, cauchy_tiles(H, N, r, M), roots, tstat, D, (float2*)K_out,
                                        status, u, y, twtab, s)
            : wave  ? launch_wconv(Bsz, H, L, M, u, y, khat, (const float2*)(base + w.tw4), s)
                    : launch_conv(Bsz, H, L, M, u, y, khat, twtab, s);
    if (e != hipSuccess || mark(3) != hipSuccess) return SSM_ERR_DEVICE;
    return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_forward(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, const ssm_c64* Lambda, const ssm_c64* P,
                const ssm_c64* Q, const ssm_c64* B, const ssm_c64* Ctilde, const float* dt, const float* D,
                const float* u, float* y, ssm_c64* K_out, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(Bsz, H, N, r, L, Lambda, P, Q, B, Ctilde, dt, D, u, y, K_out, status, ws, ws_bytes, stream,
                        nullptr, 1);
}

int ssm_forward_profiled(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, const ssm_c64* Lambda,
                         const ssm_c64* P, const ssm_c64* Q, const ssm_c64* B, const ssm_c64* Ctilde, const float* dt,
                         const float* D, const float* u, float* y, ssm_c64* K_out, int32_t* status, void* ws,
                         size_t ws_bytes, void* stream, void* const* events, int32_t repeat) {
    if (!events || !events[0] || !events[1] || !events[2] || !events[3] || repeat < 1)
        return SSM_ERR_INVALID_ARGUMENT;
    return forward_impl(Bsz, H, N, r, L, Lambda, P, Q, B, Ctilde, dt, D, u, y, K_out, status, ws, ws_bytes, stream,
                        events, repeat);
}

int ssm_forward_complex(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, const ssm_c64* Lambda,
                        const ssm_c64* P, const ssm_c64* Q, const ssm_c64* B, const ssm_c64* Ctilde, const float* dt,
                        const float* D, const float* u, float* y_re, float* y_im, ssm_c64* K_out, int32_t* status,
                        void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sizes(Bsz, H, N, r, L, true, true);
    if (rc != SSM_OK) return rc;
    const int64_t M = pow2_at_least(L);
    if (!Lambda || !P || !Q || !B || !Ctilde || !dt || !u || !y_re || !y_im) return SSM_ERR_INVALID_ARGUMENT;
    const void* c64s[] = {Lambda, P, Q, B, Ctilde, K_out};
    for (const void* p : c64s)
        if (!aligned(p, 8)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(dt, 4) || !aligned(D, 4) || !aligned(u, 4) || !aligned(y_re, 4) || !aligned(y_im, 4) ||
        !aligned(status, 4) || !aligned(ws, 256))
        return SSM_ERR_INVALID_ARGUMENT;
    const WsLayout w = layout(SSM_OP_FORWARD_COMPLEX, Bsz, H, N, r, L);
    if (ws_bytes < w.total || !ws) return SSM_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)ws;
    float2* roots = (float2*)(base + w.roots);
    int32_t* tstat = (int32_t*)(base + w.tstat);
    float2* khat = (float2*)(base + w.khat);
    float2* twtab = (float2*)(base + w.tw);
    float2* K = K_out ? (float2*)K_out : (float2*)(base + w.kbuf);
    const bool large = M > ((int64_t)1 << kMaxLdsLogM);
    const int64_t tiles = cauchy_tiles(H, N, r, M);
    hipError_t e = launch_cauchy(H, N, r, M, (const float2*)Lambda, (const float2*)P, (const float2*)Q,
                                 (const float2*)B, (const float2*)Ctilde, dt, roots, tstat, twtab,
                                 (double*)(base + w.tant), base + w.cprep, s, false);
    // real part: the spectra of Re K + D delta_0 from the root values (K written on the way)
    if (e == hipSuccess)
        e = large ? launch_spectrum_large(true, H, L, M, tiles, roots, roots, tstat, nullptr, 1, D, K, status, khat,
                                          twtab, s)
                  : launch_spectrum(true, H, L, M, tiles, roots, tstat, nullptr, 1, D, K, status, khat, twtab, s);
    const float* Kim = (const float*)K + 1;
    if (conv_complex_fits(M)) {
        // the spectra of Im K (the odd floats of K; no skip term) beside those of
        // Re K + D delta_0, then one convolution sharing the input's transforms
        float2* khat_im = (float2*)(base + w.khat2);
        if (e == hipSuccess)
            e = launch_spectrum(false, H, L, M, 0, nullptr, nullptr, Kim, 2, nullptr, nullptr, nullptr, khat_im,
                                twtab, s);
        if (e == hipSuccess) e = launch_conv_complex(Bsz, H, L, M, u, y_re, y_im, khat, khat_im, twtab, s);
        return device_status(e);
    }
    if (e == hipSuccess)
        e = large ? launch_conv_large(Bsz, H, L, M, u, y_re, khat, (float2*)(base + w.big), twtab, s)
                  : launch_conv(Bsz, H, L, M, u, y_re, khat, twtab, s);
    // imaginary part: the spectra of Im K (the odd floats of K; no skip term)
    if (e == hipSuccess)
        e = large ? launch_spectrum_large(false, H, L, M, 0, nullptr, nullptr, nullptr, Kim, 2, nullptr, nullptr,
                                          nullptr, khat, twtab, s)
                  : launch_spectrum(false, H, L, M, 0, nullptr, nullptr, Kim, 2, nullptr, nullptr, nullptr, khat,
                                    twtab, s);
    if (e == hipSuccess)
        e = large ? launch_conv_large(Bsz, H, L, M, u, y_im, khat, (float2*)(base + w.big), twtab, s)
                  : launch_conv(Bsz, H, L, M, u, y_im, khat, twtab, s);
    return device_status(e);
}

}  // extern "C"

// Scratch of ssm_forward_noalloc: one fixed array per GPU (each device that
// loads the library holds its own copy until the process ends).  Its name is a
// host-side stand-in in host code; kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// device address of the current device's scratch array, or null on failure
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int ssm_forward_noalloc(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L, const ssm_c64* Lambda,
                        const ssm_c64* P, const ssm_c64* Q, const ssm_c64* B, const ssm_c64* Ctilde, const float* dt,
                        const float* D, const float* u, float* y, ssm_c64* K_out, int32_t* status, void* stream) {
    const int rc = check_sizes(Bsz, H, N, r, L, true, true);
    if (rc != SSM_OK) return rc;
    // every workspace region the forward path reads is written earlier in the
    // same call, so the array needs no clearing between calls
    if (layout(SSM_OP_FORWARD, Bsz, H, N, r, L).total > SSM_NOALLOC_SCRATCH_BYTES) return SSM_ERR_SCRATCH_LIMIT;
    void* ws = scratch_for_current_device();
    if (!ws) return SSM_ERR_DEVICE;
    return forward_impl(Bsz, H, N, r, L, Lambda, P, Q, B, Ctilde, dt, D, u, y, K_out, status, ws,
                        SSM_NOALLOC_SCRATCH_BYTES, stream, nullptr, 1);
}

// The step layout for lanes = 0.  16-lane groups issue fewer instructions per
// sequence step but put four sequences in a wave: they pay once at least
// three sequences per SIMD keep every SIMD busy and the call has at least
// min_T steps (to amortise a longer first step, and in ssm_step the wave's
// four set-ups).  Returns SSM_OK and sets *lanes, or SSM_ERR_DEVICE.
static int choose_step_lanes(int64_t Bsz, int64_t H, int64_t N, int64_t T, int64_t min_T, int32_t* lanes) {
    *lanes = 64;
    if (N <= 64 && T >= min_T) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return SSM_ERR_DEVICE;
        if (Bsz * H >= (int64_t)3 * 4 * cus) *lanes = 16;
    }
    return SSM_OK;
}

int ssm_step(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const ssm_c64* Lambda, const ssm_c64* P,
             const ssm_c64* Q, const ssm_c64* B, const ssm_c64* C, const float* dt, const float* D, const float* u,
             float* y, ssm_c64* x, int32_t* status, int32_t lanes, void* stream) {
    if (Bsz < 1 || H < 1 || N < 1 || r < 1 || T < 1) return SSM_ERR_INVALID_ARGUMENT;
    if (!(lanes == 0 || lanes == 64 || (lanes == 16 && N <= 64))) return SSM_ERR_INVALID_ARGUMENT;
    if (r > kMaxR || N > kMaxNStep || H >= kMaxDim || Bsz >= kMaxDim || T >= kMaxDim || Bsz * H >= kMaxDim ||
        Bsz * H > ((int64_t)1 << 62) / T)
        return SSM_ERR_UNSUPPORTED;
    if (!Lambda || !P || !Q || !B || !C || !dt || !u || !y || !x) return SSM_ERR_INVALID_ARGUMENT;
    const void* c64s[] = {Lambda, P, Q, B, C, x};
    for (const void* p : c64s)
        if (!aligned(p, 8)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(dt, 4) || !aligned(D, 4) || !aligned(u, 4) || !aligned(y, 4) || !aligned(status, 4))
        return SSM_ERR_INVALID_ARGUMENT;
    if (lanes == 0) {
        const int rc = choose_step_lanes(Bsz, H, N, T, 32, &lanes);
        if (rc != SSM_OK) return rc;
    }
    return device_status(launch_step(Bsz, H, N, r, T, (const float2*)Lambda, (const float2*)P, (const float2*)Q,
                                     (const float2*)B, (const float2*)C, dt, D, u, y, (float2*)x, status, lanes,
                                     (hipStream_t)stream));
}

int ssm_step_prepare(int64_t H, int64_t N, int64_t r, const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
                     const ssm_c64* B, const ssm_c64* C, const float* dt, void* prep, size_t prep_bytes,
                     int32_t* status, void* stream) {
    if (H < 1 || N < 1 || r < 1) return SSM_ERR_INVALID_ARGUMENT;
    if (r > kMaxR || N > kMaxNStep || H >= kMaxDim) return SSM_ERR_UNSUPPORTED;
    if (!Lambda || !P || !Q || !B || !C || !dt || !prep) return SSM_ERR_INVALID_ARGUMENT;
    const void* c64s[] = {Lambda, P, Q, B, C};
    for (const void* p : c64s)
        if (!aligned(p, 8)) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(dt, 4) || !aligned(status, 4) || !aligned(prep, 256)) return SSM_ERR_INVALID_ARGUMENT;
    if (prep_bytes < (size_t)H * step_prepared_channel_bytes(N, r)) return SSM_ERR_WORKSPACE;
    return device_status(launch_step_prepare(H, N, r, (const float2*)Lambda, (const float2*)P, (const float2*)Q,
                                             (const float2*)B, (const float2*)C, dt, (uint8_t*)prep, status,
                                             (hipStream_t)stream));
}

int ssm_step_prepared(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T, const void* prep, size_t prep_bytes,
                      const float* D, const float* u, float* y, ssm_c64* x, int32_t* status, int32_t lanes,
                      void* stream) {
    if (Bsz < 1 || H < 1 || N < 1 || r < 1 || T < 1) return SSM_ERR_INVALID_ARGUMENT;
    if (!(lanes == 0 || lanes == 64 || (lanes == 16 && N <= 64))) return SSM_ERR_INVALID_ARGUMENT;
    if (r > kMaxR || N > kMaxNStep || H >= kMaxDim || Bsz >= kMaxDim || T >= kMaxDim || Bsz * H >= kMaxDim ||
        Bsz * H > ((int64_t)1 << 62) / T)
        return SSM_ERR_UNSUPPORTED;
    if (!prep || !u || !y || !x) return SSM_ERR_INVALID_ARGUMENT;
    if (!aligned(prep, 256) || !aligned(x, 8) || !aligned(D, 4) || !aligned(u, 4) || !aligned(y, 4) ||
        !aligned(status, 4))
        return SSM_ERR_INVALID_ARGUMENT;
    if (prep_bytes < (size_t)H * step_prepared_channel_bytes(N, r)) return SSM_ERR_WORKSPACE;
    if (lanes == 0) {
        const int rc = choose_step_lanes(Bsz, H, N, T, 8, &lanes);
        if (rc != SSM_OK) return rc;
    }
    return device_status(launch_step_prepared(Bsz, H, N, r, T, (const uint8_t*)prep, D, u, y, (float2*)x, status,
                                              lanes, (hipStream_t)stream));
}

}  // extern "C"
