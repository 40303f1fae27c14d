/*
 * ssm.h -- C ABI of the MI355X (gfx950) S4 DPLR filter library.
 *
 * The library computes, for H independent single-input single-output channels
 * of a diagonal-plus-low-rank (DPLR) state-space model, the bilinear
 * discretisation, the length-L convolution kernel by the filter-mode
 * evaluation at the M roots of unity, and the causal convolution
 * y = K * u + D u.  Passages defining each operation are cited by page title
 * and block:
 *   [RSS] "Recurrent, LSTM, and structured state-space models"
 *         (blocks: continuous-time linear SSM; DPLR parameterisation;
 *          radix-two DFT; Woodbury inverse; S4 Algorithm 1 / App. C)
 *   [EX]  "Recurrent, LSTM, and structured state-space models -- Examples"
 *         (the scalar example A = 0, B = C = 1, dt = 1)
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.  Complex numbers are interleaved
 *     {float re, im} (ssm_c64, the layout of torch.complex64).  Arrays are
 *     row-major with the last index fastest.  Complex arrays must be 8-byte
 *     aligned, float/int arrays 4-byte aligned, the workspace 256-byte aligned.
 *   - Per-channel parameters: Lambda [H,N], P [H,N,r], Q [H,N,r], B [H,N],
 *     C or Ctilde [H,N] (ssm_c64); dt [H], D [H] (float).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on `stream` and returns; results are ready
 *     when the stream reaches that point.  Calls are reentrant; calls that
 *     share a workspace must be ordered on one stream.
 *   - The return value reports host-detectable errors only (SSM_ERR_*).  When
 *     it is not SSM_OK nothing was enqueued.  Data-dependent conditions are
 *     reported per channel through the optional device array `status` [H]
 *     (int32, SSM_ST_*); a channel with a nonzero status has every one of its
 *     outputs filled with NaN.
 *   - Sizes: H >= 1, N >= 1, 1 <= r <= 4, 1 <= L <= 65536, Bsz >= 1;
 *     ssm_discretize also needs N <= 4096.  Other sizes give
 *     SSM_ERR_INVALID_ARGUMENT (non-positive) or SSM_ERR_UNSUPPORTED (above
 *     these caps).
 *   - M = least power of two >= L; the zero-padded product length is the least
 *     power of two >= 2L - 1 ([RSS] filter-mode block; radix-two DFT block).
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ssm_c64 {
    float re;
    float im;
} ssm_c64;

/* Return codes (host side). */
#define SSM_OK 0
#define SSM_ERR_INVALID_ARGUMENT 1 /* null required pointer, bad size, misalignment */
#define SSM_ERR_WORKSPACE 2        /* ws_bytes below ssm_workspace_bytes() */
#define SSM_ERR_DEVICE 3           /* a HIP call or kernel launch failed */
#define SSM_ERR_UNSUPPORTED 4      /* valid for the method, above this library's caps */
#define SSM_ERR_SCRATCH_LIMIT 5    /* ssm_forward_noalloc: the shape needs more scratch than
                                      SSM_NOALLOC_SCRATCH_BYTES */

/* Per-channel statuses (device int32).  When several hold, the largest code
 * is reported. */
#define SSM_ST_OK 0
#define SSM_ST_RESONANT_CORRECTION 16 /* W(z_k) = I_r + Q^* R(z_k) P exactly singular, [RSS] Alg. 1 */
#define SSM_ST_RESONANT_DIAGONAL 17   /* s(z_k) - lambda_j exactly zero, [RSS] Alg. 1 */
#define SSM_ST_SINGULAR_BILINEAR 18   /* G = I - dt A/2 singular, [RSS] recurrent solver */
#define SSM_ST_INVALID_STEP 19        /* dt not finite and positive ([RSS] requires dt > 0) */
#define SSM_ST_UNPREPARED 20          /* ssm_step_prepared: the channel's block was not written by
                                         ssm_step_prepare for these N and r */

/* Operation ids for ssm_workspace_bytes. */
#define SSM_OP_DISCRETIZE 0
#define SSM_OP_KERNEL_GEN 1
#define SSM_OP_FFTCONV 2
#define SSM_OP_FORWARD 3
#define SSM_OP_FORWARD_COMPLEX 4
#define SSM_OP_HIPPO 5           /* ssm_hippo_dplr: only N is read */
#define SSM_OP_STEP_PREPARED 6   /* the constants ssm_step_prepare writes: H, N, r read */

/*
 * Workspace size in bytes that entry point `op` needs for these sizes (Bsz is
 * ignored by ops that take no batch; N and r are ignored by SSM_OP_FFTCONV).
 * Writes *bytes and returns SSM_OK, or returns SSM_ERR_INVALID_ARGUMENT /
 * SSM_ERR_UNSUPPORTED under the size rules above (then *bytes is untouched).
 */
int ssm_workspace_bytes(int op, int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L,
                        size_t* bytes);

/* Transform sizes for a kernel length L >= 1 ([RSS] filter-mode block):
 * *M = least power of two >= L; *n_fft = least power of two >= 2L - 1.
 * Pure integer host computation; SSM_ERR_INVALID_ARGUMENT for L < 1. */
int ssm_transform_lengths(int64_t L, int64_t* M, int64_t* n_fft);

/* Launch form ssm_forward takes for Bsz rows, H channels and kernel length L:
 *   *form = 1: one launch (one workgroup per channel computes root values,
 *              kernel, spectra and all its rows' convolutions; M = 1024, at
 *              most 8 rows, H >= 256);
 *   *form = 2: root values, then a convolution kernel that forms the spectra
 *              itself (M <= 1024, at most 8 rows);
 *   *form = 3: root values, kernel transform + spectra, convolution (multi-pass
 *              transforms above M = 16384).
 * Informational only: the results are the same in every form.  Pure host
 * computation; SSM_ERR_INVALID_ARGUMENT for Bsz, H or L < 1 or null. */
int ssm_forward_form(int64_t Bsz, int64_t H, int64_t L, int32_t* form);

/* Static description of a return code or status code (never NULL). */
const char* ssm_status_string(int code);

/*
 * Bilinear discretisation ([RSS] DPLR block; recurrent solver of Alg. 1).
 * Per channel, with alpha = dt/2, G = I - alpha A, A = diag(Lambda) - P Q^*:
 *   Bbar = G^{-1} dt B                      -> Bbar   [H,N]   (nullable)
 *   Abar = G^{-1}(I + alpha A) = 2G^{-1} - I -> Abar   [H,N,N] (nullable, row-major)
 *   Ctilde = (I - Abar^M)^* C, M from L      -> Ctilde [H,N]   (nullable)
 * G is applied through the Woodbury core I_r + alpha Q^* D^{-1} P when every
 * d_j = 1 - alpha lambda_j is nonzero, else through the pages' bordered system
 * when at most r of them are zero; a singular core or bordered system, or more
 * than r zero d_j, gives SSM_ST_SINGULAR_BILINEAR.  Arithmetic is float64
 * inside; outputs are rounded to complex64.  Ctilde is formed by M adjoint
 * steps c <- Abar^* c (latency-bound, one wavefront per channel).
 * Workspace: none (pass ws = NULL, ws_bytes = 0).
 */
int ssm_discretize(int64_t H, int64_t N, int64_t r, int64_t L,
                   const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
                   const ssm_c64* B, const ssm_c64* C, const float* dt,
                   ssm_c64* Bbar, ssm_c64* Abar, ssm_c64* Ctilde, int32_t* status,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Filter-mode kernel generation ([RSS] Alg. 1 filter mode).
 * Ctilde is the supplied truncated-output vector (I - Abar^M)^* C.  For each
 * root z_k = exp(-2 pi i k/M): at z_k = -1 the value is (dt/2) Ctilde^* B;
 * otherwise H(z_k) = 2/(1+z_k) (Ctilde^* R B - Ctilde^* R P W^{-1} Q^* R B) with
 * R = diag(1/(s(z_k) - lambda_j)), s(z) = (2/dt)(1-z)/(1+z), W = I_r + Q^* R P.
 * The kernel is the first L coefficients of the inverse transform
 * K_j = (1/M) sum_k H(z_k) exp(+2 pi i jk/M).
 *   K         [H,L] complex64, nullable
 *   roots_out [H,M] complex64, nullable: the root values H(z_k) themselves
 *   status    [H] int32, nullable
 * Workspace: ssm_workspace_bytes(SSM_OP_KERNEL_GEN, ...).
 */
int ssm_kernel_gen(int64_t H, int64_t N, int64_t r, int64_t L,
                   const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
                   const ssm_c64* B, const ssm_c64* Ctilde, const float* dt,
                   ssm_c64* K, ssm_c64* roots_out, int32_t* status,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Causal convolution with skip term ([RSS] DPLR block: y_t = sum_{j<=t} K_j
 * u_{t-j} + D u_t; radix-two DFT block: exact product by zero padding to
 * length >= 2L - 1; [EX] convolution equals the recurrence).
 *   K  real kernel: element (h, j) at K[(h*L + j) * k_stride]; k_stride = 1 for
 *      a float [H,L] array, 2 to read the real parts of a complex64 [H,L] array
 *   D  [H] float, nullable (= 0)
 *   u  [Bsz,H,L] float, y [Bsz,H,L] float (y must not overlap u)
 * Workspace: ssm_workspace_bytes(SSM_OP_FFTCONV, ...).
 */
int ssm_fftconv(int64_t Bsz, int64_t H, int64_t L, const float* K, int64_t k_stride,
                const float* D, const float* u, float* y,
                void* ws, size_t ws_bytes, void* stream);

/*
 * The whole filter path: ssm_kernel_gen from the supplied Ctilde, then
 * y = (Re K) * u + D u ([RSS] DPLR block: y_t = C^* x_t + D u_t, real part).
 *   u, y [Bsz,H,L] float; D [H] float (nullable = 0)
 *   K_out [H,L] complex64, nullable; status [H] int32, nullable
 * Workspace: ssm_workspace_bytes(SSM_OP_FORWARD, ...).
 */
int ssm_forward(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L,
                const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
                const ssm_c64* B, const ssm_c64* Ctilde, const float* dt, const float* D,
                const float* u, float* y, ssm_c64* K_out, int32_t* status,
                void* ws, size_t ws_bytes, void* stream);

/*
 * The whole filter path with the complex output ([RSS] DPLR block: y_t = C^* x_t
 * + D u_t is complex for a complex C; with D real its imaginary part is
 * Im(C^* x_t) = (Im K) * u):
 *   y_re = (Re K) * u + D u   (as ssm_forward's y)
 *   y_im = (Im K) * u
 * Root values once; then the spectra of Re K (+ D, from the root values, which
 * also writes K) and the spectra of Im K (read back from K).  For M <= 1024
 * and M = 4096 one convolution shares the input's forward transforms between
 * both spectra sets; other lengths run a convolution for each.  y_re and y_im
 * [Bsz,H,L] float must not overlap u or each other.  K_out nullable (then K goes to the workspace).  Workspace:
 * ssm_workspace_bytes(SSM_OP_FORWARD_COMPLEX, ...).
 */
int ssm_forward_complex(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L,
                        const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
                        const ssm_c64* B, const ssm_c64* Ctilde, const float* dt, const float* D,
                        const float* u, float* y_re, float* y_im, ssm_c64* K_out, int32_t* status,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * ssm_forward with per-kernel timing marks for benchmarks and profilers.
 * Same results; the three stages (root values; kernel transform and spectra;
 * convolution) are each launched `repeat` >= 1 times in a row (every stage is
 * idempotent), and four caller-created hipEvent_t (passed as void*) are
 * recorded on `stream`: events[0] before the first stage, events[i] after
 * stage i.  (events[i] - events[i-1]) / repeat is then a stage's duration per
 * launch with the dispatch gaps amortised.  In form 2 (ssm_forward_form) stage
 * 2 launches nothing and stage 3 includes the kernel transform; in form 1 stage
 * 1 is the single launch and stages 2 and 3 are empty.  events must not be
 * NULL.
 */
int ssm_forward_profiled(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L,
                         const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
                         const ssm_c64* B, const ssm_c64* Ctilde, const float* dt, const float* D,
                         const float* u, float* y, ssm_c64* K_out, int32_t* status,
                         void* ws, size_t ws_bytes, void* stream, void* const* events, int32_t repeat);

/*
 * ssm_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, results and arguments as ssm_forward except that there is
 * no workspace argument.  The scratch lives in a fixed device array of
 * SSM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * first call on that GPU until the process ends; the call itself allocates and
 * frees nothing.  Shapes whose ssm_workspace_bytes(SSM_OP_FORWARD, ...) exceeds
 * that size give SSM_ERR_SCRATCH_LIMIT (nothing enqueued).  Every call on one
 * GPU uses the same array: calls that overlap on one GPU (several streams or
 * threads at once) race and must be ordered by the caller, e.g. on one stream.
 * The first call on a device must not be made during graph capture (it looks
 * up the array's device address once, a host-side query).
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssm_forward_noalloc(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t L,
                        const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
                        const ssm_c64* B, const ssm_c64* Ctilde, const float* dt, const float* D,
                        const float* u, float* y, ssm_c64* K_out, int32_t* status, void* stream);

/*
 * Recurrent (step) mode ([RSS] DPLR block: x_t = Abar x_{t-1} + Bbar u_t,
 * y_t = C^* x_t + D u_t; recurrent solver of Alg. 1): T steps of the bilinear
 * recurrence for each of Bsz x H sequences, starting from the state in x and
 * leaving the state after the last step there, so that successive calls
 * continue one stream.  Abar is never formed: each step solves with
 * G = I - (dt/2) A in O(N r) through the Woodbury core, or through the pages'
 * bordered system when some d_j = 1 - (dt/2) lambda_j is exactly zero
 * (x_t = 2 G^{-1} x_{t-1} - x_{t-1} + Bbar u_t).  The channel set-up (d, the
 * core's inverse, Bbar) is float64; the recurrence is float32.
 *   C    [H,N] complex64: the output vector itself (not C~)
 *   u, y [Bsz,H,T] float: y_t = Re(C^* x_t) + D u_t
 *   x    [Bsz,H,N] complex64, in/out (zeros for a fresh stream)
 *   D    [H] float, nullable (= 0); status [H] int32, nullable
 *   lanes  lanes of a wave per sequence: 64 (one sequence per wave, which
 *          runs its channel's set-up itself), 16 (N <= 64 only: four
 *          sequences per wave, fewer instructions per step; the wave runs its
 *          four channels' set-ups in turn, and the sums are taken in another
 *          order, so the float32 results differ from the 64-lane ones by
 *          rounding), or 0 (chosen per call: 16 when N <= 64, T >= 32 and
 *          Bsz * H is at least three sequences per SIMD of the device, else
 *          64).  A stream split into calls repeats one call's results bit for
 *          bit when every call takes the same layout.  Anything else:
 *          SSM_ERR_INVALID_ARGUMENT.
 * Statuses: invalid-step, singular-bilinear (as ssm_discretize); a failing
 * channel's y and x are filled with NaN.  Sizes: as above with T in place of
 * L (T >= 1, any length below 2^31) and N <= 256.  No workspace.
 */
int ssm_step(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T,
             const ssm_c64* Lambda, const ssm_c64* P, const ssm_c64* Q,
             const ssm_c64* B, const ssm_c64* C, const float* dt, const float* D,
             const float* u, float* y, ssm_c64* x, int32_t* status, int32_t lanes,
             void* stream);

/*
 * The recurrent mode in two calls, for streaming decode: the channel set-up
 * of ssm_step (d, the Woodbury or bordered core's inverse, Bbar; float64,
 * rounded to float32) runs once per parameter set in ssm_step_prepare, which
 * writes the float32 constants of the recurrence to a caller-owned buffer of
 * ssm_workspace_bytes(SSM_OP_STEP_PREPARED, 0, H, N, r, 0) bytes.  Each
 * ssm_step_prepared call then runs only the recurrence ([RSS] DPLR block and
 * recurrent solver of Alg. 1, as ssm_step) from those constants.
 *   ssm_step_prepare:  parameters as ssm_step; prep [prep_bytes] device,
 *                      written; status [H] int32, nullable (as ssm_step's
 *                      set-up statuses).  A failing channel's block records
 *                      its status.
 *   ssm_step_prepared: prep as written by ssm_step_prepare for the same H, N
 *                      and r (read only; one buffer may serve any number of
 *                      calls and streams); D, u, y, x, status as ssm_step.
 *                      A channel whose block holds a failure status gets it
 *                      again with NaN y and x; a block not written for these
 *                      N and r gives SSM_ST_UNPREPARED, NaN y and x.
 *   lanes              as ssm_step's, with 0 choosing 16 from T >= 8 (no
 *                      set-up to amortise).  In either fixed layout y and x
 *                      equal ssm_step's in that layout bit for bit (the same
 *                      float32 constants and recurrence).
 * Sizes as ssm_step.  SSM_ERR_WORKSPACE when prep_bytes is below the size.
 */
int ssm_step_prepare(int64_t H, int64_t N, int64_t r, const ssm_c64* Lambda, const ssm_c64* P,
                     const ssm_c64* Q, const ssm_c64* B, const ssm_c64* C, const float* dt,
                     void* prep, size_t prep_bytes, int32_t* status, void* stream);
int ssm_step_prepared(int64_t Bsz, int64_t H, int64_t N, int64_t r, int64_t T,
                      const void* prep, size_t prep_bytes, const float* D, const float* u,
                      float* y, ssm_c64* x, int32_t* status, int32_t lanes, void* stream);

/* HiPPO generators for ssm_hippo_dplr. */
#define SSM_HIPPO_LEGS 0
#define SSM_HIPPO_LEGT 1
#define SSM_HIPPO_LAGT 2

/*
 * DPLR parameters of a HiPPO generator ([RSS] block on the HiPPO generators,
 * S4 Theorem 1 and App. C.1, HiPPO sec. 2.3 and App. D.1-D.3; [RSS] DPLR
 * block: NPLR form and the unitary state change).  For the N x N generator G
 * (LegS, LegT with window theta, or LagT) and the page's similarity S (the
 * identity, or diag(sqrt(2n+1)) diag((-1)^n) for LegT), S^{-1} G S is split
 * as (c I + K) - U U^T, K skew-symmetric, with
 *   LegS: c = -1/2, U [N,1], u_n = sqrt(n + 1/2);
 *   LagT: c = -1/2, U [N,1], u_n = sqrt(1/2);
 *   LegT: c = 0, U [N,2], sqrt((2n+1)/theta) in column n mod 2, 0 elsewhere.
 * With the unitary eigenvectors V of c I + K, the model (G, B, C) becomes
 * (diag(Lambda) - P P^*, V^* S^{-1} B, V^* S C) under x = S V x~, so the
 * outputs feed the other entry points with Q = P.
 *   theta       LegT window (finite, > 0); ignored for LegS and LagT
 *   B [nb,N], C [nc,N]  input rows (complex64; nb, nc >= 0, may be 0)
 *   Lambda [N]  eigenvalues c - i mu_j by ascending imaginary part
 *   P [N,rank]  V^* U, rank 1 (LegS, LagT) or 2 (LegT); column 0 is real and
 *               non-negative, which fixes each eigenvector's phase
 *   V [N,N]     eigenvectors as columns, nullable
 *   Bt [nb,N], Ct [nc,N]  the transformed rows
 * Arithmetic is float64 on the device (Householder tridiagonalisation of K,
 * Sturm-count bisection, inverse iteration, back-transformation); outputs
 * are rounded to complex64.  Sizes: 1 <= N <= 1024 (SSM_ERR_UNSUPPORTED
 * above).  Workspace: ssm_workspace_bytes(SSM_OP_HIPPO, 0, 0, N, 0, 0, ...),
 * 32 N^2 bytes plus a little.  No status: for these generators and sizes
 * adjacent eigenvalues differ by more than 5e-7 of the largest magnitude.
 */
int ssm_hippo_dplr(int kind, int64_t N, double theta,
                   int64_t nb, const ssm_c64* B, int64_t nc, const ssm_c64* C,
                   ssm_c64* Lambda, ssm_c64* P, ssm_c64* V, ssm_c64* Bt, ssm_c64* Ct,
                   void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
