"""Plain complex128 CPU oracle for the S4 DPLR filter path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check of the entry
script and the benchmark's CPU-baseline leg may import or run this module.  It
shares no code with the HIP library (no kernels, headers, tables or constants)
and imports nothing but numpy.  Every function is written for clarity, not
speed: dense matrices, explicit loops, library solves and matrix powers.

Source pages (cited by title and block):
  [RSS]  "Recurrent, LSTM, and structured state-space models"
         - block "Continuous-time linear state-space model" (S4 sec. 2.1):
           SSM x' = Ax + Bu, y = Cx + Du, D is a separate direct term;
         - block "DPLR structured state-space parameterization" (S4 sec. 2.1,
           2.3, 3.2, App. C.3): SISO complex SSM y = C^* x, A = Lambda - P Q^*,
           bilinear matrices, the discrete recurrence, the kernel K_L and the
           truncated-output vector C~_M = (I - Abar^M)^* C;
         - block "Radix-two discrete Fourier transform" (S4 App. C.2):
           the forward/inverse DFT and its radix-two recursion, F^* F = M I,
           zero-padded polynomial products;
         - block "Woodbury inverse for a diagonal-plus-low-rank update"
           (S4 App. C.2-C.3);
         - block for S4 Algorithm 1 / App. C: the recurrent solver, the filter
           mode with root values H(z_k), the z = -1 formula, the mu-form
           Cauchy products and the statuses resonant-diagonal,
           resonant-correction and singular-bilinear-matrix;
         - block on the Cauchy matrix-vector product at the roots of unity
           and the theorem on its operation count: the balanced product
           tree, the fold modulo z^M - 1, the odd-s reindexing and the
           collision status.
  [EX]   "Recurrent, LSTM, and structured state-space models -- Examples",
         the scalar example A = 0, B = C = 1, dt = 1, D = 0 (S4 sec. 2.3-2.4).

Readings where the pages are silent (each also listed in the design notes):
  * y_t = C^* x_t + D u_t is complex; the library returns its real part.
  * Zero tests (singular pivots, resonances) are exact comparisons with 0.
  * The Woodbury formula's displayed identity is lost in the page text; the
    standard form (D + U V^*)^{-1} = D^{-1} - D^{-1} U W^{-1} V^* D^{-1},
    W = I_r + V^* D^{-1} U, is used.

Parity pins for every function live in tests/test_oracle_pins.py (the
product tree's in tests/test_product_tree_oracle.py); each is checked against
closed forms, the worked example, brute force on tiny inputs or an
independent library routine.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

OK = "ok"
SINGULAR_BILINEAR = "singular-bilinear-matrix"
RESONANT_DIAGONAL = "resonant-diagonal"
RESONANT_CORRECTION = "resonant-correction"

# precedence when several conditions hold in one channel (reading of the pages:
# a channel whose bilinear step is undefined has no kernel at all; a diagonal
# resonance makes R(z) undefined before W(z) can be formed)
_PRECEDENCE = {OK: 0, RESONANT_CORRECTION: 1, RESONANT_DIAGONAL: 2, SINGULAR_BILINEAR: 3}


def worst_status(*statuses):
    return max(statuses, key=lambda s: _PRECEDENCE[s]) if statuses else OK


# ---------------------------------------------------------------------------
# Integer sizes  ([RSS] filter-mode block: M is the least power of two >= L;
# [RSS] DFT block: an exact product needs a radix-two length >= 2n - 1)
# ---------------------------------------------------------------------------
def transform_length(L: int) -> int:
    """Least power of two M with M >= L (L >= 1)."""
    if L < 1:
        raise ValueError("L must be >= 1")
    M = 1
    while M < L:
        M *= 2
    return M


def conv_length(L: int) -> int:
    """Least power of two >= 2L - 1 (the zero-padded product length)."""
    return transform_length(2 * L - 1)


# ---------------------------------------------------------------------------
# Model and discretisation  ([RSS] DPLR block)
# ---------------------------------------------------------------------------
def dplr_matrix(Lambda, P, Q):
    """A = diag(Lambda) - P Q^*  (P, Q of shape [N, r])."""
    Lambda = np.asarray(Lambda, np.complex128)
    P = np.asarray(P, np.complex128).reshape(len(Lambda), -1)
    Q = np.asarray(Q, np.complex128).reshape(len(Lambda), -1)
    return np.diag(Lambda) - P @ Q.conj().T


def bilinear(A, B, dt):
    """Bilinear matrices Abar = G^{-1}(I + dt A/2), Bbar = G^{-1} dt B with
    G = I - dt A / 2.  Returns (Abar, Bbar, status); an exactly singular G
    (LAPACK reports a zero pivot) gives status singular-bilinear-matrix."""
    A = np.asarray(A, np.complex128)
    N = A.shape[0]
    I = np.eye(N, dtype=np.complex128)
    alpha = dt / 2.0
    G = I - alpha * A
    try:
        Abar = np.linalg.solve(G, I + alpha * A)
        Bbar = np.linalg.solve(G, dt * np.asarray(B, np.complex128))
    except np.linalg.LinAlgError:
        return None, None, SINGULAR_BILINEAR
    return Abar, Bbar, OK


def kernel_by_iteration(Abar, Bbar, C, length):
    """K_j = C^* Abar^j Bbar for j < length, by v <- Abar v from v = Bbar."""
    C = np.asarray(C, np.complex128)
    v = np.asarray(Bbar, np.complex128).copy()
    K = np.empty(length, np.complex128)
    for j in range(length):
        K[j] = np.vdot(C, v)          # vdot conjugates its first argument
        v = Abar @ v
    return K


def kernel_by_matrix_power(Abar, Bbar, C, length):
    """K_j = C^* Abar^j Bbar with each power formed literally (tiny N only)."""
    C = np.asarray(C, np.complex128)
    return np.array([np.vdot(C, np.linalg.matrix_power(Abar, j) @ Bbar)
                     for j in range(length)], dtype=np.complex128)


def truncated_output(Abar, C, M):
    """C~_M = (I - Abar^M)^* C."""
    N = Abar.shape[0]
    T = np.eye(N, dtype=np.complex128) - np.linalg.matrix_power(Abar, M)
    return T.conj().T @ np.asarray(C, np.complex128)


def recurrence(Abar, Bbar, C, D, u):
    """x_{-1} = 0, x_t = Abar x_{t-1} + Bbar u_t, y_t = C^* x_t + D u_t.

    u has shape [..., L] (leading batch dims allowed); returns complex y of the
    same shape."""
    u = np.asarray(u, np.float64)
    batch_shape, L = u.shape[:-1], u.shape[-1]
    ub = u.reshape(-1, L)                                   # [b, L]
    x = np.zeros((Abar.shape[0], ub.shape[0]), np.complex128)
    y = np.empty(ub.shape, np.complex128)
    Cc = np.asarray(C, np.complex128).conj()
    Bb = np.asarray(Bbar, np.complex128)[:, None]
    for t in range(L):
        x = Abar @ x + Bb * ub[None, :, t]
        y[:, t] = Cc @ x + D * ub[:, t]
    return y.reshape(batch_shape + (L,))


def recurrence_from(Abar, Bbar, C, D, u, x0):
    """The recurrence of one sequence from a given state ([RSS] DPLR block,
    the discrete recurrence; the step mode carries the state between calls):
    x_{-1} = x0, x_t = Abar x_{t-1} + Bbar u_t, y_t = C^* x_t + D u_t, t < T.

    u: [T]; x0: [N].  Returns (complex y [T], the state x_{T-1} [N])."""
    u = np.asarray(u, np.float64)
    x = np.array(x0, np.complex128)
    Cc = np.asarray(C, np.complex128).conj()
    Bb = np.asarray(Bbar, np.complex128)
    y = np.empty(len(u), np.complex128)
    for t in range(len(u)):
        x = Abar @ x + Bb * u[t]
        y[t] = Cc @ x + D * u[t]
    return y, x


def causal_conv(K, u, D):
    """y_t = sum_{j<=t} K_j u_{t-j} + D u_t.

    The double sum runs as a loop over the lag j, each lag added to every t >= j
    at once (same terms, same order per output).  u: [..., L]; K: [>= L]."""
    K = np.asarray(K)
    u = np.asarray(u, np.float64)
    L = u.shape[-1]
    y = (D * u).astype(np.result_type(K.dtype, np.float64))
    for j in range(L):
        y[..., j:] += K[j] * u[..., :L - j]
    return y


def causal_conv_at(K, u, D, t):
    """One output of the causal convolution: sum_{j<=t} K_j u_{t-j} + D u_t
    for a single row u [L]."""
    K = np.asarray(K)
    u = np.asarray(u, np.float64)
    return np.sum(K[:t + 1] * u[t::-1]) + D * u[t]


# ---------------------------------------------------------------------------
# Fourier transforms  ([RSS] radix-two DFT block)
# ---------------------------------------------------------------------------
def _primitive_root(M, inverse):
    if M == 1:
        return 1.0 + 0.0j
    w = np.exp(-2j * np.pi / M)
    return np.conj(w) if inverse else w


def _radix2(a, w):
    M = len(a)
    if M == 1:
        return [a[0]]
    E = _radix2(a[0::2], w * w)
    O = _radix2(a[1::2], w * w)
    out = [0j] * M
    wk = 1.0 + 0.0j
    for k in range(M // 2):
        t = wk * O[k]
        out[k] = E[k] + t
        out[k + M // 2] = E[k] - t
        wk = wk * w
    return out


def radix2_dft(a, inverse=False):
    """Forward DFT a^_k = sum_j a_j w^{jk}, w = e^{-2 pi i/M}, by the radix-two
    recursion on even/odd halves; the inverse runs it with conj(w) and divides
    by M.  len(a) must be a power of two.  Pure Python: small M only."""
    a = [complex(x) for x in np.asarray(a, np.complex128)]
    M = len(a)
    if M < 1 or (M & (M - 1)) != 0:
        raise ValueError("length must be a power of two")
    # each level squares the root it was given; the recursion needs the root
    # of the current length, so feed e^{-2 pi i / M} (or its conjugate)
    out = _radix2(a, _primitive_root(M, inverse))
    out = np.array(out, np.complex128)
    return out / M if inverse else out


def dft_matrix(M):
    """F_kj = w^{jk}, w = e^{-2 pi i/M} (w = 1 when M = 1)."""
    j = np.arange(M)
    return np.exp(-2j * np.pi * np.outer(j, j) / M) if M > 1 else np.ones((1, 1), complex)


def dft_direct(a, inverse=False):
    """O(M^2) DFT by the definition (any length)."""
    a = np.asarray(a, np.complex128)
    M = len(a)
    F = dft_matrix(M)
    return (F.conj() @ a) / M if inverse else F @ a


# ---------------------------------------------------------------------------
# Woodbury identity  ([RSS] Woodbury block, standard form restored)
# ---------------------------------------------------------------------------
def woodbury_inverse(d, U, V):
    """(diag(d) + U V^*)^{-1} via D^{-1} - D^{-1} U W^{-1} V^* D^{-1},
    W = I_r + V^* D^{-1} U.  Raises LinAlgError when W is singular."""
    d = np.asarray(d, np.complex128)
    U = np.asarray(U, np.complex128)
    V = np.asarray(V, np.complex128)
    Dinv = np.diag(1.0 / d)
    W = np.eye(U.shape[1], dtype=np.complex128) + V.conj().T @ Dinv @ U
    return Dinv - Dinv @ U @ np.linalg.solve(W, V.conj().T @ Dinv)


# ---------------------------------------------------------------------------
# Filter mode: root values  ([RSS] Algorithm-1 block)
# ---------------------------------------------------------------------------
def roots_of_unity(M):
    """z_k = w^k, w = e^{-2 pi i / M}."""
    if M == 1:
        return np.ones(1, np.complex128)
    return np.exp(-2j * np.pi * np.arange(M) / M)


def _is_minus_one(M, k):
    return M >= 2 and 2 * k == M


def root_values(Lambda, P, Q, B, Ctilde, dt, M):
    """H(z_k) for k < M by the resolvent expression.

    z = -1: H = (dt/2) C~^* B.  Otherwise s = (2/dt)(1-z)/(1+z); an exactly
    zero s - lambda_j gives resonant-diagonal; R = diag(1/(s - lambda_j)),
    W = I_r + Q^* R P, an exactly singular W gives resonant-correction; else
    H = 2/(1+z) (C~^* R B - C~^* R P W^{-1} Q^* R B).
    Returns (values [M] complex128, status)."""
    lam = np.asarray(Lambda, np.complex128)
    N = len(lam)
    P = np.asarray(P, np.complex128).reshape(N, -1)
    Q = np.asarray(Q, np.complex128).reshape(N, -1)
    B = np.asarray(B, np.complex128)
    Ct = np.asarray(Ctilde, np.complex128)
    r = P.shape[1]
    z = roots_of_unity(M)
    out = np.empty(M, np.complex128)
    status = OK
    for k in range(M):
        if _is_minus_one(M, k):
            out[k] = (dt / 2.0) * np.vdot(Ct, B)
            continue
        s = (2.0 / dt) * (1.0 - z[k]) / (1.0 + z[k])
        den = s - lam
        if np.any(den == 0):
            out[k] = np.nan
            status = worst_status(status, RESONANT_DIAGONAL)
            continue
        R = np.diag(1.0 / den)
        W = np.eye(r, dtype=np.complex128) + Q.conj().T @ R @ P
        try:
            Winv_QRB = np.linalg.solve(W, Q.conj().T @ R @ B)
        except np.linalg.LinAlgError:
            out[k] = np.nan
            status = worst_status(status, RESONANT_CORRECTION)
            continue
        out[k] = 2.0 / (1.0 + z[k]) * (Ct.conj() @ R @ B - Ct.conj() @ R @ P @ Winv_QRB)
    return out, status


def root_values_cauchy(Lambda, P, Q, B, Ctilde, dt, M):
    """H(z_k) by the pages' (r+1)^2 Cauchy products in the mu-form.

    a = 2/dt, mu_j = (a - lambda_j)/(a + lambda_j) for lambda_j != -a.  For a
    pair (u, v): S_uv(z) = (dt/2) sum_{lambda_j = -a} conj(u_j) v_j
    - 2 sum_{lambda_j != -a} conj(u_j) v_j / (a + lambda_j) / (z - mu_j).
    W = I_r + (1+z)/2 S_QP, H = S_CB - (1+z)/2 S_CP W^{-1} S_QB.  Each scalar
    Cauchy product is summed directly (not by the product tree).  A collision
    mu_j = z_k gives resonant-diagonal; singular W gives resonant-correction.
    Returns (values, status)."""
    lam = np.asarray(Lambda, np.complex128)
    N = len(lam)
    P = np.asarray(P, np.complex128).reshape(N, -1)
    Q = np.asarray(Q, np.complex128).reshape(N, -1)
    B = np.asarray(B, np.complex128)
    Ct = np.asarray(Ctilde, np.complex128)
    r = P.shape[1]
    a = 2.0 / dt
    exc = lam == -a
    reg = ~exc
    mu = np.full(N, np.nan + 0j)
    mu[reg] = (a - lam[reg]) / (a + lam[reg])
    z = roots_of_unity(M)

    def S(uvec, vvec, zk):
        w = uvec.conj() * vvec
        const = (dt / 2.0) * np.sum(w[exc])
        return const - 2.0 * np.sum(w[reg] / (a + lam[reg]) / (zk - mu[reg]))

    out = np.empty(M, np.complex128)
    status = OK
    for k in range(M):
        if _is_minus_one(M, k):
            out[k] = (dt / 2.0) * np.vdot(Ct, B)
            continue
        if np.any(mu[reg] == z[k]):
            out[k] = np.nan
            status = worst_status(status, RESONANT_DIAGONAL)
            continue
        beta = (1.0 + z[k]) / 2.0
        S_CB = S(Ct, B, z[k])
        S_CP = np.array([S(Ct, P[:, b], z[k]) for b in range(r)])
        S_QB = np.array([S(Q[:, a_], B, z[k]) for a_ in range(r)])
        S_QP = np.array([[S(Q[:, a_], P[:, b], z[k]) for b in range(r)] for a_ in range(r)])
        W = np.eye(r, dtype=np.complex128) + beta * S_QP
        try:
            x = np.linalg.solve(W, S_QB)
        except np.linalg.LinAlgError:
            out[k] = np.nan
            status = worst_status(status, RESONANT_CORRECTION)
            continue
        out[k] = S_CB - beta * (S_CP @ x)
    return out, status


# ---------------------------------------------------------------------------
# Roots-of-unity Cauchy product by the balanced product tree
# ([RSS] block on the Cauchy matrix-vector product at the roots of unity, and
# the theorem on its operation count)
# ---------------------------------------------------------------------------
COLLISION = "collision"


def _tree(mu, a, lo, hi):
    """(D_I, P_I) for the index interval [lo, hi) as ascending coefficient
    arrays: a leaf j gives D = z - mu_j, P = a_j; an internal node splits its
    interval into halves whose sizes differ by at most one and combines
    D = D1 D2, P = P1 D2 + D1 P2 (np.convolve is the polynomial product)."""
    if hi - lo == 1:
        return np.array([-mu[lo], 1.0 + 0.0j]), np.array([a[lo]], np.complex128)
    mid = lo + (hi - lo) // 2
    D1, P1 = _tree(mu, a, lo, mid)
    D2, P2 = _tree(mu, a, mid, hi)
    D = np.convolve(D1, D2)
    P12, P21 = np.convolve(P1, D2), np.convolve(D1, P2)
    P = np.zeros(max(len(P12), len(P21)), np.complex128)
    P[:len(P12)] += P12
    P[:len(P21)] += P21
    return D, P


def _fold(c, M):
    """Coefficients modulo z^M - 1: degree r collects every degree = r mod M."""
    out = np.zeros(M, np.complex128)
    for d, v in enumerate(c):
        out[d % M] += v
    return out


def cauchy_product_tree(mu, a, M, omega=None):
    """y_k = sum_j a_j / (omega^k - mu_j), 0 <= k < M = 2^q, by the balanced
    product tree: the root's D and P folded modulo z^M - 1, both evaluated at
    omega_0^j (omega_0 = e^{-2 pi i / M}) by the radix-two DFT, and, for a
    primitive root omega other than omega_0, reindexed through the odd s
    with omega = omega_0^s (value at index s k mod M goes to output k).
    Repeated poles are allowed; n = 0 gives zeros.  A zero D(omega^k) gives
    the status collision (values NaN).  Returns (y [M] complex128, status).

    Readings: omega defaults to omega_0; the search for s compares the M
    powers of omega_0 with omega to within 1e-12 (exact equality is not
    available in floating point) and requires exactly one odd match."""
    if M < 1 or (M & (M - 1)) != 0:
        raise ValueError("M must be a power of two")
    mu = np.asarray(mu, np.complex128).ravel()
    a = np.asarray(a, np.complex128).ravel()
    n = len(mu)
    if n == 0:
        return np.zeros(M, np.complex128), OK
    D, P = _tree(mu, a, 0, n)
    Dv = radix2_dft(_fold(D, M))
    Pv = radix2_dft(_fold(P, M))
    if M > 1:
        w0 = _primitive_root(M, False)
        w = w0 if omega is None else complex(omega)
        powers = [w0 ** m for m in range(M)]
        odd = [m for m in range(1, M, 2) if abs(powers[m] - w) <= 1e-12]
        if len(odd) != 1:
            raise ValueError("omega is not a primitive M-th root of unity")
        sidx = odd[0]
        idx = [(sidx * k) % M for k in range(M)]
        Dv, Pv = Dv[idx], Pv[idx]
    if np.any(Dv == 0):
        return np.full(M, np.nan + 0j), COLLISION
    return Pv / Dv, OK


def root_values_product_tree(Lambda, P, Q, B, Ctilde, dt, M):
    """H(z_k) as root_values_cauchy, each scalar Cauchy product S_uv by the
    balanced product tree (poles mu_j, weights -2 conj(u_j) v_j / (a +
    lambda_j)) plus the constant of the states with lambda_j = -a.  A
    collision (some mu_j equal to a root) gives resonant-diagonal at every
    root (the tree reports it for the whole grid); the root -1 is handled
    directly.  Returns (values, status)."""
    lam = np.asarray(Lambda, np.complex128)
    N = len(lam)
    P = np.asarray(P, np.complex128).reshape(N, -1)
    Q = np.asarray(Q, np.complex128).reshape(N, -1)
    B = np.asarray(B, np.complex128)
    Ct = np.asarray(Ctilde, np.complex128)
    r = P.shape[1]
    a = 2.0 / dt
    exc = lam == -a
    reg = ~exc
    mu = (a - lam[reg]) / (a + lam[reg])
    z = roots_of_unity(M)

    def S(uvec, vvec):
        w = uvec.conj() * vvec
        y, st = cauchy_product_tree(mu, -2.0 * w[reg] / (a + lam[reg]), M)
        return y + (dt / 2.0) * np.sum(w[exc]), st

    fams = {}
    status = OK
    for key, (uu, vv) in {"CB": (Ct, B)}.items():
        fams[key], st = S(uu, vv)
        if st != OK:
            status = RESONANT_DIAGONAL
    S_CP = []
    S_QB = []
    S_QP = [[None] * r for _ in range(r)]
    for b in range(r):
        y, st = S(Ct, P[:, b])
        S_CP.append(y)
        status = RESONANT_DIAGONAL if st != OK else status
        y, st = S(Q[:, b], B)
        S_QB.append(y)
        status = RESONANT_DIAGONAL if st != OK else status
        for c in range(r):
            y, st = S(Q[:, b], P[:, c])
            S_QP[b][c] = y
            status = RESONANT_DIAGONAL if st != OK else status
    out = np.full(M, np.nan + 0j)
    if status != OK:
        for k in range(M):
            if _is_minus_one(M, k):
                out[k] = (dt / 2.0) * np.vdot(Ct, B)
        return out, status
    for k in range(M):
        if _is_minus_one(M, k):
            out[k] = (dt / 2.0) * np.vdot(Ct, B)
            continue
        beta = (1.0 + z[k]) / 2.0
        W = np.eye(r, dtype=np.complex128) + beta * np.array([[S_QP[i][j][k] for j in range(r)] for i in range(r)])
        try:
            x = np.linalg.solve(W, np.array([S_QB[i][k] for i in range(r)]))
        except np.linalg.LinAlgError:
            status = worst_status(status, RESONANT_CORRECTION)
            continue
        out[k] = fams["CB"][k] - beta * (np.array([S_CP[i][k] for i in range(r)]) @ x)
    return out, status


def filter_kernel(Lambda, P, Q, B, Ctilde, dt, L, use_radix2=None):
    """First L coefficients of the inverse radix-two transform of H(z_k).

    The inverse transform is the oracle's radix-two recursion for M <= 1024 and
    numpy's inverse FFT (a library step with the same sign and 1/M scale)
    above that.  Returns (K [L] complex128, status); a failing status gives an
    all-NaN kernel."""
    M = transform_length(L)
    Hk, status = root_values(Lambda, P, Q, B, Ctilde, dt, M)
    if status != OK:
        return np.full(L, np.nan + 0j), status
    if use_radix2 is None:
        use_radix2 = M <= 1024
    inv = radix2_dft(Hk, inverse=True) if use_radix2 else np.fft.ifft(Hk)
    return inv[:L], OK


# ---------------------------------------------------------------------------
# DPLR recurrent solver  ([RSS] Algorithm-1 block: Woodbury / bordered system)
# ---------------------------------------------------------------------------
def dplr_solve(Lambda, P, Q, dt, b):
    """Solve G x = b, G = I - (dt/2)(Lambda - P Q^*), with the pages' structured
    branches: Woodbury when no d_j = 1 - alpha lambda_j is zero, the bordered
    system when 0 < |Z| <= r.  Returns (x, status)."""
    lam = np.asarray(Lambda, np.complex128)
    N = len(lam)
    P = np.asarray(P, np.complex128).reshape(N, -1)
    Q = np.asarray(Q, np.complex128).reshape(N, -1)
    b = np.asarray(b, np.complex128)
    r = P.shape[1]
    alpha = dt / 2.0
    d = 1.0 - alpha * lam
    Z = np.flatnonzero(d == 0)
    J = np.flatnonzero(d != 0)
    s = len(Z)
    if s == 0:
        core = np.eye(r, dtype=np.complex128) + alpha * Q.conj().T @ (P / d[:, None])
        try:
            zz = np.linalg.solve(core, Q.conj().T @ (b / d))
        except np.linalg.LinAlgError:
            return None, SINGULAR_BILINEAR
        return (b - alpha * P @ zz) / d, OK
    if s > r:
        return None, SINGULAR_BILINEAR
    dJ = d[J]
    top_left = np.eye(r, dtype=np.complex128) + alpha * Q[J].conj().T @ (P[J] / dJ[:, None])
    Mb = np.zeros((r + s, r + s), np.complex128)
    Mb[:r, :r] = top_left
    Mb[:r, r:] = -Q[Z].conj().T
    Mb[r:, :r] = alpha * P[Z]
    rhs = np.concatenate([Q[J].conj().T @ (b[J] / dJ), b[Z]])
    try:
        sol = np.linalg.solve(Mb, rhs)
    except np.linalg.LinAlgError:
        return None, SINGULAR_BILINEAR
    zz, xZ = sol[:r], sol[r:]
    x = np.empty(N, np.complex128)
    x[J] = (b[J] - alpha * P[J] @ zz) / dJ
    x[Z] = xZ
    return x, OK


# ---------------------------------------------------------------------------
# Whole-channel reference
# ---------------------------------------------------------------------------
def discretize_channel(Lambda, P, Q, B, C, dt, L):
    """Dense discretisation of one channel and its truncated-output vector.

    Returns dict(Abar, Bbar, Ctilde, M, status)."""
    M = transform_length(L)
    A = dplr_matrix(Lambda, P, Q)
    Abar, Bbar, status = bilinear(A, B, dt)
    if status != OK:
        return dict(Abar=None, Bbar=None, Ctilde=None, M=M, status=status)
    return dict(Abar=Abar, Bbar=Bbar, Ctilde=truncated_output(Abar, C, M), M=M, status=status)


def channel_reference(Lambda, P, Q, B, C, dt, D, u, L, kernel_taps=None):
    """Everything the path produces for one channel, from the definitions.

    K: first L taps of C^* Abar^j Bbar (matrix iteration); y: real part of the
    time-stepped recurrence with the skip term (u has shape [Bsz, L]).
    Statuses: singular-bilinear from the bilinear step, resonances from the
    filter-mode root values (evaluated with C~).  A failing channel has NaN
    K and y."""
    disc = discretize_channel(Lambda, P, Q, B, C, dt, L)
    Bsz = np.asarray(u).shape[0] if u is not None else 0
    if disc["status"] != OK:
        nanK = np.full(L, np.nan + 0j)
        return dict(disc, K=nanK, y=np.full((Bsz, L), np.nan))
    K = kernel_by_iteration(disc["Abar"], disc["Bbar"], C, L if kernel_taps is None else kernel_taps)
    _, st = root_values(Lambda, P, Q, B, disc["Ctilde"], dt, disc["M"])
    y = None
    if u is not None:
        y = recurrence(disc["Abar"], disc["Bbar"], C, D, u).real
    if st != OK:
        K = np.full(len(K), np.nan + 0j)
        y = None if y is None else np.full(y.shape, np.nan)
    return dict(disc, K=K, y=y, status=st)
