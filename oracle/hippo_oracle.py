"""Plain float64 / complex128 CPU oracle for the HiPPO generators and their
diagonal-plus-low-rank (DPLR) form.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check of the entry
script and the benchmark's CPU-baseline leg may import or run this module.  It
shares no code with the HIP library and imports nothing but numpy.  It is
written for clarity: explicit loops for the matrices, a library Hermitian
eigensolver for the one spectral step.

Source pages (cited by title and block):
  [RSS]  "Recurrent, LSTM, and structured state-space models"
         - block on the HiPPO generators (S4 Theorem 1 and App. C.1; HiPPO
           sec. 2.3 and App. D.1-D.3): the LegS, LegT and LagT matrices, the
           diagonal similarity used for LegT, the statement that each
           transformed matrix is a normal matrix minus a term of rank <= 1
           (LegS, LagT) or <= 2 (LegT), and how B and C change under a state
           change x = S x~ (to S^{-1} B and S^* C);
         - block "DPLR structured state-space parameterization": the DPLR form
           A = Lambda - P Q^*, the NPLR form V Lambda V^* - P Q^* with V
           unitary, and the unitary state change x~ = V^* x, which maps B and C
           to V^* B and V^* C.

Readings where the pages are silent (each also listed in the design notes):
  * The low-rank term is not printed.  It is taken as the one that leaves a
    multiple c of the identity plus a skew-symmetric matrix, which is normal:
      LegS  c = -1/2, one column u_n = sqrt(n + 1/2);
      LagT  c = -1/2, one column u_n = sqrt(1/2);
      LegT  c = 0, two columns: sqrt((2n+1)/theta) on even n (zero on odd n),
            and sqrt((2n+1)/theta) on odd n (zero on even n).
    With these, transformed matrix = (c I + K) - U U^T with K real skew, so
    P = Q = V^* U in the DPLR coordinates.
  * Eigenvalues are returned by ascending imaginary part.
  * Each eigenvector (column of V) is scaled by a unit complex number so that
    the first column of P = V^* U is real and non-negative.

Parity pins live in tests/test_hippo_oracle_pins.py: a hand-derived N = 2 LegS
case, the LagT cotangent closed form, an N = 1 LegT case, normality, the
reconstruction of the transformed matrix, an independent general eigensolver
and the invariance of the impulse kernel under the state change.
"""
from __future__ import annotations

import numpy as np

LEGS = "legs"
LEGT = "legt"
LAGT = "lagt"
KINDS = (LEGS, LEGT, LAGT)


def hippo_rank(kind):
    """Rank of the low-rank term: 1 for LegS and LagT, 2 for LegT."""
    return 2 if kind == LEGT else 1


def hippo_generator(kind, N, theta=1.0):
    """The real N x N generator, entry by entry as the HiPPO block defines it
    (rows and columns indexed 0 .. N-1)."""
    G = np.zeros((N, N))
    for n in range(N):
        for k in range(N):
            if kind == LEGS:
                if n > k:
                    G[n, k] = -np.sqrt((2 * n + 1) * (2 * k + 1))
                elif n == k:
                    G[n, k] = -(n + 1)
            elif kind == LEGT:
                if n >= k:
                    G[n, k] = -(2 * n + 1) * (-1.0) ** (n - k) / theta
                else:
                    G[n, k] = -(2 * n + 1) / theta
            elif kind == LAGT:
                if n >= k:
                    G[n, k] = -1.0
            else:
                raise ValueError(kind)
    return G


def hippo_similarity(kind, N):
    """Diagonal of the similarity S (x = S x~): the identity for LegS and
    LagT; diag(sqrt(2n+1)) diag((-1)^n) for LegT."""
    if kind == LEGT:
        return np.array([np.sqrt(2 * n + 1) * (-1.0) ** n for n in range(N)])
    return np.ones(N)


def transformed_generator(kind, N, theta=1.0):
    """S^{-1} G S."""
    G = hippo_generator(kind, N, theta)
    s = hippo_similarity(kind, N)
    return np.diag(1.0 / s) @ G @ np.diag(s)


def hippo_low_rank(kind, N, theta=1.0):
    """(c, U): the identity multiple of the normal part and the low-rank
    factor of the reading above; U is N x rank."""
    if kind == LEGS:
        return -0.5, np.array([[np.sqrt(n + 0.5)] for n in range(N)])
    if kind == LAGT:
        return -0.5, np.full((N, 1), np.sqrt(0.5))
    if kind == LEGT:
        U = np.zeros((N, 2))
        for n in range(N):
            U[n, n % 2] = np.sqrt((2 * n + 1) / theta)
        return 0.0, U
    raise ValueError(kind)


def normal_part(kind, N, theta=1.0):
    """H = S^{-1} G S + U U^T, the normal matrix of the NPLR split."""
    _, U = hippo_low_rank(kind, N, theta)
    return transformed_generator(kind, N, theta) + U @ U.T


def hippo_dplr(kind, N, theta=1.0, B=None, C=None):
    """DPLR form of a HiPPO generator.

    Returns a dict with
      Lambda [N]      eigenvalues of the normal part, ascending imaginary part;
      P [N, rank]     V^* U (equal to Q);
      V [N, N]        unitary eigenvectors (columns), phase-fixed as above;
      Bt [nb, N]      V^* S^{-1} B for each row of B (if given);
      Ct [nc, N]      V^* S^* C for each row of C (if given).
    The model (G, B, C) and (Lambda - P P^*, Bt, Ct) are related by the state
    change x = S V x~."""
    c, U = hippo_low_rank(kind, N, theta)
    H = normal_part(kind, N, theta)
    K = H - c * np.eye(N)                       # real skew-symmetric
    # i K is Hermitian: i K w = mu w  <=>  K w = -i mu w, eigenvalue c - i mu of H
    mu, W = np.linalg.eigh(1j * K)
    order = np.argsort(-mu, kind="stable")      # ascending imaginary part -mu
    mu, W = mu[order], W[:, order]
    Lambda = c - 1j * mu
    P = W.conj().T @ U
    for j in range(N):
        W[:, j] = W[:, j] * np.exp(1j * np.angle(P[j, 0]))
    P = W.conj().T @ U
    P[:, 0] = np.abs(P[:, 0])                   # real and non-negative by the phase rule
    out = dict(Lambda=Lambda, P=P, V=W, c=c, U=U)
    s = hippo_similarity(kind, N)
    if B is not None:
        B = np.atleast_2d(np.asarray(B, complex))
        out["Bt"] = np.array([W.conj().T @ (b / s) for b in B])
    if C is not None:
        C = np.atleast_2d(np.asarray(C, complex))
        out["Ct"] = np.array([W.conj().T @ (np.conj(s) * cv) for cv in C])
    return out
