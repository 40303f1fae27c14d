"""Pins for the HiPPO part of the CPU oracle: each check ties it to something
other than itself -- a case derived by hand, the LagT cotangent closed form,
an independent general eigensolver (scipy), and invariants that a mistake in
any step breaks (normality of the normal part, reconstruction of the
transformed generator, unitarity, and the impulse kernel, which a state change
must leave unchanged).  Planted mistakes at the end check that the pins catch
plausible errors in each function."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O
import oracle.hippo_oracle as HO

KINDS = HO.KINDS


def _vectors(seed, n, N):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(n, N)) + 1j * rng.normal(size=(n, N))


def test_legs_two_states_by_hand():
    # N = 2: G = [[-1, 0], [-sqrt 3, -2]], u = (sqrt(1/2), sqrt(3/2)).
    # G + u u^T = [[-1/2, sqrt3/2], [-sqrt3/2, -1/2]] = -I/2 + K with K skew;
    # K (1, -i)/sqrt2 = -i sqrt3/2 (1, -i)/sqrt2, and (1, i)/sqrt2 for +i sqrt3/2.
    # (1, -i)^* u / sqrt2 = (1 + i sqrt3)/2 = e^{i pi/3} and (1, i)^* u / sqrt2 =
    # e^{-i pi/3}: after the phase rule both vectors give P = 1.
    G = HO.hippo_generator(HO.LEGS, 2)
    assert np.array_equal(G, np.array([[-1.0, 0.0], [-np.sqrt(3.0), -2.0]]))
    d = HO.hippo_dplr(HO.LEGS, 2)
    r3 = np.sqrt(3.0) / 2
    assert np.allclose(d["Lambda"], [-0.5 - 1j * r3, -0.5 + 1j * r3], atol=1e-15)
    assert np.allclose(d["P"][:, 0], [1.0, 1.0], atol=1e-15)
    w = np.exp(1j * np.pi / 3) / np.sqrt(2)
    assert np.allclose(d["V"][:, 0], [w, -1j * w], atol=1e-15)
    assert np.allclose(d["V"][:, 1], [np.conj(w), 1j * np.conj(w)], atol=1e-15)


def test_lagt_two_states_by_hand():
    # N = 2: G = [[-1, 0], [-1, -1]], u = (1, 1)/sqrt2: G + u u^T = -I/2 + K,
    # K = (1/2) [[0, 1], [-1, 0]], eigenvalue -i/2 on (1, -i)/sqrt2 and +i/2 on
    # (1, i)/sqrt2.  (1, -i)^* u / sqrt2 = (1 + i)/2 = e^{i pi/4}/sqrt2 and
    # (1, i)^* u / sqrt2 = e^{-i pi/4}/sqrt2: both give P = 1/sqrt2.
    assert np.array_equal(HO.hippo_generator(HO.LAGT, 2), np.array([[-1.0, 0.0], [-1.0, -1.0]]))
    d = HO.hippo_dplr(HO.LAGT, 2)
    assert np.allclose(d["Lambda"], [-0.5 - 0.5j, -0.5 + 0.5j], atol=1e-15)
    assert np.allclose(d["P"][:, 0], [2 ** -0.5, 2 ** -0.5], atol=1e-15)
    w = np.exp(1j * np.pi / 4) / np.sqrt(2)
    assert np.allclose(d["V"], np.array([[w, np.conj(w)], [-1j * w, 1j * np.conj(w)]]), atol=1e-15)


@pytest.mark.parametrize("N", [1, 2, 5, 8, 33, 64])
def test_lagt_cotangent_closed_form(N):
    # The skew part of LagT has entries -1/2 below and +1/2 above the diagonal;
    # i times it has eigenvalues (1/2) cot((2m+1) pi / (2N)), m = 0 .. N-1.
    d = HO.hippo_dplr(HO.LAGT, N)
    mu = 0.5 / np.tan((2 * np.arange(N) + 1) * np.pi / (2 * N))
    expect = np.sort(-0.5 - 1j * mu, )                    # any order, then ascending imag
    expect = expect[np.argsort(expect.imag)]
    assert np.allclose(d["Lambda"], expect, atol=1e-12 * max(1, np.abs(mu).max()))
    assert np.all(d["Lambda"].real == -0.5)


def test_legt_two_states_by_hand():
    # N = 2: G = (1/theta) [[-1, -1], [3, -3]], S0 = diag(1, -sqrt 3), so
    # S0^{-1} G S0 = (1/theta) [[-1, sqrt3], [-sqrt3, -3]]; U U^T = diag(1, 3)/theta
    # leaves the skew matrix a [[0, 1], [-1, 0]], a = sqrt3/theta, with eigenvalue
    # -i a on (1, -i)/sqrt2 and +i a on (1, i)/sqrt2.  Both first entries of
    # V^* U are 1/sqrt(2 theta) > 0 (no phase change); the second entries are
    # +-i sqrt(3/(2 theta)).  The sign of S0 decides which.
    th = 0.6
    G = HO.hippo_generator(HO.LEGT, 2, th)
    assert np.allclose(G, np.array([[-1.0, -1.0], [3.0, -3.0]]) / th, atol=1e-15)
    assert np.allclose(HO.hippo_similarity(HO.LEGT, 2), [1.0, -np.sqrt(3.0)], atol=1e-15)
    b, c = np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]])
    d = HO.hippo_dplr(HO.LEGT, 2, th, b, c)
    a = np.sqrt(3.0) / th
    assert np.allclose(d["Lambda"], [-1j * a, 1j * a], atol=1e-14)
    h = 1 / np.sqrt(2)
    assert np.allclose(d["V"], np.array([[h, h], [-1j * h, 1j * h]]), atol=1e-15)
    p0, p1 = 1 / np.sqrt(2 * th), np.sqrt(3 / (2 * th))
    assert np.allclose(d["P"], np.array([[p0, 1j * p1], [p0, -1j * p1]]), atol=1e-14)
    # Bt = V^* S0^{-1} (1, 0) = (h, h); Ct = V^* S0 (0, 1) = -sqrt3 (conj(-i h), conj(i h))
    assert np.allclose(d["Bt"], [[h, h]], atol=1e-15)
    assert np.allclose(d["Ct"], [[-np.sqrt(3.0) * 1j * h, np.sqrt(3.0) * 1j * h]], atol=1e-14)


def test_legt_one_state():
    # N = 1: G = -1/theta, S = 1, U = (1/sqrt theta, 0): the normal part is 0,
    # V = 1 and P = (1/sqrt theta, 0); B and C are unchanged.
    th = 0.37
    b, c = np.array([[0.3 - 2j]]), np.array([[1.5 + 0.25j]])
    d = HO.hippo_dplr(HO.LEGT, 1, th, b, c)
    assert np.array_equal(HO.hippo_generator(HO.LEGT, 1, th), np.array([[-1 / th]]))
    assert d["Lambda"][0] == 0
    assert np.allclose(d["P"], [[1 / np.sqrt(th), 0.0]], atol=1e-15)
    assert np.allclose(d["Bt"], b) and np.allclose(d["Ct"], c)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N", [3, 16, 64])
def test_normal_part_is_normal_and_low_rank(kind, N):
    th = 1.7
    H = HO.normal_part(kind, N, th)
    assert np.abs(H.T @ H - H @ H.T).max() <= 1e-12 * max(1.0, np.abs(H).max() ** 2)
    At = HO.transformed_generator(kind, N, th)
    sv = np.linalg.svd(H - At, compute_uv=False)
    r = HO.hippo_rank(kind)
    assert np.all(sv[r:] <= 1e-10 * sv[0])
    # the similarity maps G to the transformed matrix
    s = HO.hippo_similarity(kind, N)
    assert np.allclose(np.diag(s) @ At, HO.hippo_generator(kind, N, th) @ np.diag(s))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N", [1, 4, 17, 64])
def test_dplr_reconstructs_and_is_unitary(kind, N):
    th = 0.8
    d = HO.hippo_dplr(kind, N, th)
    V, Lam, P = d["V"], d["Lambda"], d["P"]
    At = HO.transformed_generator(kind, N, th)
    scale = max(1.0, np.abs(At).max())
    assert np.abs(V.conj().T @ V - np.eye(N)).max() <= 1e-12 * N
    Adplr = np.diag(Lam) - P @ P.conj().T
    assert np.abs(V @ Adplr @ V.conj().T - At).max() <= 1e-12 * scale * N
    assert np.all(np.diff(Lam.imag) >= 0)
    assert np.all(P[:, 0].imag == 0) and np.all(P[:, 0].real >= 0)


@pytest.mark.parametrize("kind", KINDS)
def test_eigenvalues_match_general_eigensolver(kind):
    N, th = 40, 2.5
    ev = scipy.linalg.eigvals(HO.normal_part(kind, N, th))
    ev = ev[np.argsort(ev.imag)]
    lam = HO.hippo_dplr(kind, N, th)["Lambda"]
    assert np.abs(ev - lam).max() <= 1e-10 * max(1.0, np.abs(lam).max())


@pytest.mark.parametrize("kind", KINDS)
def test_state_change_keeps_the_kernel(kind):
    # the impulse kernel C^* Abar^j Bbar is invariant under x = S V x~
    N, th, dt, L = 12, 1.3, 0.05, 40
    B, C = _vectors(1, 1, N), _vectors(2, 1, N)
    d = HO.hippo_dplr(kind, N, th, B, C)
    G = HO.hippo_generator(kind, N, th)
    Ab, Bb, st = O.bilinear(G.astype(complex), B[0], dt)
    assert st == O.OK
    K0 = O.kernel_by_iteration(Ab, Bb, C[0], L)
    A2 = O.dplr_matrix(d["Lambda"], d["P"], d["P"])
    Ab2, Bb2, st2 = O.bilinear(A2, d["Bt"][0], dt)
    assert st2 == O.OK
    K1 = O.kernel_by_iteration(Ab2, Bb2, d["Ct"][0], L)
    assert np.abs(K1 - K0).max() <= 1e-10 * np.abs(K0).max()


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin above
# --------------------------------------------------------------------------
def _pins_pass():
    checks = [
        test_legs_two_states_by_hand,
        lambda: test_lagt_cotangent_closed_form(8),
        test_lagt_two_states_by_hand,
        test_legt_two_states_by_hand,
        test_legt_one_state,
        *[lambda k=k: test_normal_part_is_normal_and_low_rank(k, 16) for k in KINDS],
        *[lambda k=k: test_dplr_reconstructs_and_is_unitary(k, 17) for k in KINDS],
        *[lambda k=k: test_eigenvalues_match_general_eigensolver(k) for k in KINDS],
        *[lambda k=k: test_state_change_keeps_the_kernel(k) for k in KINDS],
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


_orig = {}


def _mut_legs_diagonal(kind, N, theta=1.0):
    G = _orig["hippo_generator"](kind, N, theta)
    if kind == HO.LEGS:
        G = G + np.eye(N)                      # -n instead of -(n + 1)
    return G


def _mut_legt_no_sign(kind, N):
    s = _orig["hippo_similarity"](kind, N)
    return np.abs(s)                            # similarity without (-1)^n


def _mut_lagt_upper(kind, N, theta=1.0):
    G = _orig["hippo_generator"](kind, N, theta)
    return G.T if kind == HO.LAGT else G        # -1 above instead of below the diagonal


def _mut_legt_rank_one(kind, N, theta=1.0):
    c, U = _orig["hippo_low_rank"](kind, N, theta)
    if kind == HO.LEGT:
        U = U.copy(); U[:, 1] = 0               # drop the odd-index column
    return c, U


def _mut_dplr_no_conj(kind, N, theta=1.0, B=None, C=None):
    d = _orig["hippo_dplr"](kind, N, theta, B, C)
    d["P"] = d["V"].T @ d["U"]                  # V^T U instead of V^* U
    return d


def _mut_dplr_lambda_sign(kind, N, theta=1.0, B=None, C=None):
    d = _orig["hippo_dplr"](kind, N, theta, B, C)
    d["Lambda"] = np.conj(d["Lambda"])          # c + i mu instead of c - i mu
    return d


def _mut_dplr_b_times_s(kind, N, theta=1.0, B=None, C=None):
    d = _orig["hippo_dplr"](kind, N, theta, B, C)
    if B is not None:
        s = HO.hippo_similarity(kind, N)
        d["Bt"] = np.array([d["V"].conj().T @ (b * s) for b in np.atleast_2d(B)])   # S B instead of S^{-1} B
    return d


def _mut_dplr_c_no_conj(kind, N, theta=1.0, B=None, C=None):
    d = _orig["hippo_dplr"](kind, N, theta, B, C)
    if C is not None:
        s = HO.hippo_similarity(kind, N)
        d["Ct"] = np.array([d["V"].T @ (s * c) for c in np.atleast_2d(C)])          # V^T instead of V^*
    return d


@pytest.mark.parametrize("name,mutant", [
    ("hippo_generator", _mut_legs_diagonal),
    ("hippo_similarity", _mut_legt_no_sign),
    ("hippo_generator", _mut_lagt_upper),
    ("hippo_low_rank", _mut_legt_rank_one),
    ("hippo_dplr", _mut_dplr_no_conj),
    ("hippo_dplr", _mut_dplr_lambda_sign),
    ("hippo_dplr", _mut_dplr_b_times_s),
    ("hippo_dplr", _mut_dplr_c_no_conj),
])
def test_planted_mistakes_are_caught(monkeypatch, name, mutant):
    assert _pins_pass()
    _orig[name] = getattr(HO, name)
    monkeypatch.setattr(HO, name, mutant)
    assert not _pins_pass(), f"no pin caught the planted mistake in {name}"


@pytest.mark.parametrize("kind", KINDS)
def test_eigenvalues_stay_separated_up_to_the_size_cap(kind):
    # The device solver has no status for close eigenvalues: inverse iteration
    # keeps the vectors orthogonal to about eps / (relative gap), and for these
    # generators the relative gap stays above 5e-7 up to N = 1024 (LegS is the
    # tightest, about 1.07e-6 at 1024), so the vectors are orthogonal to ~1e-9.
    for N in (256, 512, 1000, 1024):
        K = HO.normal_part(kind, N, 1.0) - HO.hippo_low_rank(kind, N, 1.0)[0] * np.eye(N)
        mu = np.sort(np.linalg.eigvalsh(1j * K))
        assert np.diff(mu).min() > 5e-7 * np.abs(mu).max(), (kind, N)
