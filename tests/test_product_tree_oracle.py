"""Pins of the oracle's balanced product-tree Cauchy product ("Recurrent, LSTM,
and structured state-space models", block on the Cauchy matrix-vector product
at the roots of unity, and the theorem on its operation count), and of the
root values computed through it, against what fixes them independently:

* the definition y_k = sum_j a_j / (omega^k - mu_j), summed directly on tiny
  inputs, including more poles than roots (so the fold modulo z^M - 1 acts)
  and a primitive root other than e^{-2 pi i/M} (so the odd-s reindexing
  acts);
* repeated poles, no poles, and an exact collision;
* the resolvent expression for the root values (root_values);
* the loss of accuracy in float64 at the S4 workload's poles, which is why
  the GPU path sums the Cauchy products directly.

Inputs are well conditioned (poles well inside the unit circle) except in the
last test: the algorithm is exact in exact arithmetic, and its float64 error
grows with the clustering of the poles near the unit circle."""
import numpy as np
import pytest

import oracle as O


def _direct(mu, a, omega, M):
    return np.array([np.sum(a / (omega ** k - mu)) for k in range(M)])


def _case(seed, n, radius=0.6):
    rng = np.random.default_rng(seed)
    ang = rng.uniform(0, 2 * np.pi, n)
    rad = rng.uniform(0.05, radius, n)
    mu = rad * np.exp(1j * ang)
    a = rng.normal(size=n) + 1j * rng.normal(size=n)
    return mu, a


@pytest.mark.parametrize("n,M", [(1, 1), (1, 2), (2, 4), (3, 8), (5, 4), (8, 4), (9, 16), (17, 8), (16, 16)])
def test_tree_equals_direct_sum(n, M):
    mu, a = _case(10 * n + M, n)
    y, st = O.cauchy_product_tree(mu, a, M)
    assert st == O.OK
    w0 = np.exp(-2j * np.pi / M) if M > 1 else 1.0
    ref = _direct(mu, a, w0, M)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("M,s", [(4, 3), (8, 3), (8, 5), (16, 7), (16, 15)])
def test_tree_other_primitive_root(M, s):
    """omega = omega_0^s (s odd): the output is in omega's power order."""
    mu, a = _case(M + s, 6)
    w = np.exp(-2j * np.pi * s / M)
    y, st = O.cauchy_product_tree(mu, a, M, omega=w)
    assert st == O.OK
    ref = _direct(mu, a, w, M)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    # and it differs from the omega_0 order (the reindexing is not a no-op)
    y0, _ = O.cauchy_product_tree(mu, a, M)
    assert np.abs(y - y0).max() > 1e-3 * np.abs(ref).max()


def test_tree_rejects_non_primitive_root():
    with pytest.raises(ValueError):
        O.cauchy_product_tree([0.1], [1.0], 8, omega=np.exp(-2j * np.pi * 2 / 8))  # order 4, not 8


def test_tree_repeated_poles_and_empty():
    mu, a = _case(3, 3)
    mu = np.array([mu[0], mu[0], mu[1], mu[0]])
    a = np.array([1.0, 2.0 - 1j, 0.5j, -3.0])
    y, st = O.cauchy_product_tree(mu, a, 8)
    assert st == O.OK
    ref = _direct(mu, a, np.exp(-2j * np.pi / 8), 8)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    y, st = O.cauchy_product_tree([], [], 8)
    assert st == O.OK and np.array_equal(y, np.zeros(8))


def test_tree_collision():
    """A pole on the grid (mu = 1 = omega^0, exactly representable with the
    other pole 0.5, so D(1) evaluates to exactly 0) gives collision."""
    y, st = O.cauchy_product_tree([1.0, 0.5], [1.0, 2.0], 4)
    assert st == O.COLLISION and np.isnan(y).all()
    y, st = O.cauchy_product_tree([-1.0], [1.0], 2)   # omega^1 = -1 for M = 2
    assert st == O.COLLISION


def _well_conditioned_channel(seed, N, r):
    """dt = 1 (a = 2) and eigenvalues of moderate size: the poles
    mu_j = (2 - lambda_j)/(2 + lambda_j) stay well inside the unit circle."""
    rng = np.random.default_rng(seed)
    lam = -(1.0 + rng.uniform(0, 2, N)) + 1j * rng.uniform(-2, 2, N)
    P = (rng.normal(size=(N, r)) + 1j * rng.normal(size=(N, r))) / np.sqrt(N)
    Q = (rng.normal(size=(N, r)) + 1j * rng.normal(size=(N, r))) / np.sqrt(N)
    B = rng.normal(size=N) + 1j * rng.normal(size=N)
    C = rng.normal(size=N) + 1j * rng.normal(size=N)
    return lam, P, Q, B, C, 1.0


@pytest.mark.parametrize("N,r,M", [(1, 1, 1), (3, 1, 8), (6, 2, 16), (12, 2, 4), (5, 3, 32)])
def test_tree_root_values_equal_resolvent(N, r, M):
    lam, P, Q, B, C, dt = _well_conditioned_channel(N * 7 + r + M, N, r)
    ref, st = O.root_values(lam, P, Q, B, C, dt, M)
    got, st2 = O.root_values_product_tree(lam, P, Q, B, C, dt, M)
    assert st == st2 == O.OK
    assert np.abs(got - ref).max() <= 1e-10 * np.abs(ref).max()


def test_tree_root_values_state_at_minus_a():
    """A state with lambda_j = -a (no pole) enters through the constant term."""
    lam, P, Q, B, C, dt = _well_conditioned_channel(5, 4, 1)
    lam[2] = -2.0 / dt
    ref, st = O.root_values(lam, P, Q, B, C, dt, 8)
    got, st2 = O.root_values_product_tree(lam, P, Q, B, C, dt, 8)
    assert st == st2 == O.OK
    assert np.abs(got - ref).max() <= 1e-10 * np.abs(ref).max()


def test_tree_root_values_collision_is_resonant_diagonal():
    """mu_j = 1 = z_0 exactly: lambda_j = 0 with a = 2 gives mu_j = 1."""
    lam, P, Q, B, C, dt = _well_conditioned_channel(6, 2, 1)
    lam[:] = [0.0, -0.5]
    got, st = O.root_values_product_tree(lam, P, Q, B, C, dt, 4)
    assert st == O.RESONANT_DIAGONAL


def test_tree_loses_float64_accuracy_at_s4_poles():
    """The S4 workloads' poles (lambda_n = -1/2 + i pi n, dt = 0.01, so
    a = 200) crowd near z = 1: the root polynomial's coefficients grow while
    its values on the unit circle shrink, and by N = 32 the float64 result
    has no correct digit, while the direct sum of the same terms is exact to
    rounding.  (This is the measured reason the GPU path sums directly.)"""
    N, dt, M = 32, 0.01, 256
    lam = -0.5 + 1j * np.pi * np.arange(N)
    a2 = 2.0 / dt
    mu = (a2 - lam) / (a2 + lam)
    w = np.random.default_rng(1).normal(size=N) + 1j * np.random.default_rng(2).normal(size=N)
    y, st = O.cauchy_product_tree(mu, w, M)
    ref = _direct(mu, w, np.exp(-2j * np.pi / M), M)
    err = np.abs(y - ref).max() / np.abs(ref).max() if st == O.OK else np.inf
    assert err > 0.1
    # the same tree on a well-spread set of 32 poles stays accurate
    mu2, _ = _case(9, N)
    y2, st2 = O.cauchy_product_tree(mu2, w, M)
    ref2 = _direct(mu2, w, np.exp(-2j * np.pi / M), M)
    assert st2 == O.OK and np.abs(y2 - ref2).max() <= 1e-9 * np.abs(ref2).max()


# --------------------------------------------------------------------------
# Planted mistakes (in the oracle, on the CPU): each must fail some pin above.
def _tree_pins_pass():
    try:
        test_tree_equals_direct_sum(17, 8)
        test_tree_equals_direct_sum(3, 8)
        test_tree_other_primitive_root(8, 3)
        test_tree_root_values_equal_resolvent(6, 2, 16)
        test_tree_collision()
    except (AssertionError, ValueError):
        return False
    return True


def _mut_tree_p(mu, a, lo, hi):            # P = P1 D1 + D2 P2 instead of P1 D2 + D1 P2
    if hi - lo == 1:
        return np.array([-mu[lo], 1.0 + 0.0j]), np.array([a[lo]], np.complex128)
    mid = lo + (hi - lo) // 2
    D1, P1 = _mut_tree_p(mu, a, lo, mid)
    D2, P2 = _mut_tree_p(mu, a, mid, hi)
    X, Y = np.convolve(P1, D1), np.convolve(D2, P2)
    P = np.zeros(max(len(X), len(Y)), np.complex128)
    P[:len(X)] += X
    P[:len(Y)] += Y
    return np.convolve(D1, D2), P


def _mut_tree_leaf(mu, a, lo, hi):         # leaf z + mu_j instead of z - mu_j
    if hi - lo == 1:
        return np.array([mu[lo], 1.0 + 0.0j]), np.array([a[lo]], np.complex128)
    mid = lo + (hi - lo) // 2
    D1, P1 = _mut_tree_leaf(mu, a, lo, mid)
    D2, P2 = _mut_tree_leaf(mu, a, mid, hi)
    X, Y = np.convolve(P1, D2), np.convolve(D1, P2)
    P = np.zeros(max(len(X), len(Y)), np.complex128)
    P[:len(X)] += X
    P[:len(Y)] += Y
    return np.convolve(D1, D2), P


def _mut_fold(c, M):                       # wrapped degrees overwrite instead of adding
    out = np.zeros(M, np.complex128)
    for d, v in enumerate(c):
        out[d % M] = v
    return out


_orig_cpt = O.ssm_oracle.cauchy_product_tree


def _mut_no_reindex(mu, a, M, omega=None):  # the supplied root's order ignored
    return _orig_cpt(mu, a, M)


@pytest.mark.parametrize("name,mutant", [("_tree", _mut_tree_p), ("_tree", _mut_tree_leaf), ("_fold", _mut_fold),
                                         ("cauchy_product_tree", _mut_no_reindex)])
def test_tree_planted_mistakes_are_caught(monkeypatch, name, mutant):
    import oracle.ssm_oracle as mod
    assert _tree_pins_pass()
    monkeypatch.setattr(mod, name, mutant)
    if hasattr(O, name):
        monkeypatch.setattr(O, name, mutant)
    assert not _tree_pins_pass(), f"no pin caught the planted mistake in {name}"
