"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
import numpy as np

# tolerance of the filter path: max error <= TOL * max|reference| per channel
# (kernel, root values) or per batch row (outputs)
TOL = 2e-4


def rel_err_rows(got, ref):
    """max_t |got - ref| / max_t |ref| for each row of [..., L] arrays."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-30)


def assert_rows_close(got, ref, tol=TOL, what=""):
    e = rel_err_rows(got, ref)
    assert np.all(np.isfinite(e)), f"{what}: non-finite error"
    worst = float(e.max())
    assert worst <= tol, f"{what}: worst row error {worst:.3e} > {tol:.1e}"
    return worst


def sample_channels(H, k, seed=0):
    if H <= k:
        return np.arange(H)
    rng = np.random.default_rng(1234 + seed)
    chans = set(rng.choice(H, size=k - 2, replace=False).tolist()) | {0, H - 1}
    return np.array(sorted(chans))
