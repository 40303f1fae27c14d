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


def sample_channels(H, k, seed=0, forced=()):
    """k channels: the first, the last and a seeded random draw, plus every
    channel listed in `forced` (e.g. those with the smallest and largest step)."""
    if H <= k:
        return np.arange(H)
    rng = np.random.default_rng(1234 + seed)
    chans = set(rng.choice(H, size=k - 2, replace=False).tolist()) | {0, H - 1}
    chans |= {int(h) for h in forced}
    return np.array(sorted(chans))


def extreme_step_channels(dt):
    """The channels with the smallest and the largest step size (the smallest
    step puts the roots' Cauchy denominators closest together in float32)."""
    dt = np.asarray(dt)
    return (int(np.argmin(dt)), int(np.argmax(dt)))
