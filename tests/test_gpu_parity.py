"""GPU parity: the HIP library through its C ABI against the complex128 oracle,
on the same seeded inputs.  Tolerance: max error <= 2e-4 x max|reference| per
channel (kernel, root values) and per batch row (outputs); integer and index
work (transform sizes, statuses) bit-exact."""
import functools

import numpy as np
import pytest

import oracle as O
from structured_state_space_amd import inputs as I
import sys

from tests.parity import TOL, assert_rows_close, extreme_step_channels, sample_channels

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"
STATUS_NAME = {0: O.OK, 16: O.RESONANT_CORRECTION, 17: O.RESONANT_DIAGONAL, 18: O.SINGULAR_BILINEAR}


@functools.lru_cache(maxsize=None)
def _ssm():
    from structured_state_space_amd import ssm
    return ssm


def _dev(params):
    return _ssm().to_device(params, DEV)


def _np(t):
    return t.detach().cpu().numpy()


@functools.lru_cache(maxsize=None)
def _workload(idx):
    return I.workload(idx)


def _oracle_channel(params, h, u_rows=None, taps=None):
    c = params.channel(h)
    return O.channel_reference(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], c["D"], u_rows,
                               params.L, kernel_taps=taps)


@functools.lru_cache(maxsize=None)
def _oracle_for(idx, nsample, with_y):
    w, p, u = _workload(idx)
    chans = sample_channels(p.H, nsample, seed=idx, forced=extreme_step_channels(p.dt))
    refs = {int(h): _oracle_channel(p, int(h), u[:, h, :] if with_y else None) for h in chans}
    return chans, refs


# ---------------------------------------------------------------------------
# minimum slice: root values H(z_k) from the oracle's truncated-output vector
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("idx,nsample", [(0, 1), (1, 16)])
def test_root_values_match_resolvent(idx, nsample):
    ssm = _ssm()
    w, p, u = _workload(idx)
    chans, refs = _oracle_for(idx, nsample, False)
    sub = p.select(chans)
    sub.C = np.stack([refs[int(h)]["Ctilde"] for h in chans]).astype(np.complex64)
    d = _dev(sub)
    out = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], p.L, want_kernel=True,
                         want_roots=True)
    roots, st = _np(out["roots"]), _np(out["status"])
    assert np.all(st == 0)
    M = O.transform_length(p.L)
    ref = []
    for i, h in enumerate(chans):
        c = sub.channel(i)
        Hk, s = O.root_values(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], M)
        assert s == O.OK
        ref.append(Hk)
    assert_rows_close(roots, np.array(ref), what="root values")
    # first L taps of the inverse transform against the matrix-power kernel
    K = _np(out["K"])
    Kref = np.array([O.kernel_by_iteration(refs[int(h)]["Abar"], refs[int(h)]["Bbar"], p.C[h], p.L)
                     for h in chans])
    assert_rows_close(K, Kref, what="kernel")


@pytest.mark.parametrize("L", [16385, 40000])
def test_root_values_multipass_lengths(L):
    """M = 32768 and 65536 (the multi-pass transforms): root values against the DFT of
    the first M taps of the matrix-power kernel, and the first L taps."""
    ssm = _ssm()
    p = I.random_params(L, 2, 8, 2, L, dt_range=(1e-3, 1e-2))
    M = O.transform_length(L)
    refs = [_oracle_channel(p, h, None, taps=M) for h in range(p.H)]
    sub = I.Params(p.Lambda, p.P, p.Q, p.B, np.stack([r["Ctilde"] for r in refs]).astype(np.complex64),
                   p.dt, p.D, L)
    d = _dev(sub)
    out = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_kernel=True, want_roots=True)
    assert np.all(_np(out["status"]) == 0)
    roots, K = _np(out["roots"]), _np(out["K"])
    assert_rows_close(roots, np.array([np.fft.fft(r["K"]) for r in refs]), what="root values")
    assert_rows_close(K, np.array([r["K"][:L] for r in refs]), what="kernel")


@pytest.mark.parametrize("H,N,r,L,nsample", [
    (256, 301, 1, 4096, 4),   # 4 roots per thread; 256 + 45 states, the last chunk padded to the unroll
    (256, 203, 2, 4096, 4),   # rank 2, 2 roots per thread; 128 + 75 states (padded)
    (8, 301, 1, 3000, 2),     # small grid: 1 root per thread, unroll 8; 256 + 45 states (padded)
    (4, 71, 3, 2048, 2),      # rank 3: 64 + 7 states (padded)
    (8, 300, 2, 2048, 2),     # rank 2 past one 256-state record chunk: 4 x 64 + 44 states in the sweep
    (4, 270, 3, 1024, 2),     # rank 3 past one record chunk
    (4, 66, 4, 1500, 2),      # rank 4: 64 + 2 states
    (256, 64, 1, 1024, 4),    # M = 1024, 256 channels: one launch per channel workgroup
    (256, 203, 2, 1000, 3),   # the same, rank 2, 128 + 75 states
])
def test_root_values_chunks_and_roots_per_thread(H, N, r, L, nsample):
    """Root values from a supplied C~ (random here: the kernel generator takes it
    as given) against the oracle's resolvent expression on sampled channels, at
    shapes whose state vectors span several staged chunks."""
    ssm = _ssm()
    p = I.random_params(H + N + r + L, H, N, r, L, lambda_kind="random")
    d = _dev(p)
    out = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_kernel=True,
                         want_roots=True)
    assert np.all(_np(out["status"]) == 0)
    roots, K = _np(out["roots"]), _np(out["K"])
    M = O.transform_length(L)
    chans = sample_channels(H, nsample, seed=N + r)
    ref = []
    for h in chans:
        c = p.channel(int(h))
        Hk, st = O.root_values(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], M)
        assert st == O.OK
        ref.append(Hk)
    ref = np.array(ref)
    assert_rows_close(roots[chans], ref, what="root values")
    # the kernel: first L taps of the inverse transform of the oracle's root values
    assert_rows_close(K[chans], np.fft.ifft(ref, axis=1)[:, :L], what="kernel")


# ---------------------------------------------------------------------------
# discretisation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("idx,nsample", [(0, 1), (1, 8), (2, 4), (3, 4), (4, 2)])
def test_discretize_matches_dense(idx, nsample):
    ssm = _ssm()
    w, p, u = _workload(idx)
    chans, refs = _oracle_for(idx, nsample, False)
    sub = p.select(chans)
    d = _dev(sub)
    out = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], p.L, want_abar=True)
    assert np.all(_np(out["status"]) == 0)
    Bbar, Abar, Ct = _np(out["Bbar"]), _np(out["Abar"]), _np(out["Ctilde"])
    for i, h in enumerate(chans):
        r = refs[int(h)]
        assert_rows_close(Bbar[i][None], r["Bbar"][None], what=f"Bbar ch{h}")
        assert np.abs(Abar[i] - r["Abar"]).max() <= TOL * np.abs(r["Abar"]).max()
        # C~ relative to |C| (the truncation term can be tiny)
        assert np.abs(Ct[i] - r["Ctilde"]).max() <= TOL * np.abs(p.C[h]).max()


# ---------------------------------------------------------------------------
# the whole path from the conventional C: discretize -> forward
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,r,L,bordered", [
    (100, 1, 4, True),       # states in registers, bordered form
    (200, 2, 300, False),    # states in registers, four per lane
    (300, 1, 100, False),    # LDS loop (N > 256)
    (700, 2, 3, True),       # LDS loop, bordered form
])
def test_discretize_register_and_lds_paths(N, r, L, bordered):
    """C~ by the register-resident adjoint steps (N <= 256) and by the LDS loop
    (larger N), each with and without an exactly zero d_j, against the dense
    oracle."""
    ssm = _ssm()
    H = 2
    p = I.random_params(N + 7 * r, H, N, r, L, dt_range=(1.0, 1.0) if bordered else (1e-3, 1e-1),
                        lambda_kind="random")
    if bordered:
        # d_j = 1 - (dt/2) lambda_j = 0 exactly for one state of each channel
        # (dt = 1).  Abar then has an eigenvalue of order -4/delta, delta ~ 1/N
        # from the low-rank term, so C~ is checked over a few adjoint steps only.
        p.Lambda[:, N // 3] = np.complex64(2.0)
    d = _dev(p)
    out = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L)
    assert np.all(_np(out["status"]) == 0)
    Bbar, Ct = _np(out["Bbar"]), _np(out["Ctilde"])
    for h in range(H):
        c = p.channel(h)
        ref = O.discretize_channel(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], float(c["dt"]), L)
        assert ref["status"] == O.OK
        assert_rows_close(Bbar[h][None], ref["Bbar"][None], what=f"Bbar h{h}")
        assert_rows_close(Ct[h][None], ref["Ctilde"][None], what=f"C~ h{h}")


@pytest.mark.parametrize("idx,nsample", [(0, 1), (1, 12), (2, 4), (3, 6),
                                         pytest.param(4, 4, marks=pytest.mark.timeout(600))])
def test_forward_end_to_end(idx, nsample):
    """Whole rows of K and y against the oracle on sampled channels; the
    channels with the smallest and the largest step are always among them."""
    ssm = _ssm()
    w, p, u = _workload(idx)
    chans, refs = _oracle_for(idx, nsample, True)
    d = _dev(p)
    disc = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], p.L, want_bbar=False)
    assert np.all(_np(disc["status"]) == 0)
    ut = torch.from_numpy(u).to(DEV)
    out = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], disc["Ctilde"], d["dt"], d["D"], ut, want_kernel=True)
    torch.cuda.synchronize()
    assert np.all(_np(out["status"]) == 0)
    K = _np(out["K"])
    y = _np(out["y"])
    worst_k = worst_y = 0.0
    for h in chans:
        r = refs[int(h)]
        worst_k = max(worst_k, assert_rows_close(K[h][None], r["K"][None], what=f"K ch{h}"))
        worst_y = max(worst_y, assert_rows_close(y[:, h, :], r["y"], what=f"y ch{h}"))
    # on the real stderr, so the margin under the tolerance shows in any run log
    sys.__stderr__.write(f"[parity] workload {w.name}: channels {[int(h) for h in chans]} "
                         f"(dt {float(p.dt[chans].min()):.3g}..{float(p.dt[chans].max()):.3g}): "
                         f"worst K err {worst_k:.3e}, worst y err {worst_y:.3e}\n")
    sys.__stderr__.flush()


# ---------------------------------------------------------------------------
# the convolution on its own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Bsz,H,L", [(1, 1, 1), (1, 1, 2), (3, 2, 3), (2, 3, 17), (5, 4, 100), (2, 9, 1000),
                                     (4, 8, 1024), (3, 5, 3000), (2, 3, 8192), (1, 2, 16384), (4, 2, 16384),
                                     (3, 2, 20000), (1, 1, 32768), (2, 1, 65536), (3, 1, 65536)])
def test_fftconv_matches_direct_sum(Bsz, H, L):
    ssm = _ssm()
    rng = np.random.default_rng(L * 7 + H)
    K = rng.standard_normal((H, L)).astype(np.float32) * np.exp(-np.arange(L) / max(1, L / 4)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    u = rng.standard_normal((Bsz, H, L)).astype(np.float32)
    y = _np(ssm.fftconv(torch.from_numpy(K).to(DEV), torch.from_numpy(u).to(DEV), torch.from_numpy(D).to(DEV)))
    # every row in full against the direct sum, 2e-4 x max|y| per row (at
    # L = 65536 the oracle's lag loop takes a few seconds per channel)
    worst = 0.0
    for h in range(H):
        ref = O.causal_conv(K[h].astype(np.float64), u[:, h, :], float(D[h])).real
        worst = max(worst, assert_rows_close(y[:, h, :], ref, what=f"conv h{h}"))
    sys.__stderr__.write(f"[parity] fftconv Bsz={Bsz} H={H} L={L}: worst y err {worst:.3e}\n")
    sys.__stderr__.flush()


def test_fftconv_complex_kernel_uses_real_part():
    ssm = _ssm()
    rng = np.random.default_rng(3)
    H, L = 3, 50
    Kc = (rng.standard_normal((H, L)) + 1j * rng.standard_normal((H, L))).astype(np.complex64)
    u = rng.standard_normal((2, H, L)).astype(np.float32)
    y = _np(ssm.fftconv(torch.from_numpy(Kc).to(DEV), torch.from_numpy(u).to(DEV)))
    for h in range(H):
        ref = O.causal_conv(Kc[h].real.astype(np.float64), u[:, h, :], 0.0).real
        assert_rows_close(y[:, h, :], ref, what="complex K")


# ---------------------------------------------------------------------------
# the worked example and the statuses
# ---------------------------------------------------------------------------
def test_cumsum_example_through_the_library():
    """A = 0, B = C = 1, dt = 1, D = 0: Abar = Bbar = 1 exactly, C~ = 0, K = 1, y = cumsum(u)."""
    ssm = _ssm()
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cumsum_example.json")))
    L = len(g["u"])
    p = I.cumsum_model(L)
    d = _dev(p)
    out = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_abar=True)
    assert _np(out["Abar"])[0, 0, 0] == 1 and _np(out["Bbar"])[0, 0] == 1
    assert _np(out["Ctilde"])[0, 0] == 0
    K = torch.ones((1, L), dtype=torch.float32, device=DEV)
    u = torch.tensor(g["u"], dtype=torch.float32, device=DEV).reshape(1, 1, L)
    y = _np(ssm.fftconv(K, u, torch.zeros(1, device=DEV)))[0, 0]
    np.testing.assert_allclose(y, g["y"], atol=TOL * np.abs(g["y"]).max())
    # the filter mode is resonant at z = 1 for this model (s(1) = 0 = lambda)
    kg = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L)
    assert STATUS_NAME[int(_np(kg["status"])[0])] == O.RESONANT_DIAGONAL
    assert np.isnan(_np(kg["K"])).all()


@pytest.mark.parametrize("name", ["resonant-diagonal", "resonant-correction", "singular-bilinear", "bordered"])
def test_status_cases(name):
    ssm = _ssm()
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "status_cases.json")))
    c = [c for c in g["cases"] if c["name"] == name][0]
    cp = lambda a: (np.asarray(a, np.float64)[..., 0] + 1j * np.asarray(a, np.float64)[..., 1])
    lam, P, Q, B, C = cp(c["Lambda"]), cp(c["P"]), cp(c["Q"]), cp(c["B"]), cp(c["C"])
    N, r, L = len(lam), P.shape[1], c["L"]
    p = I.Params(lam[None].astype(np.complex64), P[None].astype(np.complex64), Q[None].astype(np.complex64),
                 B[None].astype(np.complex64), C[None].astype(np.complex64),
                 np.array([c["dt"]], np.float32), np.array([0.5], np.float32), L)
    d = _dev(p)
    disc = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_abar=True)
    assert STATUS_NAME[int(_np(disc["status"])[0])] == c["expect_bilinear"]
    if c["expect_bilinear"] != O.OK:
        assert np.isnan(_np(disc["Ctilde"])).all() and np.isnan(_np(disc["Abar"])).all()
        return
    ref = O.discretize_channel(lam, P, Q, B, C, c["dt"], L)
    np.testing.assert_allclose(_np(disc["Abar"])[0], ref["Abar"], atol=1e-5 * np.abs(ref["Abar"]).max())
    np.testing.assert_allclose(_np(disc["Bbar"])[0], ref["Bbar"], atol=1e-5 * np.abs(ref["Bbar"]).max())
    # filter statuses are evaluated with C itself as the supplied vector (they do not depend on it)
    kg = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L)
    assert STATUS_NAME[int(_np(kg["status"])[0])] == c["expect_filter"]
    u = torch.ones((1, 1, L), dtype=torch.float32, device=DEV)
    fw = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u, want_kernel=True)
    assert STATUS_NAME[int(_np(fw["status"])[0])] == c["expect_filter"]
    if c["expect_filter"] != O.OK:
        assert np.isnan(_np(fw["y"])).all() and np.isnan(_np(fw["K"])).all()


def test_invalid_step_status():
    ssm = _ssm()
    p = I.random_params(5, 3, 4, 1, 16)
    p.dt[1] = 0.0
    d = _dev(p)
    kg = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], 16)
    st = _np(kg["status"])
    assert list(st) == [0, ssm.ST_INVALID_STEP, 0]
    assert np.isnan(_np(kg["K"])[1]).all() and np.isfinite(_np(kg["K"])[[0, 2]]).all()


# ---------------------------------------------------------------------------
# launch forms: the single launch (one workgroup per channel) against the
# separate root-value / transform / convolution kernels and the oracle,
# including a channel with an invalid step and one with an exact pole
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("r,L,Bsz,N", [(1, 1024, 8, 48), (2, 600, 3, 48), (1, 777, 1, 48), (3, 1000, 6, 48),
                                        (1, 900, 2, 300), (2, 1024, 4, 200), (4, 1024, 2, 40)])
def test_single_launch_form(r, L, Bsz, N):
    # N = 300 (r = 1) and 200 (r = 2) take more than one staged chunk of states
    ssm = _ssm()
    H = 256
    assert ssm.forward_form(Bsz, H, L) == 1
    p = I.random_params(7000 + 10 * r + Bsz + N, H, N, r, L)
    p.dt[5] = 0.0                       # invalid step
    p.dt[7] = 0.5                       # a = 2/dt = 4 exactly; tan(pi/4) = 1 exactly
    p.Lambda[7, 0] = 4.0j               # so s(z_{M/4}) = lambda_0: an exact pole
    u = I.random_input(L + Bsz, Bsz, H, L)
    d = _dev(p)
    ut = torch.from_numpy(u).to(DEV)
    Ct = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_bbar=False)["Ctilde"]
    fw = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], ut, want_kernel=True)
    # the kernel generator at M = 1024 and 256 channels takes the same one-launch
    # form without rows; on 128 channels it takes the separate root-value and
    # transform kernels
    kg = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], L, want_roots=True)
    hs = slice(0, 128)
    kg2 = ssm.kernel_gen(d["Lambda"][hs], d["P"][hs], d["Q"][hs], d["B"][hs], Ct[hs], d["dt"][hs], L,
                         want_roots=True)
    y_sep = ssm.fftconv(kg2["K"], ut[:, hs].contiguous(), D=d["D"][hs])
    torch.cuda.synchronize()
    st, st_kg, st_sep = _np(fw["status"]), _np(kg["status"]), _np(kg2["status"])
    expect = np.zeros(H, np.int32)
    expect[5], expect[7] = ssm.ST_INVALID_STEP, ssm.ST_RESONANT_DIAGONAL
    assert list(st) == list(expect) and list(st_kg) == list(expect) and list(st_sep) == list(expect[hs])
    K, y, Kg, Ks, ys = _np(fw["K"]), _np(fw["y"]), _np(kg["K"]), _np(kg2["K"]), _np(y_sep)
    R, Rs = _np(kg["roots"]), _np(kg2["roots"])
    for h in (5, 7):
        assert np.isnan(K[h]).all() and np.isnan(y[:, h, :]).all() and np.isnan(Kg[h]).all()
    assert np.isnan(R[5]).all() and np.isnan(Rs[5]).all()
    ok = np.array([h for h in range(H) if h not in (5, 7)])
    assert np.isfinite(K[ok]).all() and np.isfinite(y[:, ok, :]).all() and np.isfinite(Kg[ok]).all()
    for h in ok:
        assert_rows_close(Kg[h][None], K[h][None], what=f"K h{h}: kernel generator vs forward")
        if h < 128:
            assert_rows_close(K[h][None], Ks[h][None], what=f"K h{h} vs separate kernels")
            assert_rows_close(R[h][None], Rs[h][None], what=f"root values h{h} vs separate kernels")
            assert_rows_close(y[:, h, :], ys[:, h, :], what=f"y h{h} vs separate kernels")
    for h in sample_channels(H, 3, seed=r + L):
        h = int(h)
        if h in (5, 7):
            continue
        c = p.channel(h)
        ref = O.channel_reference(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], c["D"], u[:, h, :], L)
        assert_rows_close(K[h][None], ref["K"][None], what=f"K h{h} vs oracle")
        assert_rows_close(y[:, h, :], ref["y"], what=f"y h{h} vs oracle")


# ---------------------------------------------------------------------------
# ranks 2 and 3: root values on the float16 matrix cores in split precision
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("r,L", [(2, 2048), (3, 2048), (2, 20000)])
def test_split_precision_root_values_hard_cases(r, L):
    """A state 1e-6 from a root and outside the low-rank term, so H has a pole
    there (its scaled Cauchy entries pass the float16 range and the root takes
    the float32 recheck; with a low-rank coupling the Woodbury terms would cancel
    to a value the float32 inputs do not determine), weights across eight decades, B = 0
    (every family with B vanishes), the smallest and the largest step.  Root
    values against the oracle's resolvent expression (the near-pole root also
    against its own magnitude, and at M <= 4096 the rest of its row against the
    largest of the rest), the
    kernel against the inverse transform of those, and the forward outputs
    (wave-structured transforms) against the oracle's recurrence."""
    ssm = _ssm()
    H, N, Bsz = 6, 72, 2
    p = I.random_params(900 + 10 * r + L, H, N, r, L, lambda_kind="random")
    M = O.transform_length(L)
    kp = M // 4
    p.dt[0] = 0.5                                    # a = 2/dt = 4 and tan(pi/4) = 1: s(z_{M/4}) = 4i
    p.Lambda[0, 3] = np.complex64(-1e-7 + 1j * (4.0 + 1e-6))
    p.P[0, 3], p.Q[0, 3] = 0, 0                      # decoupled from the low-rank term: a pole of H itself
    w = np.logspace(0, -8, N).astype(np.float32)
    p.P[1] *= w[:, None]
    p.Q[1] *= w[::-1, None]
    p.B[1] *= w
    p.B[2] = 0
    p.dt[3], p.dt[4] = 1e-4, 1.0
    d = _dev(p)
    out = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_kernel=True,
                         want_roots=True)
    assert np.all(_np(out["status"]) == 0)
    roots, K = _np(out["roots"]), _np(out["K"])
    ref = []
    for h in range(H):
        c = p.channel(h)
        Hk, st = O.root_values(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], M)
        assert st == O.OK
        ref.append(Hk)
    ref = np.array(ref)
    assert np.abs(ref[0, kp]) > 1e2 * np.abs(np.delete(ref[0], kp)).max()   # the pole dominates its row
    assert abs(roots[0, kp] - ref[0, kp]) <= TOL * abs(ref[0, kp])
    if M <= 4096:
        # the rest of the row against its own largest value; at larger M the
        # pole's neighbours are within ~1e-3 of it, where rounding s(z_k) = i a t_k
        # to float32 alone moves them by more than the tolerance of that value
        assert_rows_close(np.delete(roots[0], kp)[None], np.delete(ref[0], kp)[None], what="root values ch0 (rest)")
    assert_rows_close(roots, ref, what="root values")
    assert not np.any(roots[2])                      # B = 0: exactly zero
    assert_rows_close(K, np.fft.ifft(ref, axis=1)[:, :L], what="kernel")
    # the forward path (roots in the transforms' order for M >= 1024)
    u = I.random_input(L + r, Bsz, H, L)
    disc = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_bbar=False)
    assert np.all(_np(disc["status"]) == 0)
    fw = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], disc["Ctilde"], d["dt"], d["D"],
                     torch.from_numpy(u).to(DEV), want_kernel=True)
    assert np.all(_np(fw["status"]) == 0)
    Kf, y = _np(fw["K"]), _np(fw["y"])
    for h in range(H):
        r_ = _oracle_channel(p, h, u[:, h, :])
        assert_rows_close(Kf[h][None], r_["K"][None], what=f"forward K h{h}")
        assert_rows_close(y[:, h, :], r_["y"], what=f"y h{h}")


@pytest.mark.parametrize("order,r,kind,N", [
    ("reversed", 2, "s4", 64), ("shuffled", 2, "s4", 64), ("shuffled", 3, "random", 64),
    ("shuffled", 2, "s4", 40), ("asis", 3, "s4", 57),
    ("reversed", 1, "s4", 256), ("shuffled", 1, "s4", 130), ("shuffled", 1, "random", 200),
])
def test_far_field_root_values(order, r, kind, N):
    """The split-precision kernel (ranks 2 and 3, and rank 1 from 128 states)
    where many waves of roots take the far-field moment form (the sum over the
    states replaced by 8 to 40 moment terms).  Poles given in reversed or
    shuffled order, steps across
    [1e-3, 1e-1], N with a ragged last block.  Root values (natural order) and
    the forward path's kernel (the transforms' order) against the oracle.  With
    the S4 poles at a tenth of the path tolerance: the expansions' tails are
    below 5 2^-24 of the sums of |terms|, so an error in a moment, a power or a
    scale shows here.  The random poles (Re down to -0.1) have resonance peaks
    where rounding s = i a t to float32 alone moves the value by ~4e-5 of the
    row's largest (with or without the far forms): those take the path
    tolerance, and so do the S4 poles of more than 64 states, whose resonances
    reach Im lambda ~ 800, where the same rounding moves a root value by up to
    ~6e-5 of the row's largest."""
    ssm = _ssm()
    H, L, Bsz = 8, 16384, 2
    p = I.random_params(7000 + 10 * r + N, H, N, r, L, lambda_kind=kind)
    if order != "asis":
        perm = np.arange(N)[::-1] if order == "reversed" else np.random.default_rng(r + N).permutation(N)
        p.Lambda, p.P, p.Q = p.Lambda[:, perm].copy(), p.P[:, perm].copy(), p.Q[:, perm].copy()
        p.B, p.C = p.B[:, perm].copy(), p.C[:, perm].copy()
    d = _dev(p)
    out = ssm.kernel_gen(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_kernel=True,
                         want_roots=True)
    assert np.all(_np(out["status"]) == 0)
    roots = _np(out["roots"])
    ref = []
    for h in range(H):
        c = p.channel(h)
        Hk, st = O.root_values(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], L)
        assert st == O.OK
        ref.append(Hk)
    ref = np.array(ref)
    tol = TOL / 10 if kind == "s4" and N <= 64 else TOL
    assert_rows_close(roots, ref, tol=tol, what="root values")
    u = I.random_input(L + N, Bsz, H, L)
    fw = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"],
                     torch.from_numpy(u).to(DEV), want_kernel=True)
    assert np.all(_np(fw["status"]) == 0)
    assert_rows_close(_np(fw["K"]), np.fft.ifft(ref, axis=1)[:, :L], tol=tol, what="forward kernel")


# ---------------------------------------------------------------------------
# edge cases: ragged and tiny lengths, odd batch, any N and r, unordered poles
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,N,r,L,Bsz,kind", [
    (1, 1, 1, 1, 1, "random"), (2, 3, 1, 2, 3, "random"), (3, 5, 2, 3, 1, "random"),
    (5, 100, 1, 100, 3, "s4"), (4, 17, 3, 257, 2, "random"), (3, 9, 4, 64, 2, "random"),
    (9, 64, 2, 1000, 5, "s4"), (2, 130, 1, 4097, 2, "random"), (2, 24, 1, 9000, 3, "random"),
    (2, 16, 1, 20000, 3, "random"),
])
def test_edge_cases_end_to_end(H, N, r, L, Bsz, kind):
    ssm = _ssm()
    p = I.random_params(H * 1000 + N + L, H, N, r, L, lambda_kind=kind)
    u = I.random_input(L, Bsz, H, L)
    d = _dev(p)
    disc = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_bbar=False)
    assert np.all(_np(disc["status"]) == 0)
    out = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], disc["Ctilde"], d["dt"], d["D"],
                      torch.from_numpy(u).to(DEV), want_kernel=True)
    assert np.all(_np(out["status"]) == 0)
    K, y = _np(out["K"]), _np(out["y"])
    for h in range(H):
        r_ = _oracle_channel(p, h, u[:, h, :])
        assert_rows_close(K[h][None], r_["K"][None], what=f"K h{h}")
        assert_rows_close(y[:, h, :], r_["y"], what=f"y h{h}")


# ---------------------------------------------------------------------------
# properties: determinism, linearity, causality, impulse response
# ---------------------------------------------------------------------------
def test_deterministic_and_linear_and_causal():
    ssm = _ssm()
    w, p, u = _workload(1)
    d = _dev(p)
    disc = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], p.L, want_bbar=False)
    ut = torch.from_numpy(u).to(DEV)
    run = lambda x: ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], disc["Ctilde"], d["dt"], d["D"], x)["y"]
    y1, y2 = run(ut), run(ut)
    assert torch.equal(y1, y2)                                   # bitwise run-to-run
    y3 = run(2.0 * ut)
    scale = y1.abs().amax(dim=-1, keepdim=True)
    assert ((y3 - 2.0 * y1).abs() <= 1e-5 * scale).all()          # linear
    t0 = 700
    up = ut.clone()
    up[:, :, t0:] += 1.0
    y4 = run(up)
    assert ((y4[:, :, :t0] - y1[:, :, :t0]).abs() <= 1e-5 * scale).all()   # causal
    # impulse response: u = delta_0 gives Re K + D delta
    imp = torch.zeros((1, p.H, p.L), device=DEV)
    imp[:, :, 0] = 1.0
    out = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], disc["Ctilde"], d["dt"], d["D"], imp, want_kernel=True)
    ref = out["K"].real.clone()
    ref[:, 0] += d["D"]
    err = (out["y"][0] - ref).abs().amax(dim=-1) / ref.abs().amax(dim=-1)
    assert float(err.max()) <= TOL


# ---------------------------------------------------------------------------
# complex output: y_im = Im(C^* x_t) = (Im K) * u, from the recurrence's
# imaginary part; y_re as ssm_forward's y
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,N,r,L,Bsz,kind", [
    (2, 8, 1, 1, 2, "random"),         # L = 1
    (3, 8, 1, 7, 5, "random"),         # several row pairs per wave, odd batch
    (3, 16, 1, 100, 3, "random"),      # shared input transforms, ragged L
    (4, 64, 2, 1024, 2, "s4"),
    (2, 16, 1, 1500, 2, "random"),     # M = 2048: two convolutions
    (2, 16, 2, 3000, 3, "random"),     # M = 4096: shared transforms, odd batch
    (2, 8, 1, 5000, 2, "random"),      # M = 8192: two convolutions
    (2, 8, 1, 20000, 1, "random"),     # multi-pass transforms (M = 32768)
])
def test_forward_complex_matches_recurrence(H, N, r, L, Bsz, kind):
    ssm = _ssm()
    p = I.random_params(H * 31 + N + L, H, N, r, L, lambda_kind=kind, dt_range=(1e-2, 1e-1))
    u = I.random_input(L + 3, Bsz, H, L)
    d = _dev(p)
    disc = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_bbar=False)
    ut = torch.from_numpy(u).to(DEV)
    out = ssm.forward_complex(d["Lambda"], d["P"], d["Q"], d["B"], disc["Ctilde"], d["dt"], d["D"], ut,
                              want_kernel=True)
    fw = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], disc["Ctilde"], d["dt"], d["D"], ut)
    torch.cuda.synchronize()
    assert np.all(_np(out["status"]) == 0)
    yre, yim, yf = _np(out["y_re"]), _np(out["y_im"]), _np(fw["y"])
    for h in sample_channels(H, 3, seed=L):
        h = int(h)
        c = p.channel(h)
        ref = O.discretize_channel(c["Lambda"], c["P"], c["Q"], c["B"], c["C"], c["dt"], L)
        y = O.recurrence(ref["Abar"], ref["Bbar"], c["C"], c["D"], u[:, h, :])
        assert_rows_close(yre[:, h, :], y.real, what=f"Re y h{h}")
        assert_rows_close(yim[:, h, :], y.imag, what=f"Im y h{h}")
        assert_rows_close(yre[:, h, :], yf[:, h, :], what=f"Re y vs ssm_forward h{h}")


def test_forward_complex_status_fills_nan():
    ssm = _ssm()
    p = I.random_params(9, 3, 6, 1, 50)
    p.dt[2] = -1.0
    u = torch.from_numpy(I.random_input(10, 2, 3, 50)).to(DEV)
    d = _dev(p)
    out = ssm.forward_complex(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u)
    torch.cuda.synchronize()
    assert list(_np(out["status"])) == [0, 0, ssm.ST_INVALID_STEP]
    for k in ("y_re", "y_im"):
        y = _np(out[k])
        assert np.isnan(y[:, 2, :]).all() and np.isfinite(y[:, :2, :]).all()
