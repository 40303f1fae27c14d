"""GPU checks of the step mode in two calls (ssm_step_prepare once per
parameter set, then ssm_step_prepared per chunk of the stream), through the C
ABI, in both layouts.  In either layout (64 lanes per sequence, or 16-lane
groups holding four sequences per wave, N <= 64) the prepared calls run
ssm_step's float32 recurrence in that layout from the same float32
constants, so y, final state and statuses equal ssm_step's bit for bit.  The
16-lane results, whose sums run in another order, are also compared with the
complex128 oracle's recurrence (max error <= 2e-4 x max|reference| per batch
row)."""
import ctypes

import numpy as np
import pytest

import oracle as O
from structured_state_space_amd import inputs as I
from tests.parity import assert_rows_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


def _ssm():
    from structured_state_space_amd import ssm
    return ssm


def _np(t):
    return t.detach().cpu().numpy()


def _random_state(seed, Bsz, H, N):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(Bsz, H, N)) + 1j * rng.normal(size=(Bsz, H, N))).astype(np.complex64)


def _both(p, u, x0, lanes=64):
    """(ssm_step result, prepared result, prepare status) on the same inputs,
    both calls in the same layout."""
    ssm = _ssm()
    d = ssm.to_device(p, DEV)
    ut = torch.from_numpy(u).to(DEV)
    ref = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], ut, x=torch.from_numpy(x0).to(DEV),
                   lanes=lanes)
    prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
    out = ssm.step_prepared(prep, d["D"], ut, x=torch.from_numpy(x0).to(DEV), lanes=lanes)
    torch.cuda.synchronize()
    return ref, out, _np(prep["status"])


def _assert_same(ref, out):
    assert np.array_equal(_np(out["status"]), _np(ref["status"]))
    assert np.array_equal(_np(out["y"]), _np(ref["y"]), equal_nan=True)
    assert np.array_equal(_np(out["x"]), _np(ref["x"]), equal_nan=True)


def _assert_oracle(p, u, x0, out, channels=None):
    """y and final state of the given channels against the oracle's recurrence."""
    y, xT = _np(out["y"]), _np(out["x"])
    for h in (range(p.H) if channels is None else channels):
        c = p.channel(h)
        Abar, Bbar, st = O.bilinear(O.dplr_matrix(c["Lambda"], c["P"], c["Q"]), c["B"], float(c["dt"]))
        assert st == O.OK
        yr, xr = [], []
        for b in range(u.shape[0]):
            yb, xb = O.recurrence_from(Abar, Bbar, c["C"], float(c["D"]), u[b, h], x0[b, h])
            yr.append(yb.real)
            xr.append(xb)
        assert_rows_close(y[:, h, :], np.array(yr), what=f"y h{h}")
        assert_rows_close(xT[:, h, :], np.array(xr), what=f"final state h{h}")


def _assert_grouped(p, u, x0, ref, out, channels=None):
    """16-lane groups: ssm_step and ssm_step_prepared equal bit for bit, and
    the values against the oracle."""
    _assert_same(ref, out)
    _assert_oracle(p, u, x0, out, channels)


@pytest.mark.parametrize("H,N,r,T,Bsz,kind", [
    (3, 8, 1, 200, 3, "random"),    # groups: one state per lane, 9 sequences (a ragged last wave)
    (3, 64, 2, 130, 2, "s4"),       # groups: four states per lane, rank 2
    (5, 30, 3, 70, 1, "random"),    # groups: two states per lane, rank 3, 5 sequences
    (2, 64, 4, 33, 3, "s4"),        # groups: rank 4
    (2, 100, 1, 64, 2, "random"),   # 64 lanes only: two states per lane (one partly empty)
    (2, 256, 1, 70, 1, "s4"),       # four states per lane
    (2, 9, 4, 1, 1, "random"),      # rank 4, a single step
    (2, 200, 4, 5, 3, "s4"),        # four states per lane, rank 4
])
def test_prepared_matches_step_and_oracle(H, N, r, T, Bsz, kind):
    p = I.random_params(100 * H + N + T, H, N, r, T, lambda_kind=kind)
    u = I.random_input(N + T, Bsz, H, T)
    x0 = _random_state(N + r, Bsz, H, N)
    ref, out, pst = _both(p, u, x0, lanes=64)
    assert np.all(pst == 0)
    _assert_same(ref, out)
    if N <= 64:
        ref, out, pst = _both(p, u, x0, lanes=16)
        _assert_grouped(p, u, x0, ref, out)


@pytest.mark.parametrize("lanes", [64, 16])
def test_prepared_matches_oracle(lanes):
    H, N, r, T, Bsz = 2, 64, 1, 150, 2
    p = I.random_params(5, H, N, r, T)
    u = I.random_input(6, Bsz, H, T)
    x0 = _random_state(7, Bsz, H, N)
    _, out, _ = _both(p, u, x0, lanes)
    y, xT = _np(out["y"]), _np(out["x"])
    for h in range(H):
        c = p.channel(h)
        Abar, Bbar, st = O.bilinear(O.dplr_matrix(c["Lambda"], c["P"], c["Q"]), c["B"], float(c["dt"]))
        assert st == O.OK
        for b in range(Bsz):
            yr, xr = O.recurrence_from(Abar, Bbar, c["C"], float(c["D"]), u[b, h], x0[b, h])
            assert_rows_close(y[b:b + 1, h, :], yr.real[None], what=f"y b{b} h{h}")
            assert_rows_close(xT[b:b + 1, h, :], xr[None], what=f"state b{b} h{h}")


def test_prepared_bordered_and_statuses():
    """The bordered form (a zero d_j) and the failing channels (invalid step,
    singular bilinear matrix): the prepare call reports the set-up statuses,
    and the prepared calls repeat them with NaN outputs, as ssm_step does."""
    from tests.test_gpu_step import _golden_case
    ssm = _ssm()
    T, Bsz = 40, 2
    p = _golden_case("bordered", T)
    u = I.random_input(9, Bsz, 1, T)
    x0 = _random_state(10, Bsz, 1, p.Lambda.shape[1])
    for lanes in (64, 16):
        ref, out, pst = _both(p, u, x0, lanes)
        assert list(pst) == [0]
        _assert_same(ref, out) if lanes == 64 else _assert_grouped(p, u, x0, ref, out)

    p = I.random_params(11, 3, 6, 1, 70)
    p.dt[1] = 0.0
    u = I.random_input(12, Bsz, 3, 70)
    x0 = _random_state(13, Bsz, 3, 6)
    for lanes in (64, 16):
        ref, out, pst = _both(p, u, x0, lanes)
        assert list(pst) == [0, ssm.ST_INVALID_STEP, 0]
        _assert_same(ref, out) if lanes == 64 else _assert_grouped(p, u, x0, ref, out, channels=[0, 2])
        assert np.isnan(_np(out["y"])[:, 1]).all() and np.isnan(_np(out["x"])[:, 1]).all()

    ps = _golden_case("singular-bilinear", 70)
    for lanes in (64, 16):
        ref, out, pst = _both(ps, u[:, :1, :].copy(), x0[:, :1, :1].copy(), lanes)
        assert list(pst) == [ssm.ST_SINGULAR_BILINEAR]
        _assert_same(ref, out)


def test_prepared_mixed_wave():
    """One wave holding a bordered channel (lambda_5 = 2/dt, so d_5 = 0
    exactly) beside Woodbury channels: the whole wave takes the bordered loop,
    and every channel still matches the oracle.  P_5 = Q_5 = 3 move the
    eigenvalue of A near lambda_5 to about -5, so that the channel is stable
    (the largest |eigenvalue| of Abar is 0.998 here) and 90 steps stay finite."""
    H, N, r, T, Bsz = 4, 16, 1, 90, 1
    p = I.random_params(31, H, N, r, T)
    p.dt[2] = 0.5
    p.Lambda[2, 5] = 4.0
    p.P[2, 5, 0] = 3.0
    p.Q[2, 5, 0] = 3.0
    u = I.random_input(32, Bsz, H, T)
    x0 = _random_state(33, Bsz, H, N)
    for lanes in (64, 16):
        ref, out, pst = _both(p, u, x0, lanes)
        assert np.all(pst == 0)
        _assert_same(ref, out) if lanes == 64 else _assert_grouped(p, u, x0, ref, out)


@pytest.mark.parametrize("N,lanes", [(64, 16), (64, 64), (100, 64), (64, 0)])
def test_prepared_streaming_equals_one_call(N, lanes):
    """One prepare, then a stream split into prepared calls of varied lengths
    (T = 1 included) and two batch sizes sharing the constants: in a fixed
    layout each equals one prepared call over the whole stream bit for bit
    (and ssm_step's: bit for bit with 64 lanes, to the parity bound with
    16).  With the layout left to the library (lanes = 0) short and long
    calls may take different layouts: the split stream then stays within
    the parity bound of the one call."""
    ssm = _ssm()
    H, r, T = 4, 1, 300
    p = I.random_params(77, H, N, r, T)
    d = ssm.to_device(p, DEV)
    prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
    for Bsz in (2, 5):
        u = torch.from_numpy(I.random_input(78 + Bsz, Bsz, H, T)).to(DEV)
        one = ssm.step_prepared(prep, d["D"], u, lanes=lanes)
        st = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u)
        x = torch.zeros((Bsz, H, N), dtype=torch.complex64, device=DEV)
        parts = []
        for a, b in [(0, 1), (1, 50), (50, 177), (177, 178), (178, 300)]:
            o = ssm.step_prepared(prep, d["D"], u[:, :, a:b].contiguous(), x=x, lanes=lanes)
            parts.append(_np(o["y"]))
        torch.cuda.synchronize()
        ys = np.concatenate(parts, axis=2)
        if lanes:
            assert np.array_equal(ys, _np(one["y"]))
            assert np.array_equal(_np(x), _np(one["x"]))
        for h in range(H):
            assert_rows_close(ys[:, h, :], _np(one["y"])[:, h, :], what=f"split vs one call h{h}")
        if lanes == 64:
            assert np.array_equal(_np(one["y"]), _np(st["y"]))
        else:
            for h in range(H):
                assert_rows_close(_np(one["y"])[:, h, :], _np(st["y"])[:, h, :], what=f"vs ssm_step h{h}")


def test_unprepared_blocks():
    """A buffer that ssm_step_prepare never wrote, and one written for another
    N: every channel reports SSM_ST_UNPREPARED with NaN outputs and state."""
    ssm = _ssm()
    H, N, r, T, Bsz = 3, 64, 1, 20, 2
    p = I.random_params(21, H, N, r, T)
    d = ssm.to_device(p, DEV)
    u = torch.from_numpy(I.random_input(22, Bsz, H, T)).to(DEV)
    nbytes = ssm.workspace_bytes(ssm.OP_STEP_PREPARED, 0, H, N, r, 0)
    blank = dict(prep=torch.zeros(nbytes, dtype=torch.uint8, device=DEV), H=H, N=N, r=r)
    for lanes in (64, 16):
        out = ssm.step_prepared(blank, d["D"], u, lanes=lanes)
        torch.cuda.synchronize()
        assert np.all(_np(out["status"]) == ssm.ST_UNPREPARED)
        assert np.isnan(_np(out["y"])).all() and np.isnan(_np(out["x"])).all()

    # written for N = 64, called with N = 32 (same block size per channel)
    prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
    N2 = 32
    assert ssm.workspace_bytes(ssm.OP_STEP_PREPARED, 0, H, N2, r, 0) == nbytes
    x = torch.zeros((Bsz, H, N2), dtype=torch.complex64, device=DEV)
    y = torch.empty_like(u)
    st = torch.empty(H, dtype=torch.int32, device=DEV)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    for lanes in (64, 16):
        rc = ssm.lib.ssm_step_prepared(Bsz, H, N2, r, T, vp(prep["prep"]), nbytes, vp(d["D"]), vp(u), vp(y), vp(x),
                                       vp(st), lanes, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == ssm.OK
        torch.cuda.synchronize()
        assert np.all(_np(st) == ssm.ST_UNPREPARED)
        assert np.isnan(_np(y)).all() and np.isnan(_np(x)).all()
        x.zero_()
        y.zero_()
