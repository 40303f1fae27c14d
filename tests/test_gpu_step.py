"""GPU parity of the recurrent (step) mode, ssm_step, through its C ABI against
the complex128 oracle's recurrence from a given state, on the same seeded
inputs.  Tolerance: max error <= 2e-4 x max|reference| per batch row for y and
per (row, channel) for the final state; statuses bit-exact."""
import json
import os

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


def _oracle(p, h, u_rows, x0_rows):
    """y (real part) and final states of channel h for every batch row."""
    c = p.channel(h)
    Abar, Bbar, st = O.bilinear(O.dplr_matrix(c["Lambda"], c["P"], c["Q"]), c["B"], float(c["dt"]))
    assert st == O.OK
    ys, xs = [], []
    for b in range(u_rows.shape[0]):
        y, x = O.recurrence_from(Abar, Bbar, c["C"], float(c["D"]), u_rows[b], x0_rows[b])
        ys.append(y.real)
        xs.append(x)
    return np.array(ys), np.array(xs)


@pytest.mark.parametrize("H,N,r,T,Bsz,kind", [
    (3, 8, 1, 200, 3, "random"),    # several 64-step blocks and a ragged tail
    (3, 64, 2, 130, 2, "s4"),       # one state per lane, rank 2
    (2, 100, 1, 64, 2, "random"),   # two states per lane (one partly empty)
    (2, 256, 1, 70, 1, "s4"),       # four states per lane
    (2, 17, 3, 65, 2, "random"),    # rank 3
    (2, 9, 4, 1, 1, "random"),      # rank 4, a single step
])
@pytest.mark.parametrize("lanes", [64, 16])
def test_step_matches_oracle(H, N, r, T, Bsz, kind, lanes):
    """Both layouts: one sequence per wave, and (N <= 64) four per wave in
    16-lane groups."""
    if lanes == 16 and N > 64:
        pytest.skip("16-lane groups hold at most 64 states")
    ssm = _ssm()
    p = I.random_params(100 * H + N + T, H, N, r, T, lambda_kind=kind)
    u = I.random_input(N + T, Bsz, H, T)
    x0 = _random_state(N + r, Bsz, H, N)
    d = ssm.to_device(p, DEV)
    xt = torch.from_numpy(x0).to(DEV)
    out = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], torch.from_numpy(u).to(DEV), x=xt,
                   lanes=lanes)
    torch.cuda.synchronize()
    assert np.all(_np(out["status"]) == 0)
    y, xT = _np(out["y"]), _np(out["x"])
    for h in range(H):
        yr, xr = _oracle(p, h, u[:, h, :], x0[:, h, :])
        assert_rows_close(y[:, h, :], yr, what=f"y h{h}")
        assert_rows_close(xT[:, h, :], xr, what=f"final state h{h}")


def test_step_streaming_equals_one_call():
    """A stream split into calls (the state carried in x) gives the same outputs
    and final state as one call: the same float32 steps, bit for bit."""
    ssm = _ssm()
    H, N, r, T, Bsz = 4, 64, 1, 300, 2
    p = I.random_params(77, H, N, r, T)
    u = torch.from_numpy(I.random_input(78, Bsz, H, T)).to(DEV)
    d = ssm.to_device(p, DEV)
    one = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u)
    x = torch.zeros((Bsz, H, N), dtype=torch.complex64, device=DEV)
    parts = []
    for a, b in [(0, 50), (50, 177), (177, 178), (178, 300)]:
        o = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u[:, :, a:b].contiguous(), x=x)
        parts.append(_np(o["y"]))
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate(parts, axis=2), _np(one["y"]))
    assert np.array_equal(_np(x), _np(one["x"]))


def test_step_from_zero_equals_forward():
    """From a zero state, T = L steps reproduce the filter path's output (the
    convolution with K_j = C^* Abar^j Bbar plus the skip term)."""
    ssm = _ssm()
    w, p, u = I.workload(1)
    sel = np.arange(0, p.H, 32)
    p = p.select(sel)
    u = np.ascontiguousarray(u[:, sel, :])
    d = ssm.to_device(p, DEV)
    ut = torch.from_numpy(u).to(DEV)
    st = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], ut)
    Ct = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], p.L, want_bbar=False)["Ctilde"]
    fw = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], ut)
    torch.cuda.synchronize()
    ys, yf = _np(st["y"]), _np(fw["y"])
    for h in range(len(sel)):
        assert_rows_close(ys[:, h, :], yf[:, h, :], what=f"step vs forward h{h}")


def _golden_case(name, T):
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "status_cases.json")))
    c = [c for c in g["cases"] if c["name"] == name][0]
    cp = lambda a: (np.asarray(a, np.float64)[..., 0] + 1j * np.asarray(a, np.float64)[..., 1])
    f = lambda a: cp(a)[None].astype(np.complex64)
    return I.Params(f(c["Lambda"]), f(c["P"]), f(c["Q"]), f(c["B"]), f(c["C"]), np.array([c["dt"]], np.float32),
                    np.array([0.5], np.float32), T)


def _run(p, u, x0):
    ssm = _ssm()
    d = ssm.to_device(p, DEV)
    out = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], torch.from_numpy(u).to(DEV),
                   x=torch.from_numpy(x0).to(DEV))
    torch.cuda.synchronize()
    return _np(out["status"]), _np(out["y"]), _np(out["x"])


def test_step_bordered_form():
    """A state with d_j = 1 - (dt/2) lambda_j exactly 0: the bordered solve,
    against the oracle's dense bilinear matrices."""
    T, Bsz = 40, 2
    p = _golden_case("bordered", T)
    u = I.random_input(9, Bsz, 1, T)
    x0 = _random_state(10, Bsz, 1, p.Lambda.shape[1])
    st, y, xT = _run(p, u, x0)
    assert list(st) == [0]
    yr, xr = _oracle(p, 0, u[:, 0, :], x0[:, 0, :])
    assert_rows_close(y[:, 0, :], yr, what="bordered y")
    assert_rows_close(xT[:, 0, :], xr, what="bordered final state")


def test_step_statuses():
    """An invalid step and a singular bilinear matrix: statuses as the
    discretisation's, NaN outputs and states for those channels only."""
    ssm = _ssm()
    T, Bsz = 70, 2
    p = I.random_params(11, 3, 6, 1, T)
    p.dt[1] = 0.0
    u = I.random_input(12, Bsz, 3, T)
    x0 = _random_state(13, Bsz, 3, 6)
    st, y, xT = _run(p, u, x0)
    assert list(st) == [0, ssm.ST_INVALID_STEP, 0]
    assert np.isnan(y[:, 1, :]).all() and np.isnan(xT[:, 1, :]).all()
    assert np.isfinite(y[:, [0, 2], :]).all() and np.isfinite(xT[:, [0, 2], :]).all()
    ps = _golden_case("singular-bilinear", T)
    st, y, xT = _run(ps, u[:, :1, :].copy(), x0[:, :1, :1].copy())
    assert list(st) == [ssm.ST_SINGULAR_BILINEAR]
    assert np.isnan(y).all() and np.isnan(xT).all()


def test_step_layout_choice():
    """lanes = 0: 16-lane groups from three sequences per SIMD (4 SIMDs per
    compute unit) and T >= 32 for ssm_step (T >= 8 for ssm_step_prepared),
    else one sequence per wave; each call equals the fixed layout it picks,
    bit for bit."""
    ssm = _ssm()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H, N, r = 64, 16, 1
    Bsz = -(-3 * 4 * cus // H)           # just enough sequences
    p = I.random_params(91, H, N, r, 40)
    d = ssm.to_device(p, DEV)
    prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
    for T, want_step, want_prep in [(40, 16, 16), (20, 64, 16), (4, 64, 64)]:
        u = torch.from_numpy(I.random_input(92 + T, Bsz, H, T)).to(DEV)
        run = lambda lanes: ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u, lanes=lanes)
        runp = lambda lanes: ssm.step_prepared(prep, d["D"], u, lanes=lanes)
        auto, fixed = run(0), run(want_step)
        pauto, pfixed = runp(0), runp(want_prep)
        torch.cuda.synchronize()
        assert torch.equal(auto["y"], fixed["y"]) and torch.equal(auto["x"], fixed["x"]), f"ssm_step T={T}"
        assert torch.equal(pauto["y"], pfixed["y"]) and torch.equal(pauto["x"], pfixed["x"]), f"prepared T={T}"
    # one sequence fewer per SIMD budget: one sequence per wave throughout
    Bsz_small = (3 * 4 * cus - 1) // H
    u = torch.from_numpy(I.random_input(99, Bsz_small, H, 40)).to(DEV)
    a = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u, lanes=0)
    b = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u, lanes=64)
    torch.cuda.synchronize()
    assert torch.equal(a["y"], b["y"])


def test_step_full_size_grouped_layout():
    """s4-h512-l3k at full size (16 x 512 sequences of 3000 steps, N = 64),
    the layout left to the library (16-lane groups here), for ssm_step and
    ssm_step_prepared: from a zero state every row must reproduce the
    filter path's output (ssm_forward, itself checked against the oracle at
    this size), and sampled sequences also the oracle's recurrence."""
    from tests.parity import sample_channels
    ssm = _ssm()
    w, p, u = I.workload("s4-h512-l3k")
    d = ssm.to_device(p, DEV)
    ut = torch.from_numpy(u).to(DEV)
    Ct = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], p.L, want_bbar=False)["Ctilde"]
    yf = _np(ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], ut)["y"])
    st = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], ut)
    prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
    sp = ssm.step_prepared(prep, d["D"], ut)
    torch.cuda.synchronize()
    for name, out in (("ssm_step", st), ("ssm_step_prepared", sp)):
        assert int(out["status"].abs().max()) == 0
        ys = _np(out["y"])
        for h in range(w.H):
            assert_rows_close(ys[:, h, :], yf[:, h, :], what=f"{name} vs forward h{h}")
    # ssm_step and ssm_step_prepared take the same layout here: equal bit for bit
    assert torch.equal(st["y"], sp["y"]) and torch.equal(st["x"], sp["x"])
    ys, xs = _np(st["y"]), _np(st["x"])
    for h in sample_channels(w.H, 3):
        b = int(h) % w.Bsz
        yr, xr = _oracle(p, int(h), u[b:b + 1, h, :], np.zeros((1, w.N), np.complex64))
        assert_rows_close(ys[b:b + 1, h, :], yr, what=f"y b{b} h{h}")
        assert_rows_close(xs[b:b + 1, h, :], xr, what=f"final state b{b} h{h}")
