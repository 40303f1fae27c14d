"""The entry points under HIP graph capture (torch.cuda.graph): the library
launches kernels only (no allocation, memset or synchronisation), so a
captured call replays the same work.  Each captured graph is replayed several
times with eager work and synchronisation between the replays and the input
changed in place before each; every replay must equal, bit for bit, an eager
call on the same input (the kernels are deterministic)."""
import numpy as np
import pytest

from structured_state_space_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


def _ssm():
    from structured_state_space_amd import ssm
    return ssm


def _setup(H, N, r, L, Bsz, seed):
    ssm = _ssm()
    p = I.random_params(seed, H, N, r, L)
    d = ssm.to_device(p, DEV)
    Ct = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_bbar=False)["Ctilde"]
    inputs = [torch.from_numpy(I.random_input(seed + k, Bsz, H, L)).to(DEV) for k in range(4)]
    return d, Ct, inputs


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


def _eager_noise():
    a = torch.randn(1 << 20, device=DEV)
    return float((a * a).sum())


@pytest.mark.parametrize("H,N,r,L,Bsz", [
    (256, 64, 1, 1024, 8),     # one launch
    (6, 16, 1, 300, 5),        # two launches (spectra formed in the convolution)
    (8, 32, 2, 3000, 3),       # three launches, LDS-resident transforms
    (3, 16, 1, 20000, 2),      # three launches, multi-pass transforms
])
def test_forward_replays(H, N, r, L, Bsz):
    ssm = _ssm()
    d, Ct, inputs = _setup(H, N, r, L, Bsz, 31)
    u = inputs[0].clone()
    y = torch.empty_like(u)
    status = torch.empty(H, dtype=torch.int32, device=DEV)
    ws = torch.empty(ssm.workspace_bytes(ssm.OP_FORWARD, Bsz, H, N, r, L), dtype=torch.uint8, device=DEV)
    call = lambda: ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], u, y=y, status=status,
                               workspace=ws)
    g, _ = _capture(call)
    for k in range(1, 4):
        u.copy_(inputs[k])
        y.fill_(float("nan"))
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        ref = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], inputs[k])["y"]
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {k}"
        assert int(status.abs().max()) == 0


@pytest.mark.parametrize("L", [1000, 3000])
def test_forward_complex_replays(L):
    ssm = _ssm()
    H, N, r, Bsz = 4, 16, 1, 3
    d, Ct, inputs = _setup(H, N, r, L, Bsz, 41)
    u = inputs[0].clone()
    ws = torch.empty(ssm.workspace_bytes(ssm.OP_FORWARD_COMPLEX, Bsz, H, N, r, L), dtype=torch.uint8, device=DEV)
    call = lambda: ssm.forward_complex(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], u, workspace=ws)
    g, out = _capture(call)
    for k in range(1, 4):
        u.copy_(inputs[k])
        out["y_re"].fill_(float("nan"))
        out["y_im"].fill_(float("nan"))
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        ref = ssm.forward_complex(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], inputs[k])
        torch.cuda.synchronize()
        assert torch.equal(out["y_re"], ref["y_re"]) and torch.equal(out["y_im"], ref["y_im"]), f"replay {k}"


def test_step_replays_continue_the_stream():
    """A captured step call updates the state in place, so successive replays
    continue one stream exactly as successive eager calls do."""
    ssm = _ssm()
    H, N, r, T, Bsz = 4, 64, 1, 100, 2
    p = I.random_params(51, H, N, r, T)
    d = ssm.to_device(p, DEV)
    chunks = [torch.from_numpy(I.random_input(52 + k, Bsz, H, T)).to(DEV) for k in range(4)]
    u = chunks[0].clone()
    x = torch.zeros((Bsz, H, N), dtype=torch.complex64, device=DEV)
    y = torch.empty_like(u)
    status = torch.empty(H, dtype=torch.int32, device=DEV)
    call = lambda: ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], u, x=x, y=y, status=status)
    g, _ = _capture(call)          # the warm-up call advanced x by one chunk
    x.zero_()
    xr = torch.zeros_like(x)
    for k in range(4):
        u.copy_(chunks[k])
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        ref = ssm.step(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], d["D"], chunks[k], x=xr)
        torch.cuda.synchronize()
        assert torch.equal(y, ref["y"]), f"replay {k}"
        assert torch.equal(x, xr), f"state after replay {k}"
    assert np.isfinite(y.cpu().numpy()).all()


@pytest.mark.parametrize("lanes", [64, 16])
def test_step_prepared_replays(lanes):
    """The prepared form under capture: one ssm_step_prepare outside the
    graph, a captured ssm_step_prepared of T = 1 (a decode step) replayed as
    a stream; each replay equals an eager ssm_step_prepared call bit for bit."""
    ssm = _ssm()
    H, N, r, Bsz = 8, 64, 1, 2
    p = I.random_params(61, H, N, r, 16)
    d = ssm.to_device(p, DEV)
    prep = ssm.step_prepare(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"])
    steps = [torch.from_numpy(I.random_input(62 + k, Bsz, H, 1)).to(DEV) for k in range(5)]
    u = steps[0].clone()
    x = torch.zeros((Bsz, H, N), dtype=torch.complex64, device=DEV)
    y = torch.empty_like(u)
    status = torch.empty(H, dtype=torch.int32, device=DEV)
    call = lambda: ssm.step_prepared(prep, d["D"], u, x=x, y=y, status=status, lanes=lanes)
    g, _ = _capture(call)
    x.zero_()
    xr = torch.zeros_like(x)
    for k in range(5):
        u.copy_(steps[k])
        _eager_noise()
        g.replay()
        torch.cuda.synchronize()
        ref = ssm.step_prepared(prep, d["D"], steps[k], x=xr, lanes=lanes)
        torch.cuda.synchronize()
        assert torch.equal(y, ref["y"]), f"replay {k}"
        assert torch.equal(x, xr), f"state after replay {k}"
    assert int(status.abs().max()) == 0
