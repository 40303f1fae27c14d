"""ssm_forward_noalloc (the library's fixed per-GPU scratch, no workspace)
against ssm_forward with a caller workspace, through the C ABI: the same
kernels on the same inputs, so the outputs must agree bit for bit (which is
inside the 2e-4 x max|y| per row bound).  Two calls in a row, the second on a
smaller shape, so that the second call runs on scratch the first one filled."""
import numpy as np
import pytest

from structured_state_space_amd import inputs as I
from tests.parity import assert_rows_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


def _case(seed, H, N, r, L, Bsz):
    from structured_state_space_amd import ssm
    p = I.random_params(seed, H, N, r, L)
    u = torch.from_numpy(I.random_input(seed, Bsz, H, L)).to(DEV)
    d = ssm.to_device(p, DEV)
    Ct = ssm.discretize(d["Lambda"], d["P"], d["Q"], d["B"], d["C"], d["dt"], L, want_bbar=False)["Ctilde"]
    return d, Ct, u


def _both(d, Ct, u):
    from structured_state_space_amd import ssm
    H, L = u.shape[1], u.shape[2]
    ref = ssm.forward(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], u, want_kernel=True)
    y = torch.full_like(u, float("nan"))
    K = torch.full((H, L), float("nan"), dtype=torch.complex64, device=DEV)
    st = torch.full((H,), -1, dtype=torch.int32, device=DEV)
    got = ssm.forward_noalloc(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], u, y=y, K_out=K, status=st)
    torch.cuda.synchronize()
    return ref, got


def _compare(ref, got):
    assert torch.equal(got["status"], ref["status"])
    assert int(ref["status"].abs().max()) == 0
    assert torch.equal(got["y"], ref["y"]), "y differs from ssm_forward"
    assert torch.equal(got["K"], ref["K"]), "K differs from ssm_forward"
    y, yr = got["y"].cpu().numpy(), ref["y"].cpu().numpy()
    assert_rows_close(y.reshape(-1, y.shape[-1]), yr.reshape(-1, yr.shape[-1]), what="y (no-allocation)")


def test_noalloc_matches_forward_two_calls():
    from structured_state_space_amd import ssm
    # first: the three-launch form at M = 4096 (root values, spectra and the
    # convolution all in the scratch); second: a smaller shape in the fused form
    shapes = [(31, 96, 64, 2, 3000, 5), (32, 24, 16, 1, 700, 3)]
    for seed, H, N, r, L, Bsz in shapes:
        assert ssm.workspace_bytes(ssm.OP_FORWARD, Bsz, H, N, r, L) <= ssm.NOALLOC_SCRATCH_BYTES
        d, Ct, u = _case(seed, H, N, r, L, Bsz)
        ref, got = _both(d, Ct, u)
        _compare(ref, got)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    from structured_state_space_amd import ssm
    H, N, r, L, Bsz = 1024, 8, 1, 16384, 2
    assert ssm.workspace_bytes(ssm.OP_FORWARD, Bsz, H, N, r, L) > ssm.NOALLOC_SCRATCH_BYTES
    d, Ct, u = _case(5, H, N, r, L, Bsz)
    with pytest.raises(ssm.SSMError) as e:
        ssm.forward_noalloc(d["Lambda"], d["P"], d["Q"], d["B"], Ct, d["dt"], d["D"], u)
    assert e.value.code == ssm.ERR_SCRATCH_LIMIT
