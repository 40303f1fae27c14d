"""GPU parity of ssm_hippo_dplr (HiPPO generator -> DPLR parameters) through
its C ABI against the float64 oracle, on the same seeded input rows.

The eigenvalues are distinct, so Lambda, V and P are unique once the order
(ascending imaginary part) and the phase rule (first column of P real and
non-negative) are fixed; every output is compared element by element.
Tolerance: max |gpu - oracle| <= 1e-6 x max |oracle| per output array.  The
device computes in float64 and rounds to complex64 (2^-24 ~ 6e-8 relative per
element); the float64 solvers agree to ~1e-12 of the largest entry.

End to end, the DPLR parameters feed the filter path (ssm_discretize,
ssm_kernel_gen): the kernel must equal the oracle's kernel of the original
generator (G, B, C), which a state change leaves unchanged, within
2e-4 x max |K| per channel."""
import numpy as np
import pytest

import oracle as O
import oracle.hippo_oracle as HO
from tests.parity import assert_rows_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"
TOL = 1e-6


def _ssm():
    from structured_state_space_amd import ssm
    return ssm


def _rows(seed, n, N):
    rng = np.random.default_rng(seed)
    return ((rng.normal(size=(n, N)) + 1j * rng.normal(size=(n, N))) / np.sqrt(2)).astype(np.complex64)


def _close(got, ref, what):
    got = got.detach().cpu().numpy().astype(np.complex128)
    err = np.abs(got - ref).max()
    scale = max(np.abs(ref).max(), 1e-30)
    assert err <= TOL * scale, f"{what}: max error {err:.3e} vs {TOL:.0e} x {scale:.3e}"


@pytest.mark.parametrize("kind", HO.KINDS)
@pytest.mark.parametrize("N,theta", [(1, 1.0), (2, 0.6), (3, 2.0), (17, 1.0), (64, 1.0), (100, 0.3), (256, 1.0)])
def test_hippo_dplr_matches_oracle(kind, N, theta):
    ssm = _ssm()
    B, C = _rows(N, 2, N), _rows(N + 1, 5, N)
    out = ssm.hippo_dplr(kind, N, theta, torch.from_numpy(B).to(DEV), torch.from_numpy(C).to(DEV), want_v=True)
    torch.cuda.synchronize()
    ref = HO.hippo_dplr(kind, N, theta, B.astype(np.complex128), C.astype(np.complex128))
    _close(out["Lambda"], ref["Lambda"], "Lambda")
    _close(out["P"], ref["P"], "P")
    _close(out["V"], ref["V"], "V")
    _close(out["Bt"], ref["Bt"], "Bt")
    _close(out["Ct"], ref["Ct"], "Ct")


@pytest.mark.parametrize("kind,N", [("legs", 1024), ("legt", 1000), ("lagt", 777)])
def test_hippo_dplr_large(kind, N):
    """Largest sizes: element parity for Lambda and P, and the unitarity and
    reconstruction of V checked on the CPU from the device output."""
    ssm = _ssm()
    out = ssm.hippo_dplr(kind, N, 1.0, None, torch.from_numpy(_rows(5, 3, N)).to(DEV), want_v=True)
    torch.cuda.synchronize()
    ref = HO.hippo_dplr(kind, N, 1.0, None, _rows(5, 3, N).astype(np.complex128))
    _close(out["Lambda"], ref["Lambda"], "Lambda")
    _close(out["P"], ref["P"], "P")
    _close(out["V"], ref["V"], "V")
    _close(out["Ct"], ref["Ct"], "Ct")
    assert out["Bt"] is None
    V = out["V"].cpu().numpy().astype(np.complex128)
    assert np.abs(V.conj().T @ V - np.eye(N)).max() <= 1e-5
    Lam = out["Lambda"].cpu().numpy().astype(np.complex128)
    P = out["P"].cpu().numpy().astype(np.complex128)
    At = HO.transformed_generator(kind, N, 1.0)
    rec = V @ (np.diag(Lam) - P @ P.conj().T) @ V.conj().T
    assert np.abs(rec - At).max() <= 1e-5 * np.abs(At).max()


def test_hippo_dplr_repeat_is_deterministic():
    """Two calls with the same workspace give identical bits (no state is
    carried between calls)."""
    ssm = _ssm()
    N = 64
    ws = torch.empty(ssm.workspace_bytes(ssm.OP_HIPPO, 0, 0, N, 0, 0), dtype=torch.uint8, device=DEV)
    C = torch.from_numpy(_rows(9, 4, N)).to(DEV)
    a = ssm.hippo_dplr("legt", N, 0.5, None, C, want_v=True, workspace=ws)
    b = ssm.hippo_dplr("legs", 32, 1.0, None, C[:, :32].contiguous(), workspace=ws)
    c = ssm.hippo_dplr("legt", N, 0.5, None, C, want_v=True, workspace=ws)
    torch.cuda.synchronize()
    for k in ("Lambda", "P", "V", "Ct"):
        assert torch.equal(a[k], c[k]), k
    _close(b["Lambda"], HO.hippo_dplr("legs", 32)["Lambda"], "Lambda (legs 32)")


@pytest.mark.parametrize("kind,N,dt,L", [("legs", 64, 0.01, 1024), ("legt", 64, 0.01, 1000), ("lagt", 32, 0.05, 300)])
def test_hippo_parameters_feed_the_filter_path(kind, N, dt, L):
    """DPLR parameters from the device, discretised and evaluated by the
    filter path, against the oracle's kernel of the dense generator."""
    ssm = _ssm()
    H = 3
    B = _rows(21, 1, N)
    C = _rows(22, H, N)
    hp = ssm.hippo_dplr(kind, N, 1.0, torch.from_numpy(B).to(DEV), torch.from_numpy(C).to(DEV))
    Lam = hp["Lambda"][None].expand(H, N).contiguous()
    P = hp["P"][None].expand(H, N, hp["P"].shape[1]).contiguous()
    Bv = hp["Bt"].expand(H, N).contiguous()
    dts = torch.full((H,), dt, dtype=torch.float32, device=DEV)
    Ct = ssm.discretize(Lam, P, P, Bv, hp["Ct"], dts, L, want_bbar=False)["Ctilde"]
    out = ssm.kernel_gen(Lam, P, P, Bv, Ct, dts, L)
    torch.cuda.synchronize()
    assert (out["status"].cpu().numpy() == 0).all()
    K = out["K"].cpu().numpy()
    G = HO.hippo_generator(kind, N, 1.0).astype(np.complex128)
    Ab, Bb, st = O.bilinear(G, B[0].astype(np.complex128), dt)
    assert st == O.OK
    ref = np.array([O.kernel_by_iteration(Ab, Bb, C[h].astype(np.complex128), L) for h in range(H)])
    assert_rows_close(K, ref, what=f"{kind} kernel")
