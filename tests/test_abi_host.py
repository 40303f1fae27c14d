"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/ssm.h declares, sizes transforms bit-exactly, and
rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")

ssm = pytest.importorskip("structured_state_space_amd.ssm", reason="HIP library not built")
import oracle as O  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(ssm.EXPORTS)
    for name in declared:
        assert hasattr(ssm.lib, name), name
    out = os.popen(f"nm -D --defined-only {ssm._LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", out), f"{name} not exported"


@pytest.mark.parametrize("L", [1, 2, 3, 5, 64, 100, 1000, 1024, 1025, 3000, 16384, 65536, 65537, 10**6])
def test_transform_lengths_bit_exact(L):
    assert ssm.transform_lengths(L) == (O.transform_length(L), O.conv_length(L))


def test_transform_lengths_rejects_nonpositive():
    with pytest.raises(ssm.SSMError):
        ssm.transform_lengths(0)


def test_forward_form_query():
    assert ssm.forward_form(8, 256, 1024) == 1     # one workgroup per channel
    assert ssm.forward_form(8, 256, 600) == 1      # M = 1024
    assert ssm.forward_form(8, 128, 1024) == 2     # too few channels for one launch
    assert ssm.forward_form(8, 256, 512) == 2      # M = 512
    assert ssm.forward_form(1, 1, 16) == 2
    assert ssm.forward_form(9, 256, 1024) == 3     # five row pairs per channel
    assert ssm.forward_form(2, 256, 1025) == 3     # M = 2048
    assert ssm.forward_form(2, 256, 8) == 3        # M = 8
    assert ssm.forward_form(2, 256, 65536) == 3    # multi-pass transforms
    for args in [(0, 1, 16), (1, 0, 16), (1, 1, 0)]:
        with pytest.raises(ssm.SSMError):
            ssm.forward_form(*args)


def test_status_strings():
    assert ssm.status_string(ssm.ST_RESONANT_DIAGONAL) == O.RESONANT_DIAGONAL
    assert ssm.status_string(ssm.ST_RESONANT_CORRECTION) == O.RESONANT_CORRECTION
    assert ssm.status_string(ssm.ST_SINGULAR_BILINEAR) == O.SINGULAR_BILINEAR
    assert ssm.status_string(ssm.OK) == "ok"
    assert ssm.status_string(ssm.ST_UNPREPARED) == "unprepared"
    assert ssm.status_string(12345) == "unknown code"


def test_workspace_sizes():
    # forward: roots [H,M] c64 + tile statuses + spectra [H,2,M] c64 + twiddle table [M] c64,
    # each region 256-byte aligned
    H, M = 256, 1024
    ws = ssm.workspace_bytes(ssm.OP_FORWARD, 8, H, 64, 1, 1024)
    assert ws >= H * M * 8 + H * 2 * M * 8 + M * 8
    assert ssm.workspace_bytes(ssm.OP_KERNEL_GEN, 1, H, 64, 1, 1024) >= H * M * 8 + M * 8
    assert ws % 256 == 0
    assert ssm.workspace_bytes(ssm.OP_DISCRETIZE, 1, H, 64, 1, 1024) == 0
    # ranks 2 and 3 add one record per channel for the split-precision root
    # values: N/8 weight blocks of 2048 bytes, 3 N floats of state headers, the
    # far roots' 5 moment blocks of 2048 bytes and 256 bytes of scales (the tile
    # count is the same as rank 1's here)
    rec = 64 * 256 + 3 * 64 * 4 + 5 * 2048 + 256
    for r in (2, 3):
        assert ssm.workspace_bytes(ssm.OP_FORWARD, 8, H, 64, r, 1024) - ws == H * rec
    assert ssm.workspace_bytes(ssm.OP_FORWARD, 8, H, 61, 2, 1024) - ws == H * rec
    assert ssm.workspace_bytes(ssm.OP_FORWARD, 8, H, 64, 4, 1024) == ws
    # fftconv for 1024 <= M <= 16384: spectra [H,2,M] c64, the table [M] c64 and the
    # wave-structured transforms' table [2M] c64 (sizes multiples of 256 here)
    assert ssm.workspace_bytes(ssm.OP_FFTCONV, 8, H, 1, 1, 1024) == H * 2 * M * 8 + M * 8 + 2 * M * 8
    # ragged L uses M = next power of two
    assert ssm.workspace_bytes(ssm.OP_FFTCONV, 1, 3, 1, 1, 3000) == 3 * 2 * 4096 * 8 + 4096 * 8 + 2 * 4096 * 8
    # below 1024 points no second table
    assert ssm.workspace_bytes(ssm.OP_FFTCONV, 1, 3, 1, 1, 512) == 3 * 2 * 512 * 8 + 512 * 8


@pytest.mark.parametrize("args,code", [
    ((ssm.OP_FORWARD, 8, 0, 64, 1, 1024), ssm.ERR_INVALID_ARGUMENT),
    ((ssm.OP_FORWARD, 0, 4, 64, 1, 1024), ssm.ERR_INVALID_ARGUMENT),
    ((ssm.OP_FORWARD, 8, 4, 0, 1, 1024), ssm.ERR_INVALID_ARGUMENT),
    ((ssm.OP_FORWARD, 8, 4, 64, 0, 1024), ssm.ERR_INVALID_ARGUMENT),
    ((ssm.OP_FORWARD, 8, 4, 64, 5, 1024), ssm.ERR_UNSUPPORTED),
    ((ssm.OP_FORWARD, 8, 4, 64, 1, 0), ssm.ERR_INVALID_ARGUMENT),
    ((ssm.OP_FORWARD, 8, 4, 64, 1, 65537), ssm.ERR_UNSUPPORTED),
    ((ssm.OP_DISCRETIZE, 1, 4, 5000, 1, 16), ssm.ERR_UNSUPPORTED),
    ((7, 1, 4, 64, 1, 16), ssm.ERR_INVALID_ARGUMENT),
])
def test_workspace_query_rejects(args, code):
    out = ctypes.c_size_t(123)
    assert ssm.lib.ssm_workspace_bytes(*args, ctypes.byref(out)) == code
    assert out.value == 123


FAKE = 0x10000000  # aligned dummy address: validation fails before any use


def _fwd(**kw):
    a = dict(Bsz=2, H=3, N=4, r=1, L=16, Lambda=FAKE, P=FAKE, Q=FAKE, B=FAKE, Ct=FAKE, dt=FAKE, D=None,
             u=FAKE, y=FAKE, K=None, status=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return ssm.lib.ssm_forward(a["Bsz"], a["H"], a["N"], a["r"], a["L"], a["Lambda"], a["P"], a["Q"], a["B"],
                               a["Ct"], a["dt"], a["D"], a["u"], a["y"], a["K"], a["status"], a["ws"],
                               a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), ssm.ERR_INVALID_ARGUMENT),
    (dict(L=0), ssm.ERR_INVALID_ARGUMENT),
    (dict(r=9), ssm.ERR_UNSUPPORTED),
    (dict(Lambda=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(u=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(Ct=FAKE + 4), ssm.ERR_INVALID_ARGUMENT),    # complex array not 8-byte aligned
    (dict(u=FAKE + 2), ssm.ERR_INVALID_ARGUMENT),     # float array not 4-byte aligned
    (dict(ws=FAKE + 64), ssm.ERR_INVALID_ARGUMENT),   # workspace not 256-byte aligned
    (dict(ws_bytes=16), ssm.ERR_WORKSPACE),
    (dict(ws=None), ssm.ERR_WORKSPACE),
])
def test_forward_rejects_before_launch(kw, code):
    assert _fwd(**kw) == code


def test_fftconv_and_kernel_gen_reject():
    lib = ssm.lib
    assert lib.ssm_fftconv(1, 1, 16, FAKE, 3, None, FAKE, FAKE, FAKE, 1 << 20, None) == ssm.ERR_INVALID_ARGUMENT
    assert lib.ssm_fftconv(1, 1, 16, FAKE, 1, None, FAKE, FAKE, FAKE, 8, None) == ssm.ERR_WORKSPACE
    assert lib.ssm_kernel_gen(1, 4, 1, 16, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE, 1 << 20,
                              None) == ssm.ERR_INVALID_ARGUMENT
    assert lib.ssm_discretize(1, 4, 1, 16, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, None, None, 0,
                              None) == ssm.ERR_INVALID_ARGUMENT


def test_forward_complex_workspace_and_rejects():
    H, L = 256, 1000
    # the forward workspace less its wave-structured transforms' table [2M] c64,
    # which the complex path does not use
    fwd = ssm.workspace_bytes(ssm.OP_FORWARD, 8, H, 64, 1, L) - 2 * 1024 * 8
    cpx = ssm.workspace_bytes(ssm.OP_FORWARD_COMPLEX, 8, H, 64, 1, L)
    assert cpx >= fwd + H * L * 8 and cpx % 256 == 0   # plus the complex kernel [H, L]
    # where the input's transforms are shared (here M = 1024) the imaginary
    # part's spectra [H, 2, M] live beside the real part's
    assert cpx >= fwd + H * L * 8 + H * 2 * 1024 * 8
    big = ssm.workspace_bytes(ssm.OP_FORWARD_COMPLEX, 8, H, 64, 1, 5000)
    assert big - (ssm.workspace_bytes(ssm.OP_FORWARD, 8, H, 64, 1, 5000) - 2 * 8192 * 8) < H * 2 * 8192 * 8

    def call(r=1, y_re=FAKE, y_im=FAKE, ws_bytes=1 << 30):
        return ssm.lib.ssm_forward_complex(2, 3, 4, r, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, y_re, y_im,
                                           None, None, FAKE, ws_bytes, None)

    assert call(y_im=None) == ssm.ERR_INVALID_ARGUMENT
    assert call(y_re=FAKE + 2) == ssm.ERR_INVALID_ARGUMENT
    assert call(ws_bytes=64) == ssm.ERR_WORKSPACE
    assert call(r=5) == ssm.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), ssm.ERR_INVALID_ARGUMENT),
    (dict(Bsz=0), ssm.ERR_INVALID_ARGUMENT),
    (dict(N=257), ssm.ERR_UNSUPPORTED),       # step mode holds at most 4 states per lane
    (dict(r=5), ssm.ERR_UNSUPPORTED),
    (dict(C=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(x=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(x=FAKE + 4), ssm.ERR_INVALID_ARGUMENT),    # state not 8-byte aligned
    (dict(u=FAKE + 2), ssm.ERR_INVALID_ARGUMENT),
    (dict(lanes=32), ssm.ERR_INVALID_ARGUMENT),            # layouts: 0 (chosen), 16 or 64
    (dict(lanes=16, N=65), ssm.ERR_INVALID_ARGUMENT),      # 16-lane groups hold at most 64 states
])
def test_step_rejects_before_launch(kw, code):
    a = dict(Bsz=2, H=3, N=4, r=1, T=16, Lambda=FAKE, P=FAKE, Q=FAKE, B=FAKE, C=FAKE, dt=FAKE, D=None, u=FAKE,
             y=FAKE, x=FAKE, status=None, lanes=0)
    a.update(kw)
    assert ssm.lib.ssm_step(a["Bsz"], a["H"], a["N"], a["r"], a["T"], a["Lambda"], a["P"], a["Q"], a["B"], a["C"],
                            a["dt"], a["D"], a["u"], a["y"], a["x"], a["status"], a["lanes"], None) == code


# --------------------------------------------------------------------------
# ssm_step_prepare / ssm_step_prepared: the constants' size and argument checks


@pytest.mark.parametrize("N,r,npl", [(1, 1, 1), (64, 1, 1), (65, 2, 2), (128, 4, 2), (129, 1, 4), (256, 4, 4)])
def test_step_prepared_bytes(N, r, npl):
    """Per channel: a 64-byte header, the order-8 inverse (64 complex64), then
    3 + 2r arrays of 64 npl complex64, rounded up to 256 bytes."""
    raw = 64 + 64 * 8 + (3 + 2 * r) * 64 * npl * 8
    per = -(-raw // 256) * 256
    for H in (1, 7):
        assert ssm.workspace_bytes(ssm.OP_STEP_PREPARED, 0, H, N, r, 0) == H * per


@pytest.mark.parametrize("args,code", [
    ((0, 4, 1), ssm.ERR_INVALID_ARGUMENT),
    ((3, 0, 1), ssm.ERR_INVALID_ARGUMENT),
    ((3, 4, 0), ssm.ERR_INVALID_ARGUMENT),
    ((3, 257, 1), ssm.ERR_UNSUPPORTED),
    ((3, 4, 5), ssm.ERR_UNSUPPORTED),
])
def test_step_prepared_bytes_rejects(args, code):
    H, N, r = args
    with pytest.raises(ssm.SSMError) as e:
        ssm.workspace_bytes(ssm.OP_STEP_PREPARED, 0, H, N, r, 0)
    assert e.value.code == code


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), ssm.ERR_INVALID_ARGUMENT),
    (dict(N=257), ssm.ERR_UNSUPPORTED),
    (dict(r=5), ssm.ERR_UNSUPPORTED),
    (dict(Q=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(prep=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(prep=FAKE + 64), ssm.ERR_INVALID_ARGUMENT),   # constants not 256-byte aligned
    (dict(dt=FAKE + 2), ssm.ERR_INVALID_ARGUMENT),
    (dict(prep_bytes=3 * 3328 - 1), ssm.ERR_WORKSPACE),  # 3 channels need 3 x 3328 bytes at N = 4, r = 1
])
def test_step_prepare_rejects_before_launch(kw, code):
    a = dict(H=3, N=4, r=1, Lambda=FAKE, P=FAKE, Q=FAKE, B=FAKE, C=FAKE, dt=FAKE, prep=FAKE, prep_bytes=1 << 20,
             status=None)
    a.update(kw)
    assert ssm.lib.ssm_step_prepare(a["H"], a["N"], a["r"], a["Lambda"], a["P"], a["Q"], a["B"], a["C"], a["dt"],
                                    a["prep"], a["prep_bytes"], a["status"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), ssm.ERR_INVALID_ARGUMENT),
    (dict(Bsz=0), ssm.ERR_INVALID_ARGUMENT),
    (dict(N=257), ssm.ERR_UNSUPPORTED),
    (dict(r=5), ssm.ERR_UNSUPPORTED),
    (dict(prep=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(prep=FAKE + 8), ssm.ERR_INVALID_ARGUMENT),
    (dict(x=FAKE + 4), ssm.ERR_INVALID_ARGUMENT),
    (dict(y=None), ssm.ERR_INVALID_ARGUMENT),
    (dict(prep_bytes=3327), ssm.ERR_WORKSPACE),
    (dict(lanes=32), ssm.ERR_INVALID_ARGUMENT),            # layouts: 0 (chosen), 16 or 64
    (dict(lanes=-1), ssm.ERR_INVALID_ARGUMENT),
    (dict(lanes=16, N=65), ssm.ERR_INVALID_ARGUMENT),      # 16-lane groups hold at most 64 states
])
def test_step_prepared_rejects_before_launch(kw, code):
    a = dict(Bsz=2, H=1, N=4, r=1, T=16, prep=FAKE, prep_bytes=1 << 20, D=None, u=FAKE, y=FAKE, x=FAKE,
             status=None, lanes=0)
    a.update(kw)
    assert ssm.lib.ssm_step_prepared(a["Bsz"], a["H"], a["N"], a["r"], a["T"], a["prep"], a["prep_bytes"], a["D"],
                                     a["u"], a["y"], a["x"], a["status"], a["lanes"], None) == code


# --------------------------------------------------------------------------
# ssm_hippo_dplr: sizes and argument checks (host only)
# --------------------------------------------------------------------------
def _hippo_ws(N):
    out = ctypes.c_size_t()
    rc = ssm.lib.ssm_workspace_bytes(ssm.OP_HIPPO, 0, 0, N, 0, 0, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("N", [1, 2, 64, 256, 1000, 1024])
def test_hippo_workspace_bytes(N):
    rc, nbytes = _hippo_ws(N)
    assert rc == ssm.OK
    # K and the reflections (float64 N x N each), the phase-fixed eigenvectors
    # (complex128 N x N), two float64 vectors; each region 256-byte aligned
    a = lambda v: (v + 255) // 256 * 256
    assert nbytes == a(8 * N * N) * 2 + a(8 * N) * 2 + a(16 * N * N)


def test_hippo_workspace_bytes_rejects():
    assert _hippo_ws(0)[0] == ssm.ERR_INVALID_ARGUMENT
    assert _hippo_ws(1025)[0] == ssm.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(kind=3), 1), (dict(kind=-1), 1), (dict(N=0), 1), (dict(nb=-1), 1), (dict(nc=-1), 1),
    (dict(kind=1, theta=0.0), 1), (dict(kind=1, theta=-2.0), 1), (dict(kind=1, theta=float("nan")), 1),
    (dict(kind=1, theta=float("inf")), 1),
    (dict(N=1025), 4),
    (dict(Lambda=None), 1), (dict(P=None), 1), (dict(ws=None), 1),
    (dict(nb=2, B=None), 1), (dict(nb=2, Bt=None), 1), (dict(nc=3, C=None), 1), (dict(nc=3, Ct=None), 1),
    (dict(Lambda=FAKE + 4), 1), (dict(ws=FAKE + 64), 1),
    (dict(ws_bytes=1000), 2),
])
def test_hippo_rejects_before_launch(kw, code):
    a = dict(kind=0, N=8, theta=1.0, nb=0, B=None, nc=0, C=None, Lambda=FAKE, P=FAKE, V=None, Bt=None, Ct=None,
             ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    assert ssm.lib.ssm_hippo_dplr(a["kind"], a["N"], a["theta"], a["nb"], a["B"], a["nc"], a["C"], a["Lambda"],
                                  a["P"], a["V"], a["Bt"], a["Ct"], a["ws"], a["ws_bytes"], None) == code
