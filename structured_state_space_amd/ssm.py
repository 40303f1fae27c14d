"""Python binding of the C ABI in include/ssm.h (argument marshalling only).

Every step of the filter path runs in the HIP library; this module only checks
tensor shapes and dtypes, allocates workspaces with torch, and passes device
pointers plus torch's current HIP stream.  Importing it loads the in-tree
library built by structured_state_space_amd/build.py and raises ImportError
when it is missing: there is no CPU fallback.

torch is imported first so that the library binds to the HIP runtime torch has
already loaded (both use the libamdhip64.so.7 soname).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libssm_hip.so")

# return codes and statuses, as declared in include/ssm.h
OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_WORKSPACE = 2
ERR_DEVICE = 3
ERR_UNSUPPORTED = 4
ERR_SCRATCH_LIMIT = 5
NOALLOC_SCRATCH_BYTES = 64 << 20
ST_OK = 0
ST_RESONANT_CORRECTION = 16
ST_RESONANT_DIAGONAL = 17
ST_SINGULAR_BILINEAR = 18
ST_INVALID_STEP = 19
ST_UNPREPARED = 20
OP_DISCRETIZE, OP_KERNEL_GEN, OP_FFTCONV, OP_FORWARD, OP_FORWARD_COMPLEX, OP_HIPPO = 0, 1, 2, 3, 4, 5
OP_STEP_PREPARED = 6
HIPPO_LEGS, HIPPO_LEGT, HIPPO_LAGT = 0, 1, 2
HIPPO_KINDS = {"legs": HIPPO_LEGS, "legt": HIPPO_LEGT, "lagt": HIPPO_LAGT}

EXPORTS = ("ssm_workspace_bytes", "ssm_transform_lengths", "ssm_forward_form", "ssm_status_string",
           "ssm_discretize", "ssm_kernel_gen", "ssm_fftconv", "ssm_forward", "ssm_forward_profiled", "ssm_step",
           "ssm_forward_complex", "ssm_hippo_dplr", "ssm_step_prepare", "ssm_step_prepared",
           "ssm_forward_noalloc")


class SSMError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {status_string(code)} (code {code})")
        self.code = code


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"HIP library not built: {_LIB_PATH} is missing "
                          "(run `python -c 'import __graft_entry__ as g; g.build()'`)")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, sz, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.ssm_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i64, ctypes.POINTER(sz)]
    lib.ssm_workspace_bytes.restype = i32
    lib.ssm_transform_lengths.argtypes = [i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.ssm_transform_lengths.restype = i32
    lib.ssm_forward_form.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_int32)]
    lib.ssm_forward_form.restype = i32
    lib.ssm_status_string.argtypes = [i32]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_discretize.argtypes = [i64, i64, i64, i64] + [vp] * 10 + [vp, sz, vp]
    lib.ssm_discretize.restype = i32
    lib.ssm_kernel_gen.argtypes = [i64, i64, i64, i64] + [vp] * 9 + [vp, sz, vp]
    lib.ssm_kernel_gen.restype = i32
    lib.ssm_fftconv.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.ssm_fftconv.restype = i32
    lib.ssm_forward.argtypes = [i64, i64, i64, i64, i64] + [vp] * 11 + [vp, sz, vp]
    lib.ssm_forward.restype = i32
    lib.ssm_forward_profiled.argtypes = [i64, i64, i64, i64, i64] + [vp] * 11 + [vp, sz, vp, vp, ctypes.c_int32]
    lib.ssm_forward_profiled.restype = i32
    lib.ssm_step.argtypes = [i64, i64, i64, i64, i64] + [vp] * 11 + [ctypes.c_int32, vp]
    lib.ssm_step.restype = i32
    lib.ssm_step_prepare.argtypes = [i64, i64, i64] + [vp] * 7 + [sz, vp, vp]
    lib.ssm_step_prepare.restype = i32
    lib.ssm_step_prepared.argtypes = [i64, i64, i64, i64, i64, vp, sz] + [vp] * 5 + [ctypes.c_int32, vp]
    lib.ssm_step_prepared.restype = i32
    lib.ssm_forward_complex.argtypes = [i64, i64, i64, i64, i64] + [vp] * 12 + [vp, sz, vp]
    lib.ssm_forward_complex.restype = i32
    lib.ssm_forward_noalloc.argtypes = [i64, i64, i64, i64, i64] + [vp] * 11 + [vp]
    lib.ssm_forward_noalloc.restype = i32
    lib.ssm_hippo_dplr.argtypes = [i32, i64, ctypes.c_double, i64, vp, i64, vp] + [vp] * 5 + [vp, sz, vp]
    lib.ssm_hippo_dplr.restype = i32
    return lib


lib = _load()


def status_string(code: int) -> str:
    return lib.ssm_status_string(int(code)).decode()


def transform_lengths(L: int):
    M, n = ctypes.c_int64(), ctypes.c_int64()
    rc = lib.ssm_transform_lengths(int(L), ctypes.byref(M), ctypes.byref(n))
    if rc != OK:
        raise SSMError("ssm_transform_lengths", rc)
    return M.value, n.value


def forward_form(Bsz: int, H: int, L: int) -> int:
    """ssm_forward_form: 1 (single launch), 2 (root values + convolution with
    spectra) or 3 (root values, spectra, convolution)."""
    out = ctypes.c_int32()
    rc = lib.ssm_forward_form(int(Bsz), int(H), int(L), ctypes.byref(out))
    if rc != OK:
        raise SSMError("ssm_forward_form", rc)
    return out.value


def workspace_bytes(op: int, Bsz: int, H: int, N: int, r: int, L: int) -> int:
    out = ctypes.c_size_t()
    rc = lib.ssm_workspace_bytes(int(op), int(Bsz), int(H), int(N), int(r), int(L), ctypes.byref(out))
    if rc != OK:
        raise SSMError("ssm_workspace_bytes", rc)
    return out.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        got = (None if not isinstance(t, torch.Tensor) else (t.dtype, tuple(t.shape)))
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {got}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name}: must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _params(Lambda, P, Q, B, Cv, dt):
    H, N = Lambda.shape
    r = P.shape[2]
    dev = Lambda.device
    _check(Lambda, "Lambda", torch.complex64, (H, N), dev)
    _check(P, "P", torch.complex64, (H, N, r), dev)
    _check(Q, "Q", torch.complex64, (H, N, r), dev)
    _check(B, "B", torch.complex64, (H, N), dev)
    _check(Cv, "C", torch.complex64, (H, N), dev)
    _check(dt, "dt", torch.float32, (H,), dev)
    return H, N, r, dev


def _workspace(nbytes, device, workspace=None):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def discretize(Lambda, P, Q, B, C, dt, L, want_bbar=True, want_abar=False, want_ctilde=True):
    """ssm_discretize: returns dict(Bbar, Abar, Ctilde, status) (None where not asked)."""
    H, N, r, dev = _params(Lambda, P, Q, B, C, dt)
    Bbar = torch.empty((H, N), dtype=torch.complex64, device=dev) if want_bbar else None
    Abar = torch.empty((H, N, N), dtype=torch.complex64, device=dev) if want_abar else None
    Ct = torch.empty((H, N), dtype=torch.complex64, device=dev) if want_ctilde else None
    status = torch.empty((H,), dtype=torch.int32, device=dev)
    rc = lib.ssm_discretize(H, N, r, int(L), _ptr(Lambda), _ptr(P), _ptr(Q), _ptr(B), _ptr(C), _ptr(dt),
                            _ptr(Bbar), _ptr(Abar), _ptr(Ct), _ptr(status), None, 0, _stream(dev))
    if rc != OK:
        raise SSMError("ssm_discretize", rc)
    return dict(Bbar=Bbar, Abar=Abar, Ctilde=Ct, status=status)


def kernel_gen(Lambda, P, Q, B, Ctilde, dt, L, want_kernel=True, want_roots=False, workspace=None):
    """ssm_kernel_gen: returns dict(K [H,L] c64, roots [H,M] c64, status [H] i32)."""
    H, N, r, dev = _params(Lambda, P, Q, B, Ctilde, dt)
    M, _ = transform_lengths(L)
    K = torch.empty((H, L), dtype=torch.complex64, device=dev) if want_kernel else None
    roots = torch.empty((H, M), dtype=torch.complex64, device=dev) if want_roots else None
    status = torch.empty((H,), dtype=torch.int32, device=dev)
    nbytes = workspace_bytes(OP_KERNEL_GEN, 1, H, N, r, L)
    ws = _workspace(nbytes, dev, workspace)
    rc = lib.ssm_kernel_gen(H, N, r, int(L), _ptr(Lambda), _ptr(P), _ptr(Q), _ptr(B), _ptr(Ctilde), _ptr(dt),
                            _ptr(K), _ptr(roots), _ptr(status), _ptr(ws), nbytes, _stream(dev))
    if rc != OK:
        raise SSMError("ssm_kernel_gen", rc)
    return dict(K=K, roots=roots, status=status)


def fftconv(K, u, D=None, y=None, workspace=None):
    """ssm_fftconv: y = K * u + D u.  K: float32 [H,L] or complex64 [H,L] (real part used)."""
    Bsz, H, L = u.shape
    dev = u.device
    _check(u, "u", torch.float32, (Bsz, H, L), dev)
    if K.dtype == torch.complex64:
        _check(K, "K", torch.complex64, (H, L), dev)
        stride = 2
    else:
        _check(K, "K", torch.float32, (H, L), dev)
        stride = 1
    _check(D, "D", torch.float32, (H,), dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", torch.float32, (Bsz, H, L), dev)
    nbytes = workspace_bytes(OP_FFTCONV, Bsz, H, 1, 1, L)
    ws = _workspace(nbytes, dev, workspace)
    rc = lib.ssm_fftconv(Bsz, H, L, _ptr(K), stride, _ptr(D), _ptr(u), _ptr(y), _ptr(ws), nbytes, _stream(dev))
    if rc != OK:
        raise SSMError("ssm_fftconv", rc)
    return y


def forward(Lambda, P, Q, B, Ctilde, dt, D, u, want_kernel=False, y=None, K_out=None, status=None,
            workspace=None, events=None, repeat=1):
    """ssm_forward: returns dict(y [Bsz,H,L] f32, K [H,L] c64 or None, status [H] i32).

    events: optional four torch.cuda.Event(enable_timing=True); then the call goes
    through ssm_forward_profiled, which launches each of its three stages
    `repeat` times and records the events around them."""
    H, N, r, dev = _params(Lambda, P, Q, B, Ctilde, dt)
    Bsz, H2, L = u.shape
    if H2 != H:
        raise ValueError("u: channel count does not match the parameters")
    _check(u, "u", torch.float32, (Bsz, H, L), dev)
    _check(D, "D", torch.float32, (H,), dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", torch.float32, (Bsz, H, L), dev)
    if K_out is None and want_kernel:
        K_out = torch.empty((H, L), dtype=torch.complex64, device=dev)
    _check(K_out, "K_out", torch.complex64, (H, L), dev)
    if status is None:
        status = torch.empty((H,), dtype=torch.int32, device=dev)
    _check(status, "status", torch.int32, (H,), dev)
    nbytes = workspace_bytes(OP_FORWARD, Bsz, H, N, r, L)
    ws = _workspace(nbytes, dev, workspace)
    args = (Bsz, H, N, r, L, _ptr(Lambda), _ptr(P), _ptr(Q), _ptr(B), _ptr(Ctilde), _ptr(dt), _ptr(D), _ptr(u),
            _ptr(y), _ptr(K_out), _ptr(status), _ptr(ws), nbytes, _stream(dev))
    if events is None:
        rc = lib.ssm_forward(*args)
        name = "ssm_forward"
    else:
        # torch creates its events lazily; record once so each has a handle
        for e in events:
            if e.cuda_event == 0:
                e.record()
        arr = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
        rc = lib.ssm_forward_profiled(*args, arr, int(repeat))
        name = "ssm_forward_profiled"
    if rc != OK:
        raise SSMError(name, rc)
    return dict(y=y, K=K_out, status=status)


def forward_noalloc(Lambda, P, Q, B, Ctilde, dt, D, u, y=None, K_out=None, status=None):
    """ssm_forward_noalloc: ssm_forward with the library's fixed per-GPU scratch
    instead of a workspace (the call allocates nothing when y, K_out and status
    are given).  Returns dict(y, K, status) as forward does."""
    H, N, r, dev = _params(Lambda, P, Q, B, Ctilde, dt)
    Bsz, H2, L = u.shape
    if H2 != H:
        raise ValueError("u: channel count does not match the parameters")
    _check(u, "u", torch.float32, (Bsz, H, L), dev)
    _check(D, "D", torch.float32, (H,), dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", torch.float32, (Bsz, H, L), dev)
    _check(K_out, "K_out", torch.complex64, (H, L), dev)
    if status is None:
        status = torch.empty((H,), dtype=torch.int32, device=dev)
    _check(status, "status", torch.int32, (H,), dev)
    rc = lib.ssm_forward_noalloc(Bsz, H, N, r, L, _ptr(Lambda), _ptr(P), _ptr(Q), _ptr(B), _ptr(Ctilde), _ptr(dt),
                                 _ptr(D), _ptr(u), _ptr(y), _ptr(K_out), _ptr(status), _stream(dev))
    if rc != OK:
        raise SSMError("ssm_forward_noalloc", rc)
    return dict(y=y, K=K_out, status=status)


def forward_complex(Lambda, P, Q, B, Ctilde, dt, D, u, want_kernel=False, workspace=None):
    """ssm_forward_complex: returns dict(y_re, y_im [Bsz,H,L] f32 (the real and
    imaginary parts of y), K [H,L] c64 or None, status [H] i32)."""
    H, N, r, dev = _params(Lambda, P, Q, B, Ctilde, dt)
    Bsz, H2, L = u.shape
    if H2 != H:
        raise ValueError("u: channel count does not match the parameters")
    _check(u, "u", torch.float32, (Bsz, H, L), dev)
    _check(D, "D", torch.float32, (H,), dev)
    y_re, y_im = torch.empty_like(u), torch.empty_like(u)
    K_out = torch.empty((H, L), dtype=torch.complex64, device=dev) if want_kernel else None
    status = torch.empty((H,), dtype=torch.int32, device=dev)
    nbytes = workspace_bytes(OP_FORWARD_COMPLEX, Bsz, H, N, r, L)
    ws = _workspace(nbytes, dev, workspace)
    rc = lib.ssm_forward_complex(Bsz, H, N, r, L, _ptr(Lambda), _ptr(P), _ptr(Q), _ptr(B), _ptr(Ctilde), _ptr(dt),
                                 _ptr(D), _ptr(u), _ptr(y_re), _ptr(y_im), _ptr(K_out), _ptr(status), _ptr(ws),
                                 nbytes, _stream(dev))
    if rc != OK:
        raise SSMError("ssm_forward_complex", rc)
    return dict(y_re=y_re, y_im=y_im, K=K_out, status=status)


def step(Lambda, P, Q, B, C, dt, D, u, x=None, y=None, status=None, lanes=0):
    """ssm_step: T steps of the recurrence from the state x (zeros when None);
    returns dict(y [Bsz,H,T] f32, x [Bsz,H,N] c64 (the state after the last
    step, updated in place when given), status [H] i32).  lanes: 64 (one
    sequence per wave), 16 (N <= 64: four per wave) or 0 (chosen per call)."""
    H, N, r, dev = _params(Lambda, P, Q, B, C, dt)
    Bsz, H2, T = u.shape
    if H2 != H:
        raise ValueError("u: channel count does not match the parameters")
    _check(u, "u", torch.float32, (Bsz, H, T), dev)
    _check(D, "D", torch.float32, (H,), dev)
    if x is None:
        x = torch.zeros((Bsz, H, N), dtype=torch.complex64, device=dev)
    _check(x, "x", torch.complex64, (Bsz, H, N), dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", torch.float32, (Bsz, H, T), dev)
    if status is None:
        status = torch.empty((H,), dtype=torch.int32, device=dev)
    _check(status, "status", torch.int32, (H,), dev)
    rc = lib.ssm_step(Bsz, H, N, r, T, _ptr(Lambda), _ptr(P), _ptr(Q), _ptr(B), _ptr(C), _ptr(dt), _ptr(D), _ptr(u),
                      _ptr(y), _ptr(x), _ptr(status), int(lanes), _stream(dev))
    if rc != OK:
        raise SSMError("ssm_step", rc)
    return dict(y=y, x=x, status=status)


def step_prepare(Lambda, P, Q, B, C, dt, prep=None, status=None):
    """ssm_step_prepare: the per-channel set-up of the step mode, once per
    parameter set.  Returns dict(prep (uint8 device buffer of the float32
    constants), status [H] i32, H, N, r), which step_prepared takes."""
    H, N, r, dev = _params(Lambda, P, Q, B, C, dt)
    nbytes = workspace_bytes(OP_STEP_PREPARED, 0, H, N, r, 0)
    if prep is None:
        prep = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    elif not (isinstance(prep, torch.Tensor) and prep.dtype == torch.uint8 and prep.is_cuda and prep.device == dev
              and prep.is_contiguous() and prep.numel() >= nbytes):
        raise ValueError(f"prep: expected a contiguous uint8 tensor of at least {nbytes} bytes on {dev}")
    if status is None:
        status = torch.empty((H,), dtype=torch.int32, device=dev)
    _check(status, "status", torch.int32, (H,), dev)
    rc = lib.ssm_step_prepare(H, N, r, _ptr(Lambda), _ptr(P), _ptr(Q), _ptr(B), _ptr(C), _ptr(dt), _ptr(prep),
                              prep.numel(), _ptr(status), _stream(dev))
    if rc != OK:
        raise SSMError("ssm_step_prepare", rc)
    return dict(prep=prep, status=status, H=H, N=N, r=r)


def step_prepared(prepared, D, u, x=None, y=None, status=None, lanes=0):
    """ssm_step_prepared: T steps of the recurrence from the state x (zeros
    when None) with the constants of step_prepare's result `prepared`;
    returns dict(y, x, status) as step does, bit for bit in the same layout.
    lanes: 64, 16 (N <= 64) or 0 (chosen by the library per call)."""
    prep, H, N, r = prepared["prep"], prepared["H"], prepared["N"], prepared["r"]
    dev = prep.device
    Bsz, H2, T = u.shape
    if H2 != H:
        raise ValueError("u: channel count does not match the prepared constants")
    _check(u, "u", torch.float32, (Bsz, H, T), dev)
    _check(D, "D", torch.float32, (H,), dev)
    if x is None:
        x = torch.zeros((Bsz, H, N), dtype=torch.complex64, device=dev)
    _check(x, "x", torch.complex64, (Bsz, H, N), dev)
    if y is None:
        y = torch.empty_like(u)
    _check(y, "y", torch.float32, (Bsz, H, T), dev)
    if status is None:
        status = torch.empty((H,), dtype=torch.int32, device=dev)
    _check(status, "status", torch.int32, (H,), dev)
    rc = lib.ssm_step_prepared(Bsz, H, N, r, T, _ptr(prep), prep.numel(), _ptr(D), _ptr(u), _ptr(y), _ptr(x),
                               _ptr(status), int(lanes), _stream(dev))
    if rc != OK:
        raise SSMError("ssm_step_prepared", rc)
    return dict(y=y, x=x, status=status)


def hippo_dplr(kind, N, theta=1.0, B=None, C=None, want_v=False, device="cuda:0", workspace=None):
    """ssm_hippo_dplr: DPLR parameters of a HiPPO generator.  kind is "legs",
    "legt" or "lagt" (or its SSM_HIPPO_* code); B [nb,N] and C [nc,N] are
    complex64 device tensors or None.  Returns dict(Lambda [N], P [N,rank],
    V [N,N] or None, Bt [nb,N] or None, Ct [nc,N] or None), all complex64."""
    code = HIPPO_KINDS[kind] if isinstance(kind, str) else int(kind)
    dev = torch.device(device)
    if B is not None:
        dev = B.device
        _check(B, "B", torch.complex64, (B.shape[0], N), dev)
    if C is not None:
        dev = C.device if B is None else dev
        _check(C, "C", torch.complex64, (C.shape[0], N), dev)
    rank = 2 if code == HIPPO_LEGT else 1
    Lam = torch.empty((N,), dtype=torch.complex64, device=dev)
    P = torch.empty((N, rank), dtype=torch.complex64, device=dev)
    V = torch.empty((N, N), dtype=torch.complex64, device=dev) if want_v else None
    nb = 0 if B is None else B.shape[0]
    nc = 0 if C is None else C.shape[0]
    Bt = torch.empty_like(B) if B is not None else None
    Ct = torch.empty_like(C) if C is not None else None
    nbytes = workspace_bytes(OP_HIPPO, 0, 0, N, 0, 0)
    ws = _workspace(nbytes, dev, workspace)
    rc = lib.ssm_hippo_dplr(code, N, float(theta), nb, _ptr(B), nc, _ptr(C), _ptr(Lam), _ptr(P), _ptr(V), _ptr(Bt),
                            _ptr(Ct), _ptr(ws), nbytes, _stream(dev))
    if rc != OK:
        raise SSMError("ssm_hippo_dplr", rc)
    return dict(Lambda=Lam, P=P, V=V, Bt=Bt, Ct=Ct)


def to_device(params, device="cuda:0"):
    """Move an inputs.Params (numpy) to torch device tensors (a plain copy)."""
    f = lambda a: torch.from_numpy(a).to(device)
    return dict(Lambda=f(params.Lambda), P=f(params.P), Q=f(params.Q), B=f(params.B), C=f(params.C),
                dt=f(params.dt), D=f(params.D))
