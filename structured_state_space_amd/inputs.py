"""Seeded synthetic workloads for the S4 DPLR filter path.

This module only draws numbers: it holds none of the method's arithmetic and
imports nothing from the HIP binding or from the CPU oracle.  Both sides of a
parity check consume the arrays it returns (complex64 / float32, already
rounded), so the oracle upcasts exactly the values the device sees.

Workloads (one per named configuration):

  name          H     N   r      L   Bsz  step size dt
  s4-tiny       1     8   1     64     1  0.01
  s4-h256-l1k 256    64   1   1024     8  log-uniform [1e-3, 1e-1]
  s4-h512-l3k 512    64   1   3000    16  0.01
  s4-h1k-l16k 1024   64   2  16384     4  log-uniform [1e-3, 1e-1]
  s4-h256-l64k 256  256   1  65536     2  log-uniform [1e-4, 1e-2]

Common recipe: lambda_n = -0.5 + i*pi*n (n < N), shared by all channels;
P, Q complex normal of shape [N, r] scaled by 1/sqrt(N), shared; B = 1;
C complex normal [H, N]; D ~ N(0, 1) per channel; u ~ N(0, 1) float32.
"Complex normal" is (X + iY)/sqrt(2) with X, Y iid N(0, 1).  Seed: the
workload's index in the table above (0-based) feeds numpy's PCG64.  Draw
order: P.re, P.im, Q.re, Q.im, C.re, C.im, dt (only when drawn), D, u.
Shared parameters are broadcast to per-channel arrays, which is the layout
the C ABI takes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    H: int
    N: int
    r: int
    L: int
    Bsz: int
    dt_fixed: Optional[float] = None
    dt_range: Optional[tuple] = None


WORKLOADS = (
    Workload("s4-tiny", 0, 1, 8, 1, 64, 1, dt_fixed=0.01),
    Workload("s4-h256-l1k", 1, 256, 64, 1, 1024, 8, dt_range=(1e-3, 1e-1)),
    Workload("s4-h512-l3k", 2, 512, 64, 1, 3000, 16, dt_fixed=0.01),
    Workload("s4-h1k-l16k", 3, 1024, 64, 2, 16384, 4, dt_range=(1e-3, 1e-1)),
    Workload("s4-h256-l64k", 4, 256, 256, 1, 65536, 2, dt_range=(1e-4, 1e-2)),
)

BY_NAME = {w.name: w for w in WORKLOADS}


@dataclass
class Params:
    """Per-channel DPLR parameters in the ABI's layout (row-major)."""
    Lambda: np.ndarray   # [H, N] complex64
    P: np.ndarray        # [H, N, r] complex64
    Q: np.ndarray        # [H, N, r] complex64
    B: np.ndarray        # [H, N] complex64
    C: np.ndarray        # [H, N] complex64 (conventional output vector)
    dt: np.ndarray       # [H] float32
    D: np.ndarray        # [H] float32
    L: int
    extra: dict = field(default_factory=dict)

    @property
    def H(self):
        return self.Lambda.shape[0]

    @property
    def N(self):
        return self.Lambda.shape[1]

    @property
    def r(self):
        return self.P.shape[2]

    def channel(self, h):
        return dict(Lambda=self.Lambda[h], P=self.P[h], Q=self.Q[h], B=self.B[h],
                    C=self.C[h], dt=float(self.dt[h]), D=float(self.D[h]))

    def select(self, chans):
        chans = np.asarray(chans)
        return Params(self.Lambda[chans], self.P[chans], self.Q[chans], self.B[chans],
                      self.C[chans], self.dt[chans], self.D[chans], self.L, dict(self.extra))


def _cnormal(rng, shape):
    re = rng.standard_normal(shape)
    im = rng.standard_normal(shape)
    return (re + 1j * im) / np.sqrt(2.0)


def make_params(w: Workload) -> tuple:
    """Return (Params, rng) with the rng positioned just before the draw of u."""
    rng = np.random.default_rng(w.seed)
    H, N, r = w.H, w.N, w.r
    lam = (-0.5 + 1j * np.pi * np.arange(N)).astype(np.complex64)
    P = (_cnormal(rng, (N, r)) / np.sqrt(N)).astype(np.complex64)
    Q = (_cnormal(rng, (N, r)) / np.sqrt(N)).astype(np.complex64)
    C = _cnormal(rng, (H, N)).astype(np.complex64)
    if w.dt_fixed is not None:
        dt = np.full(H, w.dt_fixed, dtype=np.float32)
    else:
        lo, hi = w.dt_range
        dt = np.exp(rng.uniform(np.log(lo), np.log(hi), H)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    params = Params(
        Lambda=np.array(np.broadcast_to(lam, (H, N)), order="C"),
        P=np.array(np.broadcast_to(P, (H, N, r)), order="C"),
        Q=np.array(np.broadcast_to(Q, (H, N, r)), order="C"),
        B=np.ones((H, N), dtype=np.complex64),
        C=C, dt=dt, D=D, L=w.L)
    return params, rng


def make_input(w: Workload, rng, batch: Optional[int] = None) -> np.ndarray:
    """u ~ N(0,1) float32 of shape [Bsz, H, L], drawn after the parameters."""
    b = w.Bsz if batch is None else batch
    return rng.standard_normal((b, w.H, w.L), dtype=np.float32)


def workload(name_or_index) -> tuple:
    """(Workload, Params, u) for a named workload or its 0-based index."""
    w = WORKLOADS[name_or_index] if isinstance(name_or_index, int) else BY_NAME[name_or_index]
    params, rng = make_params(w)
    u = make_input(w, rng)
    return w, params, u


def random_params(seed: int, H: int, N: int, r: int, L: int, dt_range=(1e-3, 1e-1),
                  lambda_kind: str = "s4") -> Params:
    """Generic seeded DPLR draw for edge-case tests (any H, N, r, L).

    lambda_kind "s4": lambda_n = -0.5 + i*pi*n; "random": Re in [-1, -0.1],
    Im ~ N(0, N) (unordered, exercises arbitrary poles).
    """
    rng = np.random.default_rng(seed)
    if lambda_kind == "s4":
        lam = np.broadcast_to(-0.5 + 1j * np.pi * np.arange(N), (H, N))
    else:
        lam = -rng.uniform(0.1, 1.0, (H, N)) + 1j * rng.normal(0.0, N, (H, N))
    P = _cnormal(rng, (H, N, r)) / np.sqrt(N)
    Q = _cnormal(rng, (H, N, r)) / np.sqrt(N)
    B = _cnormal(rng, (H, N))
    C = _cnormal(rng, (H, N))
    lo, hi = dt_range
    dt = np.exp(rng.uniform(np.log(lo), np.log(hi), H))
    D = rng.standard_normal(H)
    return Params(np.array(lam, dtype=np.complex64, order="C"), P.astype(np.complex64),
                  Q.astype(np.complex64), B.astype(np.complex64), C.astype(np.complex64),
                  dt.astype(np.float32), D.astype(np.float32), L)


def random_input(seed: int, Bsz: int, H: int, L: int) -> np.ndarray:
    rng = np.random.default_rng(seed + 1_000_003)
    return rng.standard_normal((Bsz, H, L), dtype=np.float32)


def cumsum_model(L: int) -> Params:
    """The scalar example A = 0, B = C = 1, dt = 1, D = 0 (one channel, N = r = 1)."""
    z = np.zeros((1, 1), dtype=np.complex64)
    return Params(Lambda=z.copy(), P=np.zeros((1, 1, 1), np.complex64),
                  Q=np.zeros((1, 1, 1), np.complex64), B=np.ones((1, 1), np.complex64),
                  C=np.ones((1, 1), np.complex64), dt=np.ones(1, np.float32),
                  D=np.zeros(1, np.float32), L=L)
