"""Host checks (no GPU) of bench.py's own logic: the one-GPU refusal, its
model of the wave-structured transforms' storage order against the library's,
the terms-summed model of the split-precision root values on limiting cases,
the algorithmic byte counts, and the reading of committed counter summaries."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from structured_state_space_amd import inputs as I  # noqa: E402

HIPCC = "/opt/rocm/bin/hipcc"


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_wave_freq_matches_the_library_order(tmp_path):
    """bench.wave_freq (used to count the terms the root-value kernel sums) is the
    library's position -> frequency map, at every transform length."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "wave_order")
    p = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}",
                        f"-I{os.path.join(ROOT, 'structured_state_space_amd', 'csrc')}",
                        os.path.join(ROOT, "tests", "wave_order_driver.hip"), "-o", exe],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stdout + p.stderr
    for logm in range(10, 17):
        r = subprocess.run([exe, "dump", str(logm)], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0
        lib = np.array(r.stdout.split(), dtype=np.int64)
        M = 1 << logm
        assert lib.shape == (M,)
        assert np.array_equal(bench.wave_freq(logm, np.arange(M)), lib), f"M = {M}"


def _params(H, N, M, dt, same_pole=False):
    p = I.random_params(11, H, N, 2, M)
    if same_pole:
        p.Lambda[:] = p.Lambda[:, :1]
    p.dt[:] = dt
    return p


def test_root_value_terms_limits():
    M, H, N = 4096, 3, 64
    roots = H * (M - 1)
    # one pole position: R = 0, no far form, every root sums the N states
    t, far = bench.root_value_terms(_params(H, N, M, 0.01, same_pole=True), M, True)
    assert (t, far) == (N * roots, 0.0)
    # moderate steps: some far waves, fewer terms than the direct sum, more than 8 per root
    t, far = bench.root_value_terms(_params(H, N, M, 0.01), M, True)
    assert 8 * roots < t < N * roots and 0.0 < far < 1.0
    # a tiny step puts every root but those near s = 0 far beyond 8 R: 8 terms per
    # root in every wave except those holding a root near k = 0 or k = M
    t, far = bench.root_value_terms(_params(H, N, M, 1e-7), M, True)
    assert far > 0.95 and t < 8 * roots + 8 * 64 * N * H
    # natural order: the same bound
    t2, far2 = bench.root_value_terms(_params(H, N, M, 1e-7), M, False)
    assert far2 > 0.95 and t2 < 8 * roots + 8 * 64 * N * H


def test_algorithmic_bytes_of_the_headline_workload():
    w = I.BY_NAME["s4-h1k-l16k"]
    alg = bench.algorithmic(w, 16384, False)
    # rows in and out (4 B each way per row and step), the stored half spectrum
    # (M complex per channel) once, D per channel
    assert alg["conv"]["work"] == 8 * 4 * 1024 * 16384 + 4 * 1024 * 16384 + 4 * 1024
    # the spectrum pass: the root values read and one M-point spectrum written per channel
    assert alg["spectrum"]["work"] == 2 * 8 * 1024 * 16384
    # the direct sum over the M - 1 roots != -1, 8 (r+1)^2 + 7 flops per (root, state)
    assert alg["cauchy"]["work"] == 1024 * 16383 * 64 * (8 * 9 + 7)


def test_read_traffic_needs_the_same_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "structured_state_space_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES["conv"]:
        (csrc / f).write_text(f"// {f}\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.source_hash("conv")
    prof = tmp_path / "profiles" / "conv_wl_hbm_counters.md"
    body = ("fetch_kib_per_dispatch: 100.0\nwrite_kib_per_dispatch: 50.0\ncopy_scale_fetch: 2.0\n"
            "copy_scale_write: 1.0\nsource_sha: {}\n")
    prof.write_text(body.format(sha))
    assert bench.read_traffic("conv", "wl") == pytest.approx((100.0 * 2.0 + 50.0) * 1024.0)
    assert bench.read_traffic("conv", "other") is None
    prof.write_text(body.format("0123456789abcdef"))
    assert bench.read_traffic("conv", "wl") is None
    # a changed source file invalidates a matching summary
    prof.write_text(body.format(sha))
    (csrc / bench.KERNEL_SOURCES["conv"][0]).write_text("// changed\n")
    assert bench.read_traffic("conv", "wl") is None
