"""Host check (no GPU) of the storage order of the wave-structured transforms:
position -> frequency is a permutation for M = 1024..65536, complementing a
position complements its frequency, the compile-time and run-time maps agree,
and k = M/2 sits at position 512.  tests/wave_order_driver.hip holds the
checks; it includes the library's transform header and makes no GPU call."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_state_space_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def test_wave_order_is_a_complement_preserving_permutation(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "wave_order")
    p = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}",
                        f"-I{CSRC}", os.path.join(ROOT, "tests", "wave_order_driver.hip"), "-o", exe],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stdout + p.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout
