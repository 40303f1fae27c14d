"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU
needed).  The C-ABI layer (argument checks, size rules, workspace layout,
status strings) is compiled host-only with both sanitizers and linked with the
library's other objects; tests/sanitizer_driver.c then calls every entry point
on the paths that return before any device work and checks each return code.
Any sanitizer report fails the run."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_state_space_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout}\n{p.stderr}"
    return p


def test_abi_host_code_under_sanitizers(tmp_path):
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in sorted(os.listdir(CSRC))
            if f.endswith(".hip") and f != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built")
    for tool in (HIPCC, CLANG, CLANGXX):
        if not os.path.exists(tool):
            pytest.skip(f"{tool} not available")
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "driver.o", "driver"))
    # the ABI layer (no kernels; its one device variable, the no-allocation
    # scratch, is built as usual): both sanitizers on the host side only
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-fno-omit-frame-pointer",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *inc,
          "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", *inc, "-c",
          os.path.join(ROOT, "tests", "sanitizer_driver.c"), "-o", drv_o])
    _run([CLANGXX, "-fsanitize=address,undefined", drv_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr
    assert p.stdout.startswith("ok "), p.stdout
