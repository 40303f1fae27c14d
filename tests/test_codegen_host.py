"""Host-side check of the built library's gfx950 machine code (no GPU needed):
every HIP source is compiled with packed-FP32 code generation switched off, so
no packed single-precision add, multiply or fused multiply-add may appear in
the device code.  The code objects are read out of the library's own offload
bundles (one per compiled source) and disassembled with ROCm's llvm-objdump."""
import os
import re
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "structured_state_space_amd", "_lib", "libssm_hip.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _gfx950_objects(data):
    """Code objects of the gfx950 entries of every offload bundle in `data`."""
    objs, pos = [], data.find(MAGIC)
    while pos >= 0:
        (n,) = struct.unpack_from("<Q", data, pos + len(MAGIC))
        off = pos + len(MAGIC) + 8
        for _ in range(n):
            eoff, esize, idlen = struct.unpack_from("<QQQ", data, off)
            off += 24
            target = data[off:off + idlen].decode()
            off += idlen
            if target.endswith("gfx950") and esize > 0:
                objs.append(data[pos + eoff:pos + eoff + esize])
        pos = data.find(MAGIC, pos + 1)
    return objs


@pytest.fixture(scope="module")
def disassembly():
    if not os.path.exists(LIB):
        pytest.skip("HIP library not built")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not available")
    objs = _gfx950_objects(open(LIB, "rb").read())
    text = []
    with tempfile.TemporaryDirectory() as d:
        for i, o in enumerate(objs):
            p = os.path.join(d, f"co{i}.elf")
            with open(p, "wb") as f:
                f.write(o)
            r = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", p], capture_output=True, text=True, check=True)
            text.append(r.stdout)
    return objs, "\n".join(text)


def test_every_source_has_a_gfx950_code_object(disassembly):
    objs, _ = disassembly
    csrc = os.path.join(ROOT, "structured_state_space_amd", "csrc")
    # a source has device code if it defines a kernel or a file-scope device
    # variable (the no-allocation scratch array)
    def has_device_code(text):
        return "__global__" in text or re.search(r"^static __device__ ", text, re.M) is not None

    with_device_code = [f for f in os.listdir(csrc)
                        if f.endswith(".hip") and has_device_code(open(os.path.join(csrc, f)).read())]
    assert len(objs) == len(with_device_code)
    assert all(o[:4] == b"\x7fELF" for o in objs)


def test_no_packed_fp32_arithmetic(disassembly):
    _, text = disassembly
    assert "v_mfma_f32_4x4x1" in text          # the disassembly is real (the root-value sweep)
    found = sorted(set(re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", text)))
    assert not found, f"packed FP32 instructions in the device code: {found}"
