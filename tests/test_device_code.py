"""Properties of the built gfx950 device code (disassembled on the CPU).

The kernels are compiled with the packed-fp32 target feature switched off, so the code object
must hold no packed fp32 add, multiply or fused multiply-add: the compiler would otherwise pack
ordinary float arithmetic into them.  This test disassembles the device code of every object
the build produced (llvm-objdump from the ROCm toolchain) and counts them.
"""
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "hybrid_linear_attention_prefill_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def _objects():
    return sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))


@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "llvm-objdump")), reason="no ROCm llvm")
def test_no_packed_fp32_instructions_in_device_code(tmp_path):
    objs = _objects()
    assert objs, "build the library first (python -m hybrid_linear_attention_prefill_amd.build)"
    kernels = 0
    for obj in objs:
        # llvm-objdump --offloading writes the embedded device code objects beside its input
        local = str(tmp_path / os.path.basename(obj))
        with open(obj, "rb") as f, open(local, "wb") as g:
            g.write(f.read())
        subprocess.check_call([os.path.join(LLVM, "llvm-objdump"), "--offloading", local],
                              stdout=subprocess.DEVNULL)
        cos = glob.glob(local + ".*gfx950*")
        assert len(cos) == 1, cos
        asm = subprocess.check_output([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950",
                                       cos[0]], text=True)
        kernels += len(re.findall(r"^[0-9a-f]+ <_Z\w+>:", asm, re.M))
        hits = [ln.strip() for ln in asm.splitlines() if PACKED_F32.search(ln)]
        assert not hits, "%s: %d packed fp32 instructions, e.g. %s" % (obj, len(hits), hits[:3])
    assert kernels > 10
