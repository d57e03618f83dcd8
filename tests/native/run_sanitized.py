"""Child process of tests/test_sanitized_host.py: runs the host-half and oracle CPU tests
against the AddressSanitizer / UndefinedBehaviorSanitizer builds named by GDN_HOSTCHECK_LIB and
GDN_ORACLE_LIB (the sanitizer runtimes are preloaded by the parent), then checks that no ROCm
library was mapped into the process."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
FILES = ["test_abi_cpu.py", "test_state_files.py", "test_host_properties.py",
         "test_host_plan.py", "test_session_store.py", "test_oracle_pins.py",
         "test_oracle_mutations.py"]

if __name__ == "__main__":
    os.chdir(ROOT)
    files = [os.path.join("tests", f) for f in FILES if os.path.exists(os.path.join("tests", f))]
    rc = pytest.main(["-q", "-x", "--capture=sys", "-p", "no:cacheprovider", "-m", "not gpu", "-k",
                      "not hip_library"] + files)
    with open("/proc/self/maps") as f:
        maps = f.read()
    rocm = sorted({ln.split()[-1] for ln in maps.splitlines()
                   if "amdhip" in ln or "libhsa" in ln or "/opt/rocm" in ln})
    if rocm:
        print("ROCm libraries mapped:", rocm)
        rc = rc or 3
    print("sanitized run exit", int(rc), flush=True)
    sys.exit(int(rc))
