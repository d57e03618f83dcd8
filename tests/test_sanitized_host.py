"""The host half and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-only library (csrc/gdn_host.cpp over the recording stand-in of the device half)
and the C oracle with -fsanitize=address,undefined, then runs their CPU tests in a child
process that preloads the sanitizer runtimes and loads no ROCm library.  Any sanitizer report
aborts the child (UBSan halts on the first error; ASan aborts on its first).
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "native"))


def _runtime(name):
    p = subprocess.check_output(["g++", "-print-file-name=" + name], text=True).strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(900)
def test_host_half_and_oracle_under_sanitizers(tmp_path):
    import build_hostcheck
    sys.path.insert(0, ROOT)
    from oracle import c_oracle
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    host = build_hostcheck.build(sanitize=True)
    orc = c_oracle.build(sanitize=True, out=str(tmp_path / "liboracle_sanitize.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan + ":" + ubsan, GDN_HOSTCHECK_LIB=host, GDN_ORACLE_LIB=orc,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, os.path.join(HERE, "native", "run_sanitized.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=880)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "sanitized run exit 0" in r.stdout, tail
