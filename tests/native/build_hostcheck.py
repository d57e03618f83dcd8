"""Build libgdn_hostcheck.so: the library's host half (csrc/gdn_host.cpp and csrc/gdn_store.cpp,
unchanged) linked
with the host-memory stand-in for its device half (gdn_backend_host.cpp), with g++ and no ROCm.

    python tests/native/build_hostcheck.py [--sanitize]

The plain build goes to tests/_build/libgdn_hostcheck.so; --sanitize builds it with
AddressSanitizer and UndefinedBehaviorSanitizer into tests/_build/sanitize/ (loaded by a
process that preloads their runtimes).  Always recompiles.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT_DIR = os.path.join(ROOT, "tests", "_build")
SOURCES = [os.path.join(ROOT, "hybrid_linear_attention_prefill_amd", "csrc", "gdn_host.cpp"),
           os.path.join(ROOT, "hybrid_linear_attention_prefill_amd", "csrc", "gdn_store.cpp"),
           os.path.join(HERE, "gdn_backend_host.cpp")]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def lib_path(sanitize=False):
    return os.path.join(OUT_DIR, "sanitize" if sanitize else "", "libgdn_hostcheck.so")


def build(sanitize=False):
    out = lib_path(sanitize)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["g++", "-std=c++17", "-O1" if sanitize else "-O2", "-fPIC", "-shared", "-Wall",
           "-Wextra", "-I", os.path.join(ROOT, "include")] + (SANITIZE if sanitize else []) + \
          ["-o", tmp] + SOURCES
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def stale(path):
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    deps = SOURCES + [os.path.join(ROOT, "include", "gdn.h"),
                      os.path.join(ROOT, "hybrid_linear_attention_prefill_amd", "csrc",
                                   "gdn_internal.h")]
    return any(os.path.getmtime(s) > t for s in deps)


if __name__ == "__main__":
    print(build(sanitize="--sanitize" in sys.argv))
