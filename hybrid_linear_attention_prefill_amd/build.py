"""Build libgdn_prefill.so in-tree with hipcc for gfx950.

    python -m hybrid_linear_attention_prefill_amd.build

Compiles csrc/gdn_host.cpp (validation, scheduling, launches), csrc/gdn_store.cpp (the session
store), csrc/gdn_kernels.hip (the
layer's kernels), csrc/gdn_linear.hip (the projection GEMM) and csrc/gdn_attention.hip (the
full-attention layers) into libgdn_prefill.so beside this file.  Always recompiles.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdn_prefill.so")
SOURCES = [os.path.join(PKG, "csrc", "gdn_host.cpp"), os.path.join(PKG, "csrc", "gdn_store.cpp"),
           os.path.join(PKG, "csrc", "gdn_kernels.hip"),
           os.path.join(PKG, "csrc", "gdn_linear.hip"), os.path.join(PKG, "csrc", "gdn_attention.hip"),
           os.path.join(PKG, "csrc", "gdn_noalloc.hip")]
ARCH = "gfx950"

# Packed fp32 arithmetic is switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # keep MFMA accumulators in ordinary VGPRs (fewer accumulator-register moves)
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose=False):
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [hipcc(), "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
               "-ffp-contract=fast", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
               "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        if r.returncode != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError("hipcc failed on " + src)
        if verbose and msgs:
            print("\n".join(msgs))
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
