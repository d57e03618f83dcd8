"""The library's host half on the CPU, for tests without a GPU and without ROCm.

Loads libgdn_hostcheck.so (built by tests/native/build_hostcheck.py, rebuilt when a source is
newer): csrc/gdn_host.cpp -- validation, grid arithmetic, checkpoint ring, state files, the
launch plan -- over a host-memory stand-in for the device half that records kernel launches
instead of running them.  GDN_HOSTCHECK_LIB names another build (the sanitizer build).  The
declarations are the product binding's (hybrid_linear_attention_prefill_amd.abi), so every call
goes through the same C signatures.
"""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from hybrid_linear_attention_prefill_amd import abi  # noqa: E402
from hybrid_linear_attention_prefill_amd.abi import *  # noqa: E402,F401,F403

sys.path.insert(0, os.path.join(HERE, "native"))
import build_hostcheck  # noqa: E402

_path = os.environ.get("GDN_HOSTCHECK_LIB")
if not _path:
    _path = build_hostcheck.lib_path()
    if build_hostcheck.stale(_path):
        build_hostcheck.build()
lib = abi.declare(ctypes.CDLL(_path), host_only=True)
lib.gdn_hostcheck_launches.restype = ctypes.c_int32
lib.gdn_hostcheck_launches.argtypes = []
lib.gdn_hostcheck_reset.restype = None
lib.gdn_hostcheck_reset.argtypes = []
lib.gdn_hostcheck_launch.restype = ctypes.c_int32
lib.gdn_hostcheck_launch.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_int64), ctypes.c_int32]
make_desc = abi.make_desc
GdnError = abi.GdnError
HEADER = os.path.join(ROOT, "include", "gdn.h")
_host = abi.HostCalls(lib)
check = _host.check
gdn_desc_check = _host.gdn_desc_check
gdn_desc_tag = _host.gdn_desc_tag
gdn_state_S_bytes = _host.gdn_state_S_bytes
gdn_state_conv_bytes = _host.gdn_state_conv_bytes
gdn_workspace_bytes = _host.gdn_workspace_bytes
gdn_state_file_header_bytes = _host.gdn_state_file_header_bytes
gdn_state_file_write = _host.gdn_state_file_write
gdn_state_file_read = _host.gdn_state_file_read
gdn_commit_rows = _host.gdn_commit_rows
gdn_shared_prefix_rows = _host.gdn_shared_prefix_rows
CkptRing = _host.CkptRing

KIND_PREFILL, KIND_DECODE, KIND_CONV, KIND_LINEAR, KIND_ATTENTION = 1, 2, 3, 4, 5
SEG_FIELDS = ("row0", "n", "sub0", "S_in", "win_in", "S_out", "win_out")


gdn_status_str = _host.gdn_status_str


def exported_names():
    return abi.declared_names(HEADER)


def launches():
    """Recorded kernel launches since the last reset: [(kind, rows, [seg dicts])]."""
    out = []
    for i in range(lib.gdn_hostcheck_launches()):
        rows, nseg = ctypes.c_int64(), ctypes.c_int32()
        buf = (ctypes.c_int64 * (7 * 32))()
        kind = lib.gdn_hostcheck_launch(i, ctypes.byref(rows), ctypes.byref(nseg), buf, 32)
        segs = [dict(zip(SEG_FIELDS, buf[7 * k:7 * k + 7])) for k in range(min(nseg.value, 32))]
        out.append((kind, rows.value, segs))
    return out


def reset():
    lib.gdn_hostcheck_reset()


class HostState:
    """A state whose S and window live in host memory (numpy), with its C struct in ``.c``;
    ``fill`` draws random contents."""

    def __init__(self, d, fill=False, seed=0):
        import numpy as np
        self.S = np.zeros((d.n_v_heads, d.d_k, d.d_v), dtype=np.float32)
        self.conv = (np.zeros((d.conv_width - 1, d.channels),
                              dtype=np.uint16 if d.act_dtype == GDN_BF16 else np.float32)
                     if d.conv_width else None)
        if fill:
            r = np.random.default_rng(seed)
            self.S[:] = r.standard_normal(self.S.shape)
            if self.conv is not None:
                self.conv.view(np.uint16)[:] = r.integers(0, 1 << 16, self.conv.view(np.uint16).shape)
        self.c = gdn_state(self.S.ctypes.data, None if self.conv is None else self.conv.ctypes.data,
                           0, gdn_desc_tag(d))

    @property
    def pos(self):
        return self.c.pos

    def ref(self):
        return ctypes.byref(self.c)
