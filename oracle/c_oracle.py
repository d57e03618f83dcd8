"""ctypes wrapper of the C float64 oracle (``gdn_oracle.c`` -> ``liboracle.so``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  ``build()`` compiles the C file with
gcc -O2 (no fast-math, so the float64 arithmetic is plain IEEE); ``load()`` builds on demand.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


class OracleDesc(ctypes.Structure):
    _fields_ = [("n_k_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("conv_silu", ctypes.c_int32),
                ("scale", ctypes.c_double), ("l2_eps", ctypes.c_double)]


SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build(sanitize=False, out=None):
    """Compile liboracle.so from gdn_oracle.c (always recompiles).  With ``sanitize`` the
    library is built with AddressSanitizer and UndefinedBehaviorSanitizer (for a process that
    preloads their runtimes) at ``out``."""
    out = out or _LIB
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                           "-shared", "-pthread"] + (SANITIZE if sanitize else []) +
                          ["-o", tmp, _SRC, "-lm"])
    os.replace(tmp, out)
    return out


def load():
    """The built library; GDN_ORACLE_LIB names another build of the same source (the
    sanitizer build of the CPU test run)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("GDN_ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(ctypes.c_double)
    lib.oracle_gdn_layer.argtypes = [ctypes.POINTER(OracleDesc), ctypes.c_int64, P, P, P, P, P, P,
                                     P, P, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                     ctypes.c_int32]
    lib.oracle_gdn_layer.restype = ctypes.c_int32
    lib.oracle_causal_conv.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P,
                                       ctypes.c_int32, P, P]
    lib.oracle_causal_conv.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def gdn_layer(x, conv_w, window, g, beta, S0, *, n_k_heads, n_v_heads, d_k, d_v, scale,
              l2_eps, conv_silu=False, heads=None, threads=None, want_o=True):
    """Run the oracle layer.  Returns (o [T,Hv,dv] or None, S [Hv,dk,dv], window_out or None).

    Only the value heads in ``heads`` (default all) are computed; other heads' outputs are
    zero and their states are S0.  ``conv_w`` None means the inputs are already post-conv.
    """
    lib = load()
    x = _f64(x)
    T, C = x.shape
    W = 0 if conv_w is None else int(np.asarray(conv_w).shape[1])
    d = OracleDesc(n_k_heads, n_v_heads, d_k, d_v, W, 1 if conv_silu else 0, scale, l2_eps)
    S = np.array(S0, dtype=np.float64, copy=True, order="C").reshape(n_v_heads, d_k, d_v)
    o = np.zeros((T, n_v_heads, d_v)) if want_o else None
    win_out = np.zeros((W - 1, C)) if W > 0 else None
    cw = _f64(conv_w)
    win = _f64(window) if W > 0 else None
    if W > 0 and win is None:
        win = np.zeros((W - 1, C))
    g = _f64(g)
    beta = _f64(beta)
    if heads is None:
        hp, nh = None, n_v_heads
    else:
        harr = np.ascontiguousarray(heads, dtype=np.int32)
        hp, nh = harr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(harr)
    if threads is None:
        threads = max(1, min(os.cpu_count() or 1, 16))
    rc = lib.oracle_gdn_layer(ctypes.byref(d), T, _p(x), _p(cw), _p(win), _p(g), _p(beta),
                              _p(S), _p(o), _p(win_out), hp, nh, threads)
    if rc != 0:
        raise RuntimeError("oracle_gdn_layer failed: %d" % rc)
    return o, S, win_out


def causal_conv(x, w, window, silu=False):
    lib = load()
    x = _f64(x)
    w = _f64(w)
    T, C = x.shape
    W = w.shape[1]
    window = _f64(window)
    y = np.zeros((T, C))
    wo = np.zeros((W - 1, C))
    lib.oracle_causal_conv(T, C, W, _p(x), _p(w), _p(window), 1 if silu else 0, _p(y), _p(wo))
    return y, wo
