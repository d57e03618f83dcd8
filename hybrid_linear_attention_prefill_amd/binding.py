"""Thin ctypes binding of libgdn_prefill.so (the C ABI in include/gdn.h).

Argument marshalling only: every function here converts torch tensors and Python values to
the C types, calls the function of the same name and raises :class:`GdnError` on a negative
status.  All compute runs in the library's HIP kernels on the caller's (torch current)
stream.  Importing this module raises if the library has not been built; there is no
fallback.
"""
import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn_prefill.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "gdn.h")

GDN_OK, GDN_EINVAL, GDN_ESHAPE, GDN_EGRID = 0, -1, -2, -3
GDN_EMISMATCH, GDN_EWORKSPACE, GDN_EDEVICE, GDN_EALIAS, GDN_EFILE = -4, -5, -6, -7, -8
GDN_F32, GDN_BF16 = 0, 1
GDN_COMMIT, GDN_FORK = 0, 1
SUB_CHUNK = 64
MAX_CHECKPOINTS = 6

_DTYPE_CODE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}
_CODE_DTYPE = {GDN_F32: torch.float32, GDN_BF16: torch.bfloat16}


class GdnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, gdn_status_str(status), status))


class gdn_desc(ctypes.Structure):
    _fields_ = [("n_k_heads", ctypes.c_int32), ("n_v_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("sub_chunk", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("conv_silu", ctypes.c_int32),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float)]

    @property
    def channels(self):
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v

    @property
    def act_torch(self):
        return _CODE_DTYPE[self.act_dtype]

    @property
    def out_torch(self):
        return _CODE_DTYPE[self.out_dtype]


class gdn_state(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("conv", ctypes.c_void_p), ("pos", ctypes.c_int64),
                ("tag", ctypes.c_uint64)]


class gdn_attn_desc(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]

    @property
    def out_torch(self):
        return _CODE_DTYPE[self.out_dtype]


class gdn_attn_seq(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("pos0", ctypes.c_int64), ("T", ctypes.c_int64)]


class gdn_ckpt_ring(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int32), ("n", ctypes.c_int32),
                ("pos", ctypes.c_int64 * MAX_CHECKPOINTS),
                ("age", ctypes.c_uint64 * MAX_CHECKPOINTS), ("clock", ctypes.c_uint64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libgdn_prefill.so is not built: run "
                          "python -m hybrid_linear_attention_prefill_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    D, S, V, I32, I64, SZ = (ctypes.POINTER(gdn_desc), ctypes.POINTER(gdn_state), ctypes.c_void_p,
                            ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t)
    R = ctypes.POINTER(gdn_ckpt_ring)
    sig = {
        "gdn_desc_check": (I32, [D]),
        "gdn_desc_tag": (ctypes.c_uint64, [D]),
        "gdn_state_S_bytes": (SZ, [D]),
        "gdn_state_conv_bytes": (SZ, [D]),
        "gdn_workspace_bytes": (SZ, [D, I64, I32]),
        "gdn_state_init": (I32, [D, S, V]),
        "gdn_state_capture": (I32, [D, S, S, V]),
        "gdn_state_restore": (I32, [D, S, S, V]),
        "gdn_state_fork": (I32, [D, S, S, I32, V]),
        "conv1d_state_step": (I32, [D, V, V, V, V, I64, V]),
        "gdn_prefill_chunked": (I32, [D, V, V, V, V, S, S, V, I64, I32,
                                      ctypes.POINTER(ctypes.c_int64), V, SZ, V]),
        "gdn_prefill_chunked_events": (I32, [D, V, V, V, V, S, S, V, I64, I32,
                                             ctypes.POINTER(ctypes.c_int64), V, SZ, V,
                                             ctypes.POINTER(ctypes.c_void_p), I32]),
        "gdn_prefill_branches": (I32, [D, I32, ctypes.POINTER(ctypes.c_int64), V, V, V, V,
                                       ctypes.POINTER(S), ctypes.POINTER(S), V, V, SZ, V]),
        "gdn_decode_step": (I32, [D, I32, V, V, V, V, ctypes.POINTER(S), ctypes.POINTER(S), V, V]),
        "gdn_state_file_header_bytes": (SZ, []),
        "gdn_state_file_write": (I32, [D, V, V, I64, ctypes.c_uint64, ctypes.c_char_p]),
        "gdn_state_file_read": (I32, [D, V, V, ctypes.POINTER(ctypes.c_int64), ctypes.c_uint64,
                                      ctypes.c_char_p]),
        "gdn_state_save": (I32, [D, S, ctypes.c_uint64, ctypes.c_char_p, V]),
        "gdn_state_load": (I32, [D, S, ctypes.c_uint64, ctypes.c_char_p, V]),
        "gdn_linear": (I32, [I64, I32, I32, V, V, V, I32, V]),
        "gdn_attention_prefill": (I32, [ctypes.POINTER(gdn_attn_desc), I32,
                                        ctypes.POINTER(gdn_attn_seq), V]),
        "gdn_commit_rows": (I64, [I64, I32]),
        "gdn_shared_prefix_rows": (I64, [I64, I64]),
        "gdn_ckpt_init": (I32, [R, I32]),
        "gdn_ckpt_push": (I32, [R, I64]),
        "gdn_ckpt_find": (I32, [R, I64]),
        "gdn_ckpt_drop_above": (I32, [R, I64]),
        "gdn_status_str": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


lib = _load()


def exported_names():
    """Function names declared in include/gdn.h (for the ABI tests)."""
    names = []
    with open(HEADER) as f:
        for line in f:
            m = re.match(r"^(?:const\s+)?[A-Za-z_]\w*\s*\*?\s*([A-Za-z_]\w*)\s*\(", line)
            if m:
                names.append(m.group(1))
    return names


def gdn_status_str(status):
    return lib.gdn_status_str(int(status)).decode()


def _check(status, where):
    if status != GDN_OK:
        raise GdnError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(n_k_heads, n_v_heads, d_k, d_v, *, conv_width=4, grid=512,
              act_dtype=torch.bfloat16, out_dtype=torch.bfloat16, conv_silu=False, scale=None,
              l2_eps=1e-6, sub_chunk=SUB_CHUNK):
    d = gdn_desc(n_k_heads, n_v_heads, d_k, d_v, conv_width, sub_chunk, grid,
                 _DTYPE_CODE[act_dtype], _DTYPE_CODE[out_dtype], 1 if conv_silu else 0,
                 float(d_k ** -0.5 if scale is None else scale), float(l2_eps))
    return d


def gdn_desc_check(desc):
    return lib.gdn_desc_check(ctypes.byref(desc))


def gdn_desc_tag(desc):
    return lib.gdn_desc_tag(ctypes.byref(desc))


def gdn_state_S_bytes(desc):
    return lib.gdn_state_S_bytes(ctypes.byref(desc))


def gdn_state_conv_bytes(desc):
    return lib.gdn_state_conv_bytes(ctypes.byref(desc))


def gdn_workspace_bytes(desc, max_rows, max_segments=1):
    return lib.gdn_workspace_bytes(ctypes.byref(desc), int(max_rows), int(max_segments))


class State:
    """Device storage of one state (torch tensors) plus its C struct (pos, tag)."""

    def __init__(self, desc, device="cuda"):
        self.desc = desc
        self.S = torch.empty((desc.n_v_heads, desc.d_k, desc.d_v), dtype=torch.float32,
                             device=device)
        self.conv = (torch.empty((desc.conv_width - 1, desc.channels), dtype=desc.act_torch,
                                 device=device) if desc.conv_width > 0 else None)
        self.c = gdn_state(self.S.data_ptr(), _ptr(self.conv), 0, 0)

    @property
    def pos(self):
        return self.c.pos

    @property
    def tag(self):
        return self.c.tag

    def ref(self):
        return ctypes.byref(self.c)


def workspace(desc, max_rows, max_segments=1, device="cuda"):
    n = gdn_workspace_bytes(desc, max_rows, max_segments)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def gdn_state_init(desc, state, stream=None):
    _check(lib.gdn_state_init(ctypes.byref(desc), state.ref(), _stream(stream)), "gdn_state_init")


def gdn_state_capture(desc, live, snap, stream=None):
    _check(lib.gdn_state_capture(ctypes.byref(desc), live.ref(), snap.ref(), _stream(stream)),
           "gdn_state_capture")


def gdn_state_restore(desc, live, snap, stream=None):
    _check(lib.gdn_state_restore(ctypes.byref(desc), live.ref(), snap.ref(), _stream(stream)),
           "gdn_state_restore")


def gdn_state_fork(desc, src, dsts, stream=None):
    arr = (gdn_state * len(dsts))(*[d.c for d in dsts])
    st = lib.gdn_state_fork(ctypes.byref(desc), src.ref(), arr, len(dsts), _stream(stream))
    _check(st, "gdn_state_fork")
    for i, d in enumerate(dsts):
        d.c.pos, d.c.tag = arr[i].pos, arr[i].tag


def conv1d_state_step(desc, x, conv_w, window, y, T=None, stream=None):
    T = x.shape[0] if T is None else T
    _check(lib.conv1d_state_step(ctypes.byref(desc), _ptr(x), _ptr(conv_w), _ptr(window), _ptr(y),
                                 int(T), _stream(stream)), "conv1d_state_step")


def gdn_prefill_chunked(desc, x, conv_w, g, beta, state_in, state_out, o, T=None,
                        mode=GDN_COMMIT, ws=None, stream=None):
    """Returns rows_done."""
    T = x.shape[0] if T is None else T
    rows = ctypes.c_int64(-1)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.gdn_prefill_chunked(ctypes.byref(desc), _ptr(x), _ptr(conv_w), _ptr(g), _ptr(beta),
                                 state_in.ref(), state_out.ref(), _ptr(o), int(T), int(mode),
                                 ctypes.byref(rows), _ptr(ws), nbytes, _stream(stream))
    _check(st, "gdn_prefill_chunked")
    return rows.value


def gdn_prefill_chunked_events(desc, x, conv_w, g, beta, state_in, state_out, o, T=None,
                               mode=GDN_COMMIT, ws=None, events=(), stream=None):
    """gdn_prefill_chunked recording torch.cuda.Event objects around each kernel."""
    T = x.shape[0] if T is None else T
    rows = ctypes.c_int64(-1)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    for e in events:  # torch creates the underlying event on its first record
        if not e.cuda_event:
            e.record()
    ev = (ctypes.c_void_p * max(1, len(events)))(*[e.cuda_event for e in events])
    st = lib.gdn_prefill_chunked_events(ctypes.byref(desc), _ptr(x), _ptr(conv_w), _ptr(g),
                                        _ptr(beta), state_in.ref(), state_out.ref(), _ptr(o),
                                        int(T), int(mode), ctypes.byref(rows), _ptr(ws), nbytes,
                                        _stream(stream), ev, len(events))
    _check(st, "gdn_prefill_chunked_events")
    return rows.value


def gdn_prefill_branches(desc, cu_rows, x, conv_w, g, beta, inits, outs, o, ws, stream=None):
    B = len(inits)
    cu = (ctypes.c_int64 * (B + 1))(*[int(v) for v in cu_rows])
    ip = (ctypes.POINTER(gdn_state) * B)(*[ctypes.pointer(s.c) for s in inits])
    op = None if outs is None else (ctypes.POINTER(gdn_state) * B)(
        *[ctypes.pointer(s.c) for s in outs])
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.gdn_prefill_branches(ctypes.byref(desc), B, cu, _ptr(x), _ptr(conv_w), _ptr(g),
                                  _ptr(beta), ip, op, _ptr(o), _ptr(ws), nbytes, _stream(stream))
    _check(st, "gdn_prefill_branches")


def gdn_decode_step(desc, x, conv_w, g, beta, inits, outs, o, stream=None):
    """One token for each of len(inits) sequences: x [B][C], g/beta [B][Hv], o [B][Hv][d_v];
    outs[b] receives sequence b's state (it may be inits[b] itself)."""
    B = len(inits)
    ip = (ctypes.POINTER(gdn_state) * B)(*[ctypes.pointer(s.c) for s in inits])
    op = (ctypes.POINTER(gdn_state) * B)(*[ctypes.pointer(s.c) for s in outs])
    st = lib.gdn_decode_step(ctypes.byref(desc), B, _ptr(x), _ptr(conv_w), _ptr(g), _ptr(beta),
                             ip, op, _ptr(o), _stream(stream))
    _check(st, "gdn_decode_step")


def gdn_state_file_header_bytes():
    return lib.gdn_state_file_header_bytes()


def _np_ptr(a):
    return None if a is None else a.ctypes.data


def gdn_state_file_write(desc, S_host, conv_host, pos, weights_hash, path):
    """Host-buffer form: S_host [Hv][d_k][d_v] float32 and conv_host [W-1][C] numpy arrays of
    the activation dtype's bytes (float32, or uint16 holding bf16 bits)."""
    _check(lib.gdn_state_file_write(ctypes.byref(desc), _np_ptr(S_host), _np_ptr(conv_host),
                                    int(pos), int(weights_hash), os.fsencode(path)),
           "gdn_state_file_write")


def gdn_state_file_read(desc, weights_hash, path):
    """Returns (S [Hv][d_k][d_v] float32, window as raw numpy (float32 or uint16) or None, pos)."""
    import numpy as np
    S = np.empty((desc.n_v_heads, desc.d_k, desc.d_v), dtype=np.float32)
    conv = None
    if desc.conv_width > 0:
        conv = np.empty((desc.conv_width - 1, desc.channels),
                        dtype=np.uint16 if desc.act_dtype == GDN_BF16 else np.float32)
    pos = ctypes.c_int64(-1)
    _check(lib.gdn_state_file_read(ctypes.byref(desc), _np_ptr(S), _np_ptr(conv),
                                   ctypes.byref(pos), int(weights_hash), os.fsencode(path)),
           "gdn_state_file_read")
    return S, conv, pos.value


def gdn_state_save(desc, state, weights_hash, path, stream=None):
    _check(lib.gdn_state_save(ctypes.byref(desc), state.ref(), int(weights_hash),
                              os.fsencode(path), _stream(stream)), "gdn_state_save")


def gdn_state_load(desc, state, weights_hash, path, stream=None):
    _check(lib.gdn_state_load(ctypes.byref(desc), state.ref(), int(weights_hash),
                              os.fsencode(path), _stream(stream)), "gdn_state_load")


def gdn_linear(x, w, y, stream=None):
    """y[T][N] = x[T][K] w[N][K]^T (x, w bf16 device tensors; y bf16 or float32)."""
    T, K = x.shape
    N = w.shape[0]
    _check(lib.gdn_linear(int(T), int(K), int(N), _ptr(x), _ptr(w), _ptr(y),
                          _DTYPE_CODE[y.dtype], _stream(stream)), "gdn_linear")


def make_attn_desc(n_q_heads, n_kv_heads, head_dim, *, out_dtype=torch.bfloat16, scale=None):
    return gdn_attn_desc(n_q_heads, n_kv_heads, head_dim, _DTYPE_CODE[out_dtype],
                         float(head_dim ** -0.5 if scale is None else scale))


def gdn_attention_prefill(desc, seqs, stream=None):
    """seqs: list of (q [T][Hq][D], k cache [>= pos0+T][Hkv][D], v cache, o [T][Hq][D], pos0)."""
    arr = (gdn_attn_seq * max(1, len(seqs)))()
    for i, (q, k, v, o, pos0) in enumerate(seqs):
        arr[i] = gdn_attn_seq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(pos0), int(q.shape[0]))
    _check(lib.gdn_attention_prefill(ctypes.byref(desc), len(seqs), arr, _stream(stream)),
           "gdn_attention_prefill")


def gdn_commit_rows(n, grid):
    return lib.gdn_commit_rows(int(n), int(grid))


def gdn_shared_prefix_rows(state_pos, prefix_end):
    return lib.gdn_shared_prefix_rows(int(state_pos), int(prefix_end))


class CkptRing:
    """The library's checkpoint ring (host only)."""

    def __init__(self, cap=MAX_CHECKPOINTS):
        self.c = gdn_ckpt_ring()
        _check(lib.gdn_ckpt_init(ctypes.byref(self.c), int(cap)), "gdn_ckpt_init")

    def push(self, pos):
        return lib.gdn_ckpt_push(ctypes.byref(self.c), int(pos))

    def find(self, d):
        return lib.gdn_ckpt_find(ctypes.byref(self.c), int(d))

    def drop_above(self, d):
        return lib.gdn_ckpt_drop_above(ctypes.byref(self.c), int(d))

    def positions(self):
        return [self.c.pos[i] for i in range(self.c.cap)]
