"""Thin ctypes binding of libgdn_prefill.so (the C ABI in include/gdn.h).

Argument marshalling only: every function here converts torch tensors and Python values to
the C types, calls the function of the same name and raises :class:`GdnError` on a negative
status.  All compute runs in the library's HIP kernels on the caller's (torch current)
stream.  Importing this module raises if the library has not been built; there is no
fallback.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn_prefill.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "gdn.h")

from .abi import (GDN_OK, GDN_EINVAL, GDN_ESHAPE, GDN_EGRID, GDN_EMISMATCH,  # noqa: F401
                  GDN_EWORKSPACE, GDN_EDEVICE, GDN_EALIAS, GDN_EFILE, GDN_F32, GDN_BF16,
                  GDN_COMMIT, GDN_FORK, SUB_CHUNK, MAX_CHECKPOINTS, gdn_desc, gdn_state,
                  gdn_attn_desc, gdn_attn_seq, gdn_ckpt_ring, dtype_code, GDN_STORE_UNUSED,
                  GDN_STORE_RESIDENT, GDN_STORE_ON_DISK, GDN_STORE_DROPPED,
                  GDN_STORE_WAS_RESIDENT, GDN_STORE_FROM_DISK, GDN_STORE_FRESH)
from . import abi as _abi

_DTYPE_CODE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


GdnError = _abi.GdnError


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libgdn_prefill.so is not built: run "
                          "python -m hybrid_linear_attention_prefill_amd.build")
    return _abi.declare(ctypes.CDLL(LIB_PATH))


lib = _load()
_host = _abi.HostCalls(lib)
# host-only calls (no device memory): descriptor, sizes, grid arithmetic, checkpoint ring,
# state files in host buffers
gdn_status_str = _host.gdn_status_str
_check = _host.check
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


def exported_names():
    """Function names declared in include/gdn.h (for the ABI tests)."""
    return _abi.declared_names(HEADER)


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
    return _abi.make_desc(n_k_heads, n_v_heads, d_k, d_v, conv_width=conv_width, grid=grid,
                          act_dtype=act_dtype, out_dtype=out_dtype, conv_silu=conv_silu,
                          scale=scale, l2_eps=l2_eps, sub_chunk=sub_chunk)


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


def gdn_prefill_chunked_noalloc(desc, x, conv_w, g, beta, state_in, state_out, o, T=None,
                                mode=GDN_COMMIT, stream=None):
    """gdn_prefill_chunked with the library's static workspace (no workspace argument).
    Returns rows_done."""
    T = x.shape[0] if T is None else T
    rows = ctypes.c_int64(-1)
    st = lib.gdn_prefill_chunked_noalloc(ctypes.byref(desc), _ptr(x), _ptr(conv_w), _ptr(g),
                                         _ptr(beta), state_in.ref(), state_out.ref(), _ptr(o),
                                         int(T), int(mode), ctypes.byref(rows), _stream(stream))
    _check(st, "gdn_prefill_chunked_noalloc")
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
    return gdn_attn_desc(n_q_heads, n_kv_heads, head_dim, dtype_code(out_dtype),
                         float(head_dim ** -0.5 if scale is None else scale))


def gdn_attention_prefill(desc, seqs, stream=None):
    """seqs: list of (q [T][Hq][D], k cache [>= pos0+T][Hkv][D], v cache, o [T][Hq][D], pos0)."""
    arr = (gdn_attn_seq * max(1, len(seqs)))()
    for i, (q, k, v, o, pos0) in enumerate(seqs):
        arr[i] = gdn_attn_seq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(pos0), int(q.shape[0]))
    _check(lib.gdn_attention_prefill(ctypes.byref(desc), len(seqs), arr, _stream(stream)),
           "gdn_attention_prefill")


class SessionStore(_abi.Store):
    """gdn_store over n_slots device states made here; acquire() returns (State, origin) and
    raises GdnError on failure."""

    def __init__(self, desc, n_slots, cap_bytes, directory=None, weights_hash=0, max_entries=None,
                 device="cuda"):
        super().__init__(lib, desc, [State(desc, device=device) for _ in range(n_slots)], cap_bytes,
                         directory, weights_hash, max_entries)
        _check(self.status, "gdn_store_init")

    def acquire(self, sid, stream=None):
        st, slot, origin = super().acquire(sid, _stream(stream))
        _check(st, "gdn_store_acquire")
        return slot, origin

    def evict(self, sid, stream=None):
        _check(super().evict(sid, _stream(stream)), "gdn_store_evict")

    def flush(self, stream=None):
        _check(super().flush(_stream(stream)), "gdn_store_flush")

    def drop(self, sid):
        _check(super().drop(sid), "gdn_store_drop")
