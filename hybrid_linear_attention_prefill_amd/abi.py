"""ctypes declarations of the C ABI in include/gdn.h: constants, structs and the signature of
every exported function.

Loads no library and imports no torch: :mod:`.binding` applies these declarations to the HIP
library ``libgdn_prefill.so``; the CPU tests apply them to a host-only build of the same host
code.  Argument marshalling only; nothing of the method is computed here.
"""
import ctypes
import os

GDN_OK, GDN_EINVAL, GDN_ESHAPE, GDN_EGRID = 0, -1, -2, -3
GDN_EMISMATCH, GDN_EWORKSPACE, GDN_EDEVICE, GDN_EALIAS, GDN_EFILE = -4, -5, -6, -7, -8
GDN_F32, GDN_BF16 = 0, 1
GDN_COMMIT, GDN_FORK = 0, 1
SUB_CHUNK = 64
MAX_CHECKPOINTS = 6



GDN_STORE_UNUSED, GDN_STORE_RESIDENT, GDN_STORE_ON_DISK, GDN_STORE_DROPPED = 0, 1, 2, 3
GDN_STORE_WAS_RESIDENT, GDN_STORE_FROM_DISK, GDN_STORE_FRESH = 0, 1, 2


def dtype_code(dtype):
    """GDN_F32 / GDN_BF16 for a code, a torch dtype or a name ("float32", "bfloat16")."""
    if isinstance(dtype, int):
        return dtype
    name = str(dtype).replace("torch.", "")
    return {"float32": GDN_F32, "bfloat16": GDN_BF16}[name]


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
        import torch
        return {GDN_F32: torch.float32, GDN_BF16: torch.bfloat16}[self.act_dtype]

    @property
    def out_torch(self):
        import torch
        return {GDN_F32: torch.float32, GDN_BF16: torch.bfloat16}[self.out_dtype]


class gdn_state(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("conv", ctypes.c_void_p), ("pos", ctypes.c_int64),
                ("tag", ctypes.c_uint64)]


class gdn_attn_desc(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]

    @property
    def out_torch(self):
        import torch
        return {GDN_F32: torch.float32, GDN_BF16: torch.bfloat16}[self.out_dtype]


class gdn_attn_seq(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("pos0", ctypes.c_int64), ("T", ctypes.c_int64)]


class gdn_ckpt_ring(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int32), ("n", ctypes.c_int32),
                ("pos", ctypes.c_int64 * MAX_CHECKPOINTS),
                ("age", ctypes.c_uint64 * MAX_CHECKPOINTS), ("clock", ctypes.c_uint64)]


class gdn_store_entry(ctypes.Structure):
    _fields_ = [("id", ctypes.c_uint64), ("pos", ctypes.c_int64), ("last_use", ctypes.c_uint64),
                ("slot", ctypes.c_int32), ("where", ctypes.c_int32)]


class gdn_store(ctypes.Structure):
    _fields_ = [("desc", gdn_desc), ("slots", ctypes.POINTER(gdn_state)),
                ("n_slots", ctypes.c_int32), ("max_resident", ctypes.c_int32),
                ("cap_bytes", ctypes.c_size_t), ("state_bytes", ctypes.c_size_t),
                ("entries", ctypes.POINTER(gdn_store_entry)), ("max_entries", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("weights_hash", ctypes.c_uint64),
                ("clock", ctypes.c_uint64), ("dir", ctypes.c_char * 512)]


def signatures():
    """{name: (restype, argtypes)} of every function include/gdn.h declares."""
    D, S, V, I32, I64, SZ = (ctypes.POINTER(gdn_desc), ctypes.POINTER(gdn_state), ctypes.c_void_p,
                            ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t)
    R = ctypes.POINTER(gdn_ckpt_ring)
    return {
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
        "gdn_prefill_chunked_noalloc": (I32, [D, V, V, V, V, S, S, V, I64, I32,
                                              ctypes.POINTER(ctypes.c_int64), V]),
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
        "gdn_store_init": (I32, [ctypes.POINTER(gdn_store), D, S, I32, SZ, ctypes.c_char_p,
                                 ctypes.c_uint64, ctypes.POINTER(gdn_store_entry), I32]),
        "gdn_store_acquire": (I32, [ctypes.POINTER(gdn_store), ctypes.c_uint64,
                                    ctypes.POINTER(S), ctypes.POINTER(I32), V]),
        "gdn_store_evict": (I32, [ctypes.POINTER(gdn_store), ctypes.c_uint64, V]),
        "gdn_store_flush": (I32, [ctypes.POINTER(gdn_store), V]),
        "gdn_store_drop": (I32, [ctypes.POINTER(gdn_store), ctypes.c_uint64]),
        "gdn_store_find": (I32, [ctypes.POINTER(gdn_store), ctypes.c_uint64]),
    }


# Functions defined in the HIP sources only (absent from a host-only build of the host half).
DEVICE_ONLY = ("gdn_prefill_chunked_noalloc",)
NOALLOC_WORKSPACE_BYTES = 32 << 20


def declare(lib, host_only=False):
    """Sets restype and argtypes of every declared function on a loaded library (with
    host_only, of those a host-only build defines)."""
    for name, (res, args) in signatures().items():
        if host_only and name in DEVICE_ONLY:
            continue
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


def make_desc(n_k_heads, n_v_heads, d_k, d_v, *, conv_width=4, grid=512, act_dtype="bfloat16",
              out_dtype="bfloat16", conv_silu=False, scale=None, l2_eps=1e-6, sub_chunk=SUB_CHUNK):
    return gdn_desc(n_k_heads, n_v_heads, d_k, d_v, conv_width, sub_chunk, grid,
                    dtype_code(act_dtype), dtype_code(out_dtype), 1 if conv_silu else 0,
                    float(d_k ** -0.5 if scale is None else scale), float(l2_eps))


def declared_names(header):
    """Function names declared in a C header such as include/gdn.h."""
    import re
    names = []
    with open(header) as f:
        for line in f:
            m = re.match(r"^(?:const\s+)?[A-Za-z_]\w*\s*\*?\s*([A-Za-z_]\w*)\s*\(", line)
            if m:
                names.append(m.group(1))
    return names


class GdnError(RuntimeError):
    def __init__(self, status, where, text=""):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, text, status))


def _np_ptr(a):
    return None if a is None else a.ctypes.data


class HostCalls:
    """The calls that touch no device memory, over a loaded library: descriptor checks and
    tags, sizes, the grid arithmetic, the checkpoint ring and state files in host buffers."""

    def __init__(self, lib):
        self.lib = lib
        host = self

        class CkptRing:
            """The library's checkpoint ring (host only)."""

            def __init__(self, cap=MAX_CHECKPOINTS):
                self.c = gdn_ckpt_ring()
                host.check(host.lib.gdn_ckpt_init(ctypes.byref(self.c), int(cap)), "gdn_ckpt_init")

            def push(self, pos):
                return host.lib.gdn_ckpt_push(ctypes.byref(self.c), int(pos))

            def find(self, d):
                return host.lib.gdn_ckpt_find(ctypes.byref(self.c), int(d))

            def drop_above(self, d):
                return host.lib.gdn_ckpt_drop_above(ctypes.byref(self.c), int(d))

            def positions(self):
                return [self.c.pos[i] for i in range(self.c.cap)]

        self.CkptRing = CkptRing

    def gdn_status_str(self, status):
        return self.lib.gdn_status_str(int(status)).decode()

    def check(self, status, where):
        if status != GDN_OK:
            raise GdnError(status, where, self.gdn_status_str(status))

    def gdn_desc_check(self, desc):
        return self.lib.gdn_desc_check(ctypes.byref(desc))

    def gdn_desc_tag(self, desc):
        return self.lib.gdn_desc_tag(ctypes.byref(desc))

    def gdn_state_S_bytes(self, desc):
        return self.lib.gdn_state_S_bytes(ctypes.byref(desc))

    def gdn_state_conv_bytes(self, desc):
        return self.lib.gdn_state_conv_bytes(ctypes.byref(desc))

    def gdn_workspace_bytes(self, desc, max_rows, max_segments=1):
        return self.lib.gdn_workspace_bytes(ctypes.byref(desc), int(max_rows), int(max_segments))

    def gdn_state_file_header_bytes(self):
        return self.lib.gdn_state_file_header_bytes()

    def gdn_state_file_write(self, desc, S_host, conv_host, pos, weights_hash, path):
        """Host-buffer form: S_host [Hv][d_k][d_v] float32 and conv_host [W-1][C] numpy arrays
        of the activation dtype's bytes (float32, or uint16 holding bf16 bits)."""
        self.check(self.lib.gdn_state_file_write(ctypes.byref(desc), _np_ptr(S_host),
                                                 _np_ptr(conv_host), int(pos), int(weights_hash),
                                                 os.fsencode(path)), "gdn_state_file_write")

    def gdn_state_file_read(self, desc, weights_hash, path):
        """Returns (S [Hv][d_k][d_v] float32, window as raw numpy (float32 or uint16) or None,
        pos)."""
        import numpy as np
        S = np.empty((desc.n_v_heads, desc.d_k, desc.d_v), dtype=np.float32)
        conv = None
        if desc.conv_width > 0:
            conv = np.empty((desc.conv_width - 1, desc.channels),
                            dtype=np.uint16 if desc.act_dtype == GDN_BF16 else np.float32)
        pos = ctypes.c_int64(-1)
        self.check(self.lib.gdn_state_file_read(ctypes.byref(desc), _np_ptr(S), _np_ptr(conv),
                                                ctypes.byref(pos), int(weights_hash),
                                                os.fsencode(path)), "gdn_state_file_read")
        return S, conv, pos.value

    def gdn_commit_rows(self, n, grid):
        return self.lib.gdn_commit_rows(int(n), int(grid))

    def gdn_shared_prefix_rows(self, state_pos, prefix_end):
        return self.lib.gdn_shared_prefix_rows(int(state_pos), int(prefix_end))


class Store:
    """A session store (gdn_store) over the caller's slot objects, each holding its C state in
    ``.c`` (device states from the binding, or host states in the CPU tests).  The slots' C
    structs are moved into one array that the library reads and updates; each slot object's
    ``.c`` then refers to its element of that array."""

    def __init__(self, lib, desc, slots, cap_bytes, directory=None, weights_hash=0,
                 max_entries=None):
        self.lib, self.desc, self.slot_objs = lib, desc, list(slots)
        n = len(self.slot_objs)
        self.slots = (gdn_state * n)(*[s.c for s in self.slot_objs])
        for i, s in enumerate(self.slot_objs):
            s.c = self.slots[i]
        self.max_entries = max_entries or 4 * n
        self.entries = (gdn_store_entry * self.max_entries)()
        self.c = gdn_store()
        d = None if directory is None else os.fsencode(directory)
        self.status = lib.gdn_store_init(ctypes.byref(self.c), ctypes.byref(desc), self.slots, n,
                                         int(cap_bytes), d, int(weights_hash), self.entries,
                                         self.max_entries)

    def acquire(self, sid, stream=None):
        """(status, slot object or None, origin)."""
        p = ctypes.POINTER(gdn_state)()
        origin = ctypes.c_int32(-1)
        st = self.lib.gdn_store_acquire(ctypes.byref(self.c), int(sid), ctypes.byref(p),
                                        ctypes.byref(origin), stream)
        if st != GDN_OK:
            return st, None, origin.value
        k = (ctypes.addressof(p.contents) - ctypes.addressof(self.slots)) // ctypes.sizeof(gdn_state)
        return st, self.slot_objs[k], origin.value

    def evict(self, sid, stream=None):
        return self.lib.gdn_store_evict(ctypes.byref(self.c), int(sid), stream)

    def flush(self, stream=None):
        return self.lib.gdn_store_flush(ctypes.byref(self.c), stream)

    def drop(self, sid):
        return self.lib.gdn_store_drop(ctypes.byref(self.c), int(sid))

    def entry(self, sid):
        """The session's entry (a copy) or None."""
        i = self.lib.gdn_store_find(ctypes.byref(self.c), int(sid))
        if i < 0:
            return None
        e = self.entries[i]
        return dict(id=e.id, pos=e.pos, last_use=e.last_use, slot=e.slot, where=e.where)

    def resident(self):
        return sorted(e.id for e in self.entries if e.where == GDN_STORE_RESIDENT)
