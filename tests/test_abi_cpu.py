"""The C-ABI library on the CPU: exports, validation, grid arithmetic, checkpoint ring.

No compute call runs here: every call below is refused by host validation before any HIP
call, or is host-only integer logic.  Fake device addresses are never dereferenced.
"""
import ctypes
import os
import itertools

import pytest

from tests import hostlib as b

FAKE = 0x7F0000000000  # never dereferenced: validation refuses first


def layer_desc(**kw):
    return b.make_desc(16, 32, 128, 128, **kw)


def test_hip_library_loads_and_exports_every_declared_symbol():
    """The built HIP library (libgdn_prefill.so) loads on a machine without a GPU and exports
    every function include/gdn.h declares; the Python binding wraps each of them.  (Only this
    test loads the ROCm-linked library; the others run the host half without ROCm.)"""
    import re
    from hybrid_linear_attention_prefill_amd import abi
    pkg = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "hybrid_linear_attention_prefill_amd")
    names = b.exported_names()
    assert len(names) >= 19
    hip = ctypes.CDLL(os.path.join(pkg, "libgdn_prefill.so"))
    assert set(abi.signatures()) == set(names)
    with open(os.path.join(pkg, "binding.py")) as f:
        src = f.read()
    wrapped = (set(re.findall(r"^def (\w+)\(", src, re.M)) | set(re.findall(r"^(\w+) = ", src, re.M))
               | set(re.findall(r"^class (\w+)", src, re.M)))
    for n in names:
        assert hasattr(hip, n), n
        if n not in abi.DEVICE_ONLY:
            assert hasattr(b.lib, n), n  # the host-only build exports the same host half
        # the checkpoint ring and the session store are wrapped as classes (CkptRing, SessionStore)
        as_method = n.startswith("gdn_ckpt_") or n.startswith("gdn_store_")
        assert n in wrapped or as_method, "binding lacks " + n
    assert "SessionStore" in wrapped and "CkptRing" in wrapped


def test_desc_check_refusals():
    assert b.gdn_desc_check(layer_desc()) == b.GDN_OK
    assert b.gdn_desc_check(b.make_desc(1, 1, 64, 64, conv_width=0,
                                        act_dtype="float32")) == b.GDN_OK
    bad = [
        (dict(), dict(d_v=64), b.GDN_ESHAPE),          # d_k != d_v
        (dict(), dict(d_k=96, d_v=96), b.GDN_ESHAPE),  # unsupported head dim
        (dict(), dict(n_v_heads=24, n_k_heads=16), b.GDN_ESHAPE),
        (dict(conv_width=3), dict(), b.GDN_ESHAPE),
        (dict(grid=100), dict(), b.GDN_ESHAPE),
        (dict(grid=0), dict(), b.GDN_ESHAPE),
        (dict(sub_chunk=32), dict(), b.GDN_ESHAPE),
        (dict(), dict(n_k_heads=0), b.GDN_EINVAL),
    ]
    for kw, fields, code in bad:
        d = layer_desc(**kw)
        for f, v in fields.items():
            setattr(d, f, v)
        assert b.gdn_desc_check(d) == code, (kw, fields)
    d = layer_desc()
    d.act_dtype = 7
    assert b.gdn_desc_check(d) == b.GDN_EINVAL
    assert b.lib.gdn_desc_check(None) == b.GDN_EINVAL


def test_tag_identifies_shape_and_grid_not_scale():
    t = b.gdn_desc_tag(layer_desc())
    assert t == b.gdn_desc_tag(layer_desc(scale=0.5, l2_eps=1e-3))
    assert t != b.gdn_desc_tag(layer_desc(grid=1024))
    assert t != b.gdn_desc_tag(b.make_desc(16, 32, 64, 64))
    assert t != b.gdn_desc_tag(layer_desc(act_dtype="float32"))


def test_sizes():
    d = layer_desc()
    assert b.gdn_state_S_bytes(d) == 32 * 128 * 128 * 4
    assert b.gdn_state_conv_bytes(d) == 3 * 8192 * 2
    assert b.gdn_state_conv_bytes(b.make_desc(1, 1, 64, 64, conv_width=0)) == 0
    w1 = b.gdn_workspace_bytes(d, 8192, 1)
    w2 = b.gdn_workspace_bytes(d, 8192 + 64, 1)
    assert 0 < w1 < w2
    bad = layer_desc(grid=7)
    assert b.gdn_workspace_bytes(bad, 10, 1) == 0 and b.gdn_state_S_bytes(bad) == 0


def _state(pos=0, tag=None, S=FAKE, conv=FAKE + (1 << 30)):
    s = b.gdn_state(S, conv, pos, b.gdn_desc_tag(layer_desc()) if tag is None else tag)
    return s


# distinct fake device addresses for the buffers of a call (states sit at FAKE and FAKE + 1 GiB)
X_, W_, G_, B_, O_ = (FAKE + (k << 30) for k in (10, 11, 12, 13, 14))


def _chunked(d, sin, sout, T=512, mode=b.GDN_COMMIT, ws=FAKE + (2 << 30), ws_bytes=1 << 40,
             x=X_, conv_w=W_, g=G_, beta=B_, o=O_):
    rows = ctypes.c_int64(-7)
    st = b.lib.gdn_prefill_chunked(ctypes.byref(d), x, conv_w, g, beta, ctypes.byref(sin),
                                   ctypes.byref(sout), o, T, mode, ctypes.byref(rows), ws,
                                   ws_bytes, None)
    return st, rows.value


def test_prefill_validation_refuses_before_device_work():
    d = layer_desc()
    s = _state(pos=512)
    before = (s.pos, s.tag)
    cases = [
        (dict(sin=_state(pos=100), sout=_state(pos=100)), b.GDN_EGRID),          # commit off grid
        (dict(sin=_state(pos=32), sout=_state(S=FAKE + (5 << 30), conv=FAKE + (6 << 30)),
              mode=b.GDN_FORK), b.GDN_EGRID),                                    # fork off 64
        (dict(sin=s, sout=s, mode=b.GDN_FORK), b.GDN_EALIAS),                    # fork in place
        (dict(sin=_state(tag=123), sout=_state(tag=123)), b.GDN_EMISMATCH),      # foreign state
        (dict(sin=s, sout=s, ws=None), b.GDN_EWORKSPACE),
        (dict(sin=s, sout=s, ws_bytes=1000), b.GDN_EWORKSPACE),
        (dict(sin=s, sout=s, mode=5), b.GDN_EINVAL),
        (dict(sin=s, sout=s, T=-1), b.GDN_EINVAL),
        (dict(sin=s, sout=s, x=None), b.GDN_EINVAL),
        (dict(sin=s, sout=s, conv_w=None), b.GDN_EINVAL),
        # overlapping but not identical output state in a commit
        (dict(sin=s, sout=_state(pos=512, S=FAKE + 64, conv=FAKE + (7 << 30))), b.GDN_EALIAS),
        # misaligned device pointers
        (dict(sin=s, sout=s, x=X_ + 2), b.GDN_EINVAL),
        (dict(sin=s, sout=s, o=O_ + 8), b.GDN_EINVAL),
        (dict(sin=s, sout=s, conv_w=W_ + 4), b.GDN_EINVAL),
        (dict(sin=s, sout=s, g=G_ + 2), b.GDN_EINVAL),
        (dict(sin=s, sout=s, beta=B_ + 1), b.GDN_EINVAL),
        # written buffers overlapping anything else the call touches
        (dict(sin=s, sout=s, o=X_ + (1 << 20)), b.GDN_EALIAS),                     # o inside x
        (dict(sin=s, sout=s, o=G_), b.GDN_EALIAS),                                 # o on g
        (dict(sin=s, sout=s, ws=O_ + 4096), b.GDN_EALIAS),                         # workspace in o
        (dict(sin=s, sout=s, ws=W_), b.GDN_EALIAS),                                # workspace on conv w
        (dict(sin=s, sout=s, o=FAKE + 4096), b.GDN_EALIAS),                        # o in the state
        (dict(sin=s, sout=_state(pos=512, S=X_, conv=FAKE + (7 << 30))), b.GDN_EALIAS),  # S out on x
        (dict(sin=_state(pos=512, S=FAKE + 2), sout=_state(pos=512, S=FAKE + 2)), b.GDN_EINVAL),
        (dict(sin=s, sout=_state(pos=512, S=FAKE + (15 << 30), conv=FAKE + (16 << 30) + 8)),
         b.GDN_EINVAL),
    ]
    for kw, code in cases:
        sin, sout = kw.pop("sin"), kw.pop("sout")
        pos_in, pos_out = sin.pos, sout.pos
        st, rows = _chunked(d, sin, sout, **kw)
        assert st == code, (kw, st)
        assert rows == -7 and sin.pos == pos_in and sout.pos == pos_out
    assert (s.pos, s.tag) == before


def test_branches_validation():
    d = layer_desc()
    s = _state(pos=960)
    sp = ctypes.pointer(s)

    def call(B, cu, inits, outs=None, ws_bytes=1 << 40, x=X_, o=O_):
        cu_a = (ctypes.c_int64 * len(cu))(*cu)
        ia = (ctypes.POINTER(b.gdn_state) * B)(*inits)
        oa = None if outs is None else (ctypes.POINTER(b.gdn_state) * B)(*outs)
        return b.lib.gdn_prefill_branches(ctypes.byref(d), B, cu_a, x, W_, G_, B_, ia,
                                          oa, o, FAKE + (3 << 30), ws_bytes, None)

    assert call(2, [0, 10, 10], [sp, sp]) == b.GDN_EINVAL            # empty branch
    assert call(1, [5, 10], [sp]) == b.GDN_EINVAL                     # offsets must start at 0
    assert b.lib.gdn_prefill_branches(ctypes.byref(d), 0, None, FAKE, FAKE, FAKE, FAKE, None,
                                      None, FAKE, FAKE, 1 << 40, None) == b.GDN_EINVAL
    off = _state(pos=1000)
    assert call(1, [0, 10], [ctypes.pointer(off)]) == b.GDN_EGRID     # start not on 64
    assert call(1, [0, 10], [sp], [sp]) == b.GDN_EALIAS               # out overlaps an init
    o1 = _state(S=FAKE + (8 << 30), conv=FAKE + (9 << 30))
    assert call(2, [0, 3, 6], [sp, sp], [ctypes.pointer(o1), ctypes.pointer(o1)]) == b.GDN_EALIAS
    assert call(1, [0, 10], [sp], ws_bytes=10) == b.GDN_EWORKSPACE
    foreign = _state(pos=0, tag=99)
    assert call(1, [0, 10], [ctypes.pointer(foreign)]) == b.GDN_EMISMATCH
    assert call(1, [0, 10], [sp], o=X_) == b.GDN_EALIAS                # o on x
    assert call(1, [0, 10], [sp], o=FAKE + 64) == b.GDN_EALIAS         # o in an entry state
    o2 = _state(S=X_ + 256, conv=FAKE + (9 << 30))
    assert call(1, [0, 10], [sp], [ctypes.pointer(o2)]) == b.GDN_EALIAS  # final S on x


def test_decode_validation_refuses_before_device_work():
    d = layer_desc()
    a = _state(pos=700)
    c = _state(pos=33, S=FAKE + (20 << 30), conv=FAKE + (21 << 30))
    ap, cp = ctypes.pointer(a), ctypes.pointer(c)

    def call(B, inits, outs, x=X_, conv_w=W_, g=G_, beta=B_, o=O_, desc=d):
        ia = None if inits is None else (ctypes.POINTER(b.gdn_state) * max(B, 1))(*inits)
        oa = None if outs is None else (ctypes.POINTER(b.gdn_state) * max(B, 1))(*outs)
        return b.lib.gdn_decode_step(ctypes.byref(desc), B, x, conv_w, g, beta, ia, oa, o, None)

    assert call(0, [ap], [ap]) == b.GDN_EINVAL
    assert call(1, None, [ap]) == b.GDN_EINVAL
    assert call(1, [ap], None) == b.GDN_EINVAL
    for kw in (dict(x=None), dict(g=None), dict(beta=None), dict(o=None), dict(conv_w=None),
               dict(x=X_ + 2), dict(o=O_ + 8), dict(g=G_ + 2), dict(conv_w=W_ + 4)):
        assert call(1, [ap], [ap], **kw) == b.GDN_EINVAL, kw
    # the output row overlapping the input row, a gate, or the state it updates
    assert call(1, [ap], [ap], o=X_ + 1024) == b.GDN_EALIAS
    assert call(1, [ap], [ap], o=B_) == b.GDN_EALIAS
    assert call(1, [ap], [ap], o=FAKE + 512) == b.GDN_EALIAS
    foreign = _state(tag=77)
    assert call(1, [ctypes.pointer(foreign)], [ctypes.pointer(foreign)]) == b.GDN_EMISMATCH
    # a shared input updated in place by one sequence while another reads it
    assert call(2, [ap, ap], [ap, cp]) == b.GDN_EALIAS
    # two sequences writing the same state
    assert call(2, [ap, cp], [ctypes.pointer(_state(S=FAKE + (22 << 30), conv=FAKE + (23 << 30)))] * 2) == b.GDN_EALIAS
    # an output overlapping its own input without being it
    part = _state(pos=700, S=FAKE + 256, conv=FAKE + (24 << 30))
    assert call(1, [ap], [ctypes.pointer(part)]) == b.GDN_EALIAS
    # output state with a misaligned window
    bad = _state(S=FAKE + (25 << 30), conv=FAKE + (26 << 30) + 8)
    assert call(1, [ap], [ctypes.pointer(bad)]) == b.GDN_EINVAL
    # S only 4-byte aligned: enough for a prefill, not for the step's 16-byte accesses
    s4 = _state(pos=5, S=FAKE + (27 << 30) + 4, conv=FAKE + (28 << 30))
    assert call(1, [ctypes.pointer(s4)], [ctypes.pointer(s4)]) == b.GDN_EINVAL
    assert (a.pos, c.pos, part.pos) == (700, 33, 700)


def test_linear_validation():
    def call(T=64, K=128, N=32, x=X_, w=W_, y=O_, od=b.GDN_BF16):
        return b.lib.gdn_linear(T, K, N, x, w, y, od, None)

    for kw in (dict(K=96), dict(K=0), dict(N=24), dict(N=0), dict(T=-1), dict(od=5),
               dict(x=None), dict(w=None), dict(y=None), dict(x=X_ + 8), dict(y=O_ + 4)):
        assert call(**kw) == b.GDN_EINVAL, kw
    assert call(T=0, x=None, w=None, y=None) == b.GDN_OK  # nothing to do, nothing touched
    # the output overlapping an input: x (64 x 128 bf16 = 16 KiB) or w
    assert call(y=X_ + 4096) == b.GDN_EALIAS
    assert call(y=W_ - 1024) == b.GDN_EALIAS


def test_state_ops_validation():
    d = layer_desc()
    live = _state(pos=512)
    other = _state(tag=5, S=FAKE + (10 << 30), conv=FAKE + (11 << 30))
    assert b.lib.gdn_state_restore(ctypes.byref(d), ctypes.byref(live), ctypes.byref(other),
                                   None) == b.GDN_EMISMATCH
    assert live.pos == 512
    assert b.lib.gdn_state_capture(ctypes.byref(d), ctypes.byref(live), ctypes.byref(live),
                                   None) == b.GDN_EALIAS
    assert b.lib.gdn_state_fork(ctypes.byref(d), ctypes.byref(live), None, 2, None) == b.GDN_EINVAL
    dst = (b.gdn_state * 2)(_state(S=FAKE + (12 << 30), conv=FAKE + (13 << 30)),
                            _state(S=FAKE + (12 << 30), conv=FAKE + (14 << 30)))
    assert b.lib.gdn_state_fork(ctypes.byref(d), ctypes.byref(live), dst, 2, None) == b.GDN_EALIAS
    assert b.lib.conv1d_state_step(ctypes.byref(b.make_desc(1, 1, 64, 64, conv_width=0)), FAKE,
                                   FAKE, FAKE, FAKE, 10, None) == b.GDN_ESHAPE
    assert b.lib.conv1d_state_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, -1, None) == b.GDN_EINVAL
    # T == 0 is a no-op that touches nothing
    assert b.lib.conv1d_state_step(ctypes.byref(d), None, FAKE, FAKE, None, 0, None) == b.GDN_OK
    # written buffers (y, window) overlapping another buffer of the call
    assert b.lib.conv1d_state_step(ctypes.byref(d), X_, W_, FAKE, X_ + 64, 8, None) == b.GDN_EALIAS
    assert b.lib.conv1d_state_step(ctypes.byref(d), X_, W_, X_ + 16, O_, 8, None) == b.GDN_EALIAS
    assert b.lib.conv1d_state_step(ctypes.byref(d), X_, W_, FAKE, FAKE + 8, 8, None) == b.GDN_EALIAS
    # every pointer the kernel moves 16-byte pieces through must be 16-byte aligned
    for i in range(4):
        args = [X_, W_, FAKE, O_]
        args[i] += 8
        assert b.lib.conv1d_state_step(ctypes.byref(d), *args, 8, None) == b.GDN_EINVAL, i


def test_commit_rows_exhaustive():
    for grid in (64, 128, 512, 2048):
        for n in range(0, 5000, 7):
            r = b.gdn_commit_rows(n, grid)
            assert r % grid == 0 and 0 <= n - r < grid
    assert b.gdn_commit_rows(-1, 512) == -1 and b.gdn_commit_rows(10, 0) == -1


def test_shared_prefix_split_rule():
    """Each prefix runs to its last multiple of 64; the remainder joins every later run."""
    for P in (0, 1, 63, 64, 65, 300, 1000):
        run = b.gdn_shared_prefix_rows(0, P)
        assert run == (P // 64) * 64 and 0 <= P - run < 64
    # groups of 0/1/70/128 tokens after a 1,000-token request prefix (state at 960)
    assert [b.gdn_shared_prefix_rows(960, 1000 + gl) for gl in (0, 1, 70, 128)] == [0, 0, 64, 128]
    for pos in range(0, 1024, 64):
        for end in range(pos, pos + 300, 5):
            run = b.gdn_shared_prefix_rows(pos, end)
            assert run >= 0 and (pos + run) % 64 == 0 and 0 <= end - pos - run
            assert run == 0 or end - (pos + run) < 64
    assert b.gdn_shared_prefix_rows(30, 100) == -1 and b.gdn_shared_prefix_rows(64, 10) == -1


def test_checkpoint_ring():
    r = b.CkptRing(6)
    assert r.find(10 ** 9) == -1                      # none: start over
    slots = [r.push(p) for p in (512, 1024, 2048, 3072, 4096, 5120)]
    assert sorted(slots) == list(range(6))
    assert r.push(1024) == slots[1]                   # same position reuses its slot
    s = r.push(6144)                                  # full: the oldest (512) is evicted
    assert s == slots[0] and 512 not in r.positions()
    assert r.positions()[r.find(3000)] == 2048        # newest at or below the divergence
    assert r.positions()[r.find(3072)] == 3072
    assert r.find(1000) == -1                         # 512 was evicted: start over
    assert r.drop_above(3000) == 4 and max(r.positions()) == 2048  # 3072, 4096, 5120, 6144
    with pytest.raises(b.GdnError):
        b.CkptRing(7)


def test_checkpoint_ring_matches_brute_force():
    import random
    rnd = random.Random(0)
    for trial in range(200):
        cap = rnd.randint(1, 6)
        r = b.CkptRing(cap)
        model = []  # (pos, stamp)
        stamp = 0
        for _ in range(rnd.randint(1, 15)):
            p = rnd.randrange(0, 20) * 512
            stamp += 1
            if any(q == p for q, _ in model):
                model = [(q, stamp if q == p else t) for q, t in model]
            elif len(model) < cap:
                model.append((p, stamp))
            else:
                oldest = min(model, key=lambda e: e[1])
                model.remove(oldest)
                model.append((p, stamp))
            r.push(p)
            for d in range(0, 21 * 512, 256):
                cands = [q for q, _ in model if q <= d]
                got = r.find(d)
                assert (got == -1) == (not cands)
                if cands:
                    assert r.positions()[got] == max(cands)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert isinstance(b.gdn_status_str(code), str) and b.gdn_status_str(code)


def test_attention_validation():
    def call(Hq=8, Hkv=1, D=128, od=b.GDN_BF16, scale=0.1, seqs=None, B=None):
        d = b.gdn_attn_desc(Hq, Hkv, D, od, scale)
        if seqs is None:
            seqs = [b.gdn_attn_seq(FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20), 0, 16)]
        arr = (b.gdn_attn_seq * max(1, len(seqs)))(*seqs)
        return b.lib.gdn_attention_prefill(ctypes.byref(d), len(seqs) if B is None else B,
                                           arr, None)

    for kw in (dict(Hq=6, Hkv=4), dict(Hq=12, Hkv=4), dict(Hq=0), dict(D=64), dict(D=192)):
        assert call(**kw) == b.GDN_ESHAPE, kw
    for kw in (dict(od=7), dict(scale=0.0), dict(scale=float("inf")), dict(scale=float("nan")),
               dict(B=-1)):
        assert call(**kw) == b.GDN_EINVAL, kw
    S = b.gdn_attn_seq
    bad = [S(None, FAKE, FAKE, FAKE, 0, 4), S(FAKE + 8, FAKE, FAKE, FAKE, 0, 4),
           S(FAKE, FAKE, FAKE, FAKE, -1, 4), S(FAKE, FAKE, FAKE, FAKE, 0, -2)]
    for s in bad:
        assert call(seqs=[s]) == b.GDN_EINVAL
    # o overlapping q or the caches
    assert call(seqs=[S(FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + 256, 0, 16)]) == b.GDN_EALIAS
    assert call(seqs=[S(FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (2 << 20) + 512, 0, 16)]) \
        == b.GDN_EALIAS
    # nothing to do: empty sequences are fine with any pointers
    assert call(seqs=[S(None, None, None, None, 5, 0)]) == b.GDN_OK
    assert call(seqs=[], B=0) == b.GDN_OK


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU: asked for more it exits with a message, before touching a
    device (the layer's heads would shard with no exchange step, but that path is not built)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_algorithmic_counts():
    """The bench's algorithmic byte and flop counts at the 16/32/128 layer, T = 8192: 24,832
    bytes per token (bf16 x in, fp32 g and beta, bf16 o) plus the state and window in and out
    and the conv weights per call; 3.98 MFLOP per token."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bm = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bm)
    per_token, per_call = bm.algorithmic_bytes(8192, 16, 32, 128)
    assert per_token == 24832
    assert per_call == 8192 * 24832 + 2 * 32 * 128 * 128 * 4 + 2 * 3 * 8192 * 2 + 8192 * 4 * 2
    flops = bm.algorithmic_flops(8192, 16, 32, 128)
    assert abs(flops / 8192 / 3.98e6 - 1) < 0.01
    split = bm.kernel_bytes(8192, 16, 32, 128)
    assert split["prep_kernel"] + split["chain_kernel"] == per_call  # every byte in one kernel
