"""The host half's launch plan and state operations, run for real on the CPU.

The host-only build (tests/hostlib.py) records each kernel launch instead of running it and
treats "device" pointers as host memory, so these tests check what the library would enqueue
(sequences, rows, sub-chunks, which state each launch reads and writes) and run the state
copies on host buffers.
"""
import ctypes
import os

import numpy as np
import pytest

from tests import hostlib as b

FAKE = 0x7F0000000000  # inputs the recording launchers never dereference
X_, W_, G_, B_, O_ = (FAKE + (k << 30) for k in (10, 11, 12, 13, 14))


def layer_desc(**kw):
    return b.make_desc(16, 32, 128, 128, **kw)


HostState = b.HostState


def _fork(d, sin, sout, T, ws_bytes=None, ws=FAKE + (2 << 30)):
    rows = ctypes.c_int64(-1)
    ws_bytes = b.gdn_workspace_bytes(d, T, 1) if ws_bytes is None else ws_bytes
    st = b.lib.gdn_prefill_chunked(ctypes.byref(d), X_, W_, G_, B_, sin.ref(), sout.ref(), O_, T,
                                   b.GDN_FORK, ctypes.byref(rows), ws, ws_bytes, None)
    return st, rows.value


def test_one_call_is_one_launch_of_all_sub_chunks():
    d = layer_desc()
    sin, sout = HostState(d), HostState(d)
    b.reset()
    st, rows = _fork(d, sin, sout, 1000)
    assert st == b.GDN_OK and rows == 1000 and sout.c.pos == 1000
    (kind, n_sub, segs), = b.launches()
    assert kind == b.KIND_PREFILL and n_sub == 16
    assert segs == [dict(row0=0, n=1000, sub0=0, S_in=sin.S.ctypes.data, win_in=sin.conv.ctypes.data,
                         S_out=sout.S.ctypes.data, win_out=sout.conv.ctypes.data)]


def test_calls_that_absorb_no_rows_copy_the_state_and_launch_nothing():
    """A FORK of zero rows, and a COMMIT of fewer rows than the grid (the whole call is the
    pending tail), absorb nothing: they enqueue no kernel, touch no input pointer (the inputs
    may even be null), and leave the output state equal to the input state, copied bit for bit
    when they are distinct buffers."""
    d = layer_desc()
    live = HostState(d, fill=True, seed=3)
    live.c.pos = 1024
    for mode, T in ((b.GDN_FORK, 0), (b.GDN_COMMIT, 0), (b.GDN_COMMIT, 511)):
        out = HostState(d, fill=True, seed=4)
        b.reset()
        rows = ctypes.c_int64(-1)
        st = b.lib.gdn_prefill_chunked(ctypes.byref(d), None, None, None, None, live.ref(),
                                       out.ref(), None, T, mode, ctypes.byref(rows), None, 0, None)
        assert st == b.GDN_OK and rows.value == 0, (mode, T, st)
        assert [k for k, _, _ in b.launches() if k == b.KIND_PREFILL] == []
        assert np.array_equal(out.S.view(np.int32), live.S.view(np.int32))
        assert np.array_equal(out.conv, live.conv)
        assert out.c.pos == 1024 and out.c.tag == live.c.tag
    # in place: a commit of a pending tail only leaves the state as it was
    before = live.S.copy()
    rows = ctypes.c_int64(-1)
    assert b.lib.gdn_prefill_chunked(ctypes.byref(d), None, None, None, None, live.ref(), live.ref(),
                                     None, 300, b.GDN_COMMIT, ctypes.byref(rows), None, 0,
                                     None) == b.GDN_OK
    assert rows.value == 0 and live.c.pos == 1024 and np.array_equal(live.S, before)


@pytest.mark.parametrize("cap,T", [(256, 1000), (64, 200), (512, 1024)])
def test_long_sequence_runs_as_chained_launches(monkeypatch, cap, T):
    """A sequence longer than the per-launch row cap runs as launches that each start at a
    multiple of 64 and continue from the output state: the first reads the entry state, every
    later one the output state the previous launch wrote."""
    d = layer_desc()
    sin, sout = HostState(d), HostState(d)
    monkeypatch.setenv("GDN_TEST_LAUNCH_ROWS", str(cap))
    b.reset()
    st, rows = _fork(d, sin, sout, T, ws_bytes=b.gdn_workspace_bytes(d, cap, 1))
    assert st == b.GDN_OK and rows == T
    ls = b.launches()
    assert len(ls) == (T + cap - 1) // cap
    for i, (kind, n_sub, segs) in enumerate(ls):
        (s,) = segs
        assert kind == b.KIND_PREFILL and s["row0"] == i * cap and s["n"] == min(cap, T - i * cap)
        assert s["S_in"] == (sin if i == 0 else sout).S.ctypes.data
        assert s["win_in"] == (sin if i == 0 else sout).conv.ctypes.data
        assert s["S_out"] == sout.S.ctypes.data and s["win_out"] == sout.conv.ctypes.data
        assert n_sub == (s["n"] + 63) // 64


def test_launch_row_cap_override_only_lowers_and_needs_multiples_of_64(monkeypatch):
    d = layer_desc()
    sin, sout = HostState(d), HostState(d)
    for bad in ("100", "-64", "abc", "0", str(1 << 40)):
        monkeypatch.setenv("GDN_TEST_LAUNCH_ROWS", bad)
        b.reset()
        assert _fork(d, sin, sout, 1000)[0] == b.GDN_OK
        assert len(b.launches()) == 1, bad


def test_channel_count_too_wide_for_one_sub_chunk_per_launch_is_refused():
    """x and o are addressed with 32-bit offsets per launch; a layer whose 64 rows overflow them
    is refused up front (it would otherwise never finish its launch loop)."""
    d = b.make_desc(32768, 32768, 128, 128, act_dtype="float32", out_dtype="float32")
    assert b.gdn_desc_check(d) == b.GDN_ESHAPE
    assert b.gdn_desc_check(b.make_desc(16384, 16384, 128, 128, act_dtype="float32")) == b.GDN_OK


@pytest.mark.parametrize("B,rows", [(1, 64), (8, 64), (32, 64), (4, 200), (40, 70)])
def test_branches_without_final_states_fit_the_documented_workspace(B, rows):
    """gdn_workspace_bytes(desc, total rows, B) covers the scratch final states a branch batch
    writes when it is given no output states."""
    d = layer_desc()
    init = HostState(d)
    init.c.pos = 960
    cu = (ctypes.c_int64 * (B + 1))(*[i * rows for i in range(B + 1)])
    ia = (ctypes.POINTER(b.gdn_state) * B)(*[ctypes.pointer(init.c)] * B)
    need = b.gdn_workspace_bytes(d, B * rows, B)
    b.reset()
    st = b.lib.gdn_prefill_branches(ctypes.byref(d), B, cu, X_, W_, G_, B_, ia, None, O_,
                                    FAKE + (2 << 30), need, None)
    assert st == b.GDN_OK, b.gdn_status_str(st)
    ls = b.launches()
    assert len(ls) == (B + 31) // 32
    outs = [s["S_out"] for _, _, segs in ls for s in segs]
    ws0, ws1 = FAKE + (2 << 30), FAKE + (2 << 30) + need
    assert all(ws0 <= p < ws1 for p in outs) and len(set(outs)) == min(B, 32)
    # one byte short is refused before any launch
    b.reset()
    st = b.lib.gdn_prefill_branches(ctypes.byref(d), B, cu, X_, W_, G_, B_, ia, None, O_,
                                    FAKE + (2 << 30), need - 1, None)
    assert st in (b.GDN_OK, b.GDN_EWORKSPACE)
    if st == b.GDN_EWORKSPACE:
        assert b.launches() == []


def _misaligned(d, which):
    s = HostState(d)
    buf = np.zeros(s.S.size + 8, dtype=np.float32)
    cbuf = np.zeros(s.conv.size + 16, dtype=np.uint16)
    S_p, c_p = s.S.ctypes.data, s.conv.ctypes.data
    if which == "S":
        S_p = buf.ctypes.data + 2
    else:
        c_p = cbuf.ctypes.data + 8
    s.c = b.gdn_state(S_p, c_p, 0, b.gdn_desc_tag(d))
    s._keep = (buf, cbuf)
    return s


@pytest.mark.parametrize("which", ["S", "conv"])
def test_state_operations_refuse_misaligned_destinations(which):
    d = layer_desc()
    src = HostState(d, fill=True)
    dst = _misaligned(d, which)
    before = (dst.c.pos, dst.c.tag)
    assert b.lib.gdn_state_init(ctypes.byref(d), dst.ref(), None) == b.GDN_EINVAL
    assert b.lib.gdn_state_capture(ctypes.byref(d), src.ref(), dst.ref(), None) == b.GDN_EINVAL
    assert b.lib.gdn_state_restore(ctypes.byref(d), dst.ref(), src.ref(), None) == b.GDN_EINVAL
    arr = (b.gdn_state * 1)(dst.c)
    assert b.lib.gdn_state_fork(ctypes.byref(d), src.ref(), arr, 1, None) == b.GDN_EINVAL
    assert (dst.c.pos, dst.c.tag) == before


def test_state_operations_on_host_memory():
    """init zeroes; capture, restore and fork copy S, the window, pos and tag bit for bit."""
    d = layer_desc()
    live = HostState(d, fill=True, seed=1)
    live.c.pos = 1536
    snap, other = HostState(d), HostState(d, fill=True, seed=2)
    assert b.lib.gdn_state_capture(ctypes.byref(d), live.ref(), snap.ref(), None) == b.GDN_OK
    assert np.array_equal(snap.S.view(np.int32), live.S.view(np.int32))
    assert np.array_equal(snap.conv, live.conv) and snap.c.pos == 1536
    assert b.lib.gdn_state_restore(ctypes.byref(d), other.ref(), snap.ref(), None) == b.GDN_OK
    assert np.array_equal(other.S.view(np.int32), live.S.view(np.int32)) and other.c.pos == 1536
    outs = [HostState(d) for _ in range(3)]
    arr = (b.gdn_state * 3)(*[o.c for o in outs])
    assert b.lib.gdn_state_fork(ctypes.byref(d), live.ref(), arr, 3, None) == b.GDN_OK
    for i, o in enumerate(outs):
        assert np.array_equal(o.S, live.S) and np.array_equal(o.conv, live.conv)
        assert arr[i].pos == 1536
    assert b.lib.gdn_state_init(ctypes.byref(d), live.ref(), None) == b.GDN_OK
    assert not live.S.any() and not live.conv.any() and live.c.pos == 0


def test_state_save_and_load_through_files(tmp_path):
    d = layer_desc()
    live = HostState(d, fill=True, seed=3)
    live.c.pos = 4096
    path = os.fsencode(str(tmp_path / "s.gdn"))
    assert b.lib.gdn_state_save(ctypes.byref(d), live.ref(), 77, path, None) == b.GDN_OK
    back = HostState(d)
    back.c.tag = 0
    assert b.lib.gdn_state_load(ctypes.byref(d), back.ref(), 78, path, None) == b.GDN_EMISMATCH
    assert not back.S.any() and back.c.pos == 0
    assert b.lib.gdn_state_load(ctypes.byref(d), back.ref(), 77, path, None) == b.GDN_OK
    assert np.array_equal(back.S.view(np.int32), live.S.view(np.int32))
    assert np.array_equal(back.conv, live.conv)
    assert back.c.pos == 4096 and back.c.tag == b.gdn_desc_tag(d)
