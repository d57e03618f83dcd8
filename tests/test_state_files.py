"""State files on the host: format, exact round trip, refusals, and the failed-write rule.

The pages: a session goes to disk and comes back exact, and a file made for another model or
grid is not read ("The shadow reader", sections "Memory and the disk" and "Memory"); a copy
made for other layers reads as missing, and a failed write leaves the slot missing, never
stale ("Long context and sessions", section "On disk, across reloads").  Everything here runs
through the library's host-buffer forms; no device memory is touched.
"""
import ctypes
import os
import struct

import numpy as np
import pytest

from tests import hostlib as b

WEIGHTS = 0x5EED5EED12345678


def small_desc(**kw):
    return b.make_desc(2, 4, 64, 64, **kw)


def random_state(desc, seed=0):
    r = np.random.default_rng(seed)
    S = r.standard_normal((desc.n_v_heads, desc.d_k, desc.d_v)).astype(np.float32)
    conv = r.integers(0, 1 << 16, size=(desc.conv_width - 1, desc.channels), dtype=np.uint16)
    return S, conv


def test_round_trip_is_exact_and_layout_is_as_declared(tmp_path):
    d = small_desc()
    S, conv = random_state(d, 1)
    path = str(tmp_path / "s.gdn")
    b.gdn_state_file_write(d, S, conv, 1536, WEIGHTS, path)
    S2, conv2, pos = b.gdn_state_file_read(d, WEIGHTS, path)
    assert pos == 1536
    assert np.array_equal(S.view(np.uint32), S2.view(np.uint32))
    assert np.array_equal(conv, conv2)
    raw = open(path, "rb").read()
    hb = b.gdn_state_file_header_bytes()
    assert hb == 104 and len(raw) == hb + S.nbytes + conv.nbytes
    assert raw[:8] == b"GDNSTAT1"
    version, hbytes = struct.unpack_from("<II", raw, 8)
    fields = struct.unpack_from("<8i", raw, 16)
    tag, wh, fpos, sb, cb = struct.unpack_from("<QQqQQ", raw, 48)
    assert (version, hbytes) == (1, 104)
    assert fields == (2, 4, 64, 64, 4, 64, 512, b.GDN_BF16)
    assert (tag, wh, fpos, sb, cb) == (b.gdn_desc_tag(d), WEIGHTS, 1536, S.nbytes, conv.nbytes)
    assert raw[hb:hb + S.nbytes] == S.tobytes() and raw[hb + S.nbytes:] == conv.tobytes()
    assert os.listdir(tmp_path) == ["s.gdn"]  # no temporary file left


def _read_status(desc, path, weights=WEIGHTS):
    try:
        b.gdn_state_file_read(desc, weights, path)
    except b.GdnError as e:
        return e.status
    return b.GDN_OK


def test_other_layer_grid_dtype_or_weights_is_refused(tmp_path):
    d = small_desc()
    S, conv = random_state(d, 2)
    path = str(tmp_path / "s.gdn")
    b.gdn_state_file_write(d, S, conv, 512, WEIGHTS, path)
    assert _read_status(d, path) == b.GDN_OK
    assert _read_status(small_desc(grid=2048), path) == b.GDN_EMISMATCH
    assert _read_status(b.make_desc(2, 4, 128, 128), path) == b.GDN_EMISMATCH
    assert _read_status(b.make_desc(1, 4, 64, 64), path) == b.GDN_EMISMATCH
    assert _read_status(small_desc(act_dtype="float32"), path) == b.GDN_EMISMATCH
    assert _read_status(d, path, weights=WEIGHTS + 1) == b.GDN_EMISMATCH
    # scale and eps do not change what a state means: the same file reads
    assert _read_status(small_desc(scale=0.3, l2_eps=1e-3), path) == b.GDN_OK


def test_refused_read_leaves_the_buffers(tmp_path):
    d = small_desc()
    S, conv = random_state(d, 3)
    path = str(tmp_path / "s.gdn")
    b.gdn_state_file_write(d, S, conv, 512, WEIGHTS, path)
    dst_S = np.full_like(S, 7.0)
    dst_c = np.full_like(conv, 9)
    pos = ctypes.c_int64(-3)
    st = b.lib.gdn_state_file_read(ctypes.byref(d), dst_S.ctypes.data, dst_c.ctypes.data,
                                   ctypes.byref(pos), WEIGHTS + 5, os.fsencode(path))
    assert st == b.GDN_EMISMATCH
    assert (dst_S == 7.0).all() and (dst_c == 9).all() and pos.value == -3


@pytest.mark.parametrize("damage", ["payload_byte", "pos_field", "magic", "truncate",
                                    "trailing", "empty"])
def test_damaged_file_reads_as_missing(tmp_path, damage):
    d = small_desc()
    S, conv = random_state(d, 4)
    path = str(tmp_path / "s.gdn")
    b.gdn_state_file_write(d, S, conv, 1024, WEIGHTS, path)
    raw = bytearray(open(path, "rb").read())
    if damage == "payload_byte":
        raw[200] ^= 0x01
    elif damage == "pos_field":
        raw[64] ^= 0x40  # pos: caught by the header checksum
    elif damage == "magic":
        raw[0] = ord("X")
    elif damage == "truncate":
        raw = raw[:-5]
    elif damage == "trailing":
        raw += b"\0"
    else:
        raw = bytearray()
    open(path, "wb").write(bytes(raw))
    assert _read_status(d, path) == b.GDN_EFILE


def test_missing_file(tmp_path):
    assert _read_status(small_desc(), str(tmp_path / "nope.gdn")) == b.GDN_EFILE


def test_failed_write_leaves_no_file_never_a_stale_one(tmp_path):
    d = small_desc()
    S, conv = random_state(d, 5)
    path = str(tmp_path / "s.gdn")
    b.gdn_state_file_write(d, S, conv, 512, WEIGHTS, path)  # an older save of the session
    # make the next write fail: its temporary file name is taken by a directory
    os.mkdir(path + ".tmp.%d" % os.getpid())
    S2, conv2 = random_state(d, 6)
    with pytest.raises(b.GdnError) as e:
        b.gdn_state_file_write(d, S2, conv2, 1024, WEIGHTS, path)
    assert e.value.status == b.GDN_EFILE
    assert not os.path.exists(path)  # missing, not the stale older save
    os.rmdir(path + ".tmp.%d" % os.getpid())
    # a write into a directory that does not exist fails the same way
    with pytest.raises(b.GdnError):
        b.gdn_state_file_write(d, S2, conv2, 1024, WEIGHTS, str(tmp_path / "no" / "s.gdn"))


def test_rewrite_replaces_the_session(tmp_path):
    d = small_desc()
    path = str(tmp_path / "s.gdn")
    for i, pos in enumerate((512, 1024, 4096)):
        S, conv = random_state(d, 10 + i)
        b.gdn_state_file_write(d, S, conv, pos, WEIGHTS, path)
        S2, conv2, p2 = b.gdn_state_file_read(d, WEIGHTS, path)
        assert p2 == pos and np.array_equal(S, S2) and np.array_equal(conv, conv2)
    assert os.listdir(tmp_path) == ["s.gdn"]


def test_no_conv_layer_and_argument_checks(tmp_path):
    d = b.make_desc(1, 1, 64, 64, conv_width=0, act_dtype="float32")
    S = np.arange(64 * 64, dtype=np.float32).reshape(1, 64, 64)
    path = str(tmp_path / "one.gdn")
    b.gdn_state_file_write(d, S, None, 0, 0, path)
    S2, conv2, pos = b.gdn_state_file_read(d, 0, path)
    assert conv2 is None and pos == 0 and np.array_equal(S, S2)
    assert os.path.getsize(path) == 104 + S.nbytes
    with pytest.raises(b.GdnError) as e:
        b.gdn_state_file_write(d, S, None, -1, 0, path)
    assert e.value.status == b.GDN_EINVAL
    assert b.lib.gdn_state_file_write(ctypes.byref(d), S.ctypes.data, None, 0, 0, None) == b.GDN_EINVAL
    d4 = small_desc()
    assert b.lib.gdn_state_file_write(ctypes.byref(d4), S.ctypes.data, None, 0, 0,
                                      os.fsencode(path)) == b.GDN_EINVAL  # window required
