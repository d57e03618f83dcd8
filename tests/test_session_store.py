"""The session store (gdn_store_*) on the CPU: least recently used sessions leave their slots
for files and come back exactly; without a disk they are dropped and start over ("The shadow
reader", section "Memory and the disk"; "Long context and sessions", section "Sessions on one
engine").  Slots are host-memory states here (tests/hostlib.py), so every copy and file write
runs for real."""
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tests import hostlib as b

D = b.make_desc(2, 4, 64, 64)  # a small layer: 64 KiB of S and a 3 x 512 window


def state_bytes():
    return b.gdn_state_S_bytes(D) + b.gdn_state_conv_bytes(D)


def make_store(n_slots=2, cap_states=2.0, directory=None, weights_hash=7, max_entries=None):
    slots = [b.HostState(D) for _ in range(n_slots)]
    s = b.abi.Store(b.lib, D, slots, int(cap_states * state_bytes()), directory, weights_hash,
                    max_entries)
    assert s.status == b.GDN_OK
    return s


def acquire(s, sid):
    st, slot, origin = s.acquire(sid)
    assert st == b.GDN_OK, b.gdn_status_str(st)
    return slot, origin


def feed(slot, seed, rows=512):
    """Stands in for a commit into the slot: new contents and a later position."""
    r = np.random.default_rng(seed)
    slot.S[:] = r.standard_normal(slot.S.shape)
    slot.conv[:] = r.integers(0, 1 << 16, slot.conv.shape)
    slot.c.pos += rows
    return slot.S.copy(), slot.conv.copy(), slot.c.pos


def test_least_recently_used_goes_to_disk_and_comes_back_exact(tmp_path):
    s = make_store(directory=str(tmp_path))
    a, o = acquire(s, 1)
    assert o == b.GDN_STORE_FRESH and a.pos == 0 and not a.S.any()
    snap_a = feed(a, 10)
    bb, o = acquire(s, 2)
    assert o == b.GDN_STORE_FRESH
    snap_b = feed(bb, 11, rows=1024)
    c, o = acquire(s, 3)  # no free slot: session 1 (least recently used) is written out
    assert o == b.GDN_STORE_FRESH and c is a
    assert s.entry(1)["where"] == b.GDN_STORE_ON_DISK and s.entry(1)["pos"] == 512
    assert os.path.exists(tmp_path / ("gdn-%016x.state" % 1))
    assert s.resident() == [2, 3]
    _, o = acquire(s, 2)
    assert o == b.GDN_STORE_WAS_RESIDENT
    a2, o = acquire(s, 1)  # session 3 is now the least recently used
    assert o == b.GDN_STORE_FROM_DISK and s.entry(3)["where"] == b.GDN_STORE_ON_DISK
    assert np.array_equal(a2.S.view(np.int32), snap_a[0].view(np.int32))
    assert np.array_equal(a2.conv, snap_a[1]) and a2.pos == snap_a[2] == 512
    b2, o = acquire(s, 2)
    assert o == b.GDN_STORE_WAS_RESIDENT and np.array_equal(b2.S, snap_b[0]) and b2.pos == 1024


def test_cap_bounds_the_resident_sessions(tmp_path):
    s = make_store(n_slots=4, cap_states=2.5, directory=str(tmp_path))
    assert s.c.max_resident == 2 and s.c.state_bytes == state_bytes()
    for sid in range(1, 9):
        acquire(s, sid)
        assert len(s.resident()) <= 2
    assert s.resident() == [7, 8]
    on_disk = [sid for sid in range(1, 7) if s.entry(sid)["where"] == b.GDN_STORE_ON_DISK]
    assert on_disk == [1, 2, 3, 4, 5, 6]


def test_without_a_disk_an_evicted_session_is_dropped_and_starts_over():
    s = make_store(directory=None)
    a, _ = acquire(s, 1)
    feed(a, 20)
    acquire(s, 2)
    acquire(s, 3)
    assert s.entry(1)["where"] == b.GDN_STORE_DROPPED
    a2, o = acquire(s, 1)
    assert o == b.GDN_STORE_FRESH and a2.pos == 0 and not a2.S.any() and not a2.conv.any()


@pytest.mark.parametrize("damage", ["truncate", "flip", "weights", "remove"])
def test_unreadable_or_foreign_file_reads_as_fresh(tmp_path, damage):
    s = make_store(directory=str(tmp_path))
    a, _ = acquire(s, 1)
    feed(a, 30)
    assert s.evict(1) == b.GDN_OK and s.entry(1)["where"] == b.GDN_STORE_ON_DISK
    path = tmp_path / ("gdn-%016x.state" % 1)
    raw = path.read_bytes()
    if damage == "truncate":
        path.write_bytes(raw[:-100])
    elif damage == "flip":
        path.write_bytes(raw[:200] + bytes([raw[200] ^ 1]) + raw[201:])
    elif damage == "remove":
        path.unlink()
    else:  # the same directory read by a store for other weights
        s = make_store(directory=str(tmp_path), weights_hash=8)
        # the new store does not know the session: teach it by evicting a fresh one of the id
        acquire(s, 1)
        assert s.evict(1) == b.GDN_OK
        path.write_bytes(raw)  # the file written for the other weights
    a2, o = acquire(s, 1)
    assert o == b.GDN_STORE_FRESH and a2.pos == 0 and not a2.S.any()
    assert not path.exists()


def test_flush_writes_every_resident_session_and_drop_forgets(tmp_path):
    s = make_store(directory=str(tmp_path))
    a, _ = acquire(s, 5)
    snap = feed(a, 40)
    acquire(s, 6)
    assert s.flush() == b.GDN_OK
    assert s.resident() == [5, 6]
    for sid in (5, 6):
        assert os.path.exists(tmp_path / ("gdn-%016x.state" % sid))
    # the flushed file of session 5 reads back into a new store exactly
    s2 = make_store(directory=str(tmp_path))
    # s2 learns of the session through an eviction record: evict a fresh one, then restore file
    path = tmp_path / ("gdn-%016x.state" % 5)
    raw = path.read_bytes()
    acquire(s2, 5)
    s2.evict(5)
    path.write_bytes(raw)
    a2, o = acquire(s2, 5)
    assert o == b.GDN_STORE_FROM_DISK and np.array_equal(a2.S, snap[0]) and a2.pos == snap[2]
    assert s.drop(5) == b.GDN_OK and s.entry(5) is None and not path.exists()
    assert s.resident() == [6]


def test_refusals():
    slots = [b.HostState(D) for _ in range(2)]
    bad = b.abi.Store(b.lib, D, slots, state_bytes() - 1)  # the cap holds no state
    assert bad.status == b.GDN_EINVAL
    bad = b.abi.Store(b.lib, D, slots, 10 * state_bytes(), max_entries=1)
    assert bad.status == b.GDN_EINVAL
    bad = b.abi.Store(b.lib, D, slots, 10 * state_bytes(), directory="x" * 600)
    assert bad.status == b.GDN_EINVAL
    s = make_store()
    assert s.evict(99) == b.GDN_EINVAL


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(n_slots=st.integers(1, 4), cap=st.integers(1, 5), disk=st.booleans(),
       seq=st.lists(st.integers(1, 7), min_size=1, max_size=40))
def test_store_follows_least_recently_used(tmp_path_factory, n_slots, cap, disk, seq):
    """Against a plain model of the rules: at most min(slots, cap) resident; a miss evicts the
    least recently used resident session (to disk, or dropped); a session comes back with the
    bytes and position it left with, or fresh when it was dropped."""
    d = str(tmp_path_factory.mktemp("store")) if disk else None
    s = make_store(n_slots=n_slots, cap_states=cap + 0.5, directory=d, max_entries=16)
    limit = min(n_slots, cap)
    resident, stamp, saved, clock = [], {}, {}, 0
    for i, sid in enumerate(seq):
        slot, origin = acquire(s, sid)
        clock += 1
        if sid in resident:
            assert origin == b.GDN_STORE_WAS_RESIDENT
        else:
            if len(resident) == limit:
                victim = min(resident, key=lambda k: stamp[k])
                resident.remove(victim)
                if not disk:
                    saved.pop(victim, None)
            if sid in saved:
                assert origin == b.GDN_STORE_FROM_DISK
                S, pos = saved[sid]
                assert np.array_equal(slot.S, S) and slot.pos == pos
            else:
                assert origin == b.GDN_STORE_FRESH and slot.pos == 0 and not slot.S.any()
            resident.append(sid)
        stamp[sid] = clock
        S, _, pos = feed(slot, 1000 + i, rows=64)
        saved[sid] = (S, pos)
        assert sorted(resident) == s.resident()
