"""Property-based tests of the library's host logic (no device): the commit-grid and
shared-prefix row counts, the checkpoint ring against a plain model of its documented rules,
state-file damage detection, and workspace sizing.

- A COMMIT absorbs whole grid chunks only, and a shared prefix runs up to its last multiple
  of 64 ("The shadow reader", section "Exact on a grid"; PR "qwen3_5: run prompts that share
  prefixes once per prefix", section Purpose).
- At most six checkpoints; a restore takes the newest at or below the divergence; those above
  it are forgotten ("The shadow reader", section "One session's state").
- A damaged or short state file reads as missing ("Long context and sessions", section "On
  disk, across reloads").
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tests import hostlib as b

SETTINGS = settings(max_examples=300, deadline=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])


@SETTINGS
@given(n=st.integers(0, 1 << 40), k=st.integers(1, 256))
def test_commit_rows_are_whole_chunks(n, k):
    grid = 64 * k
    r = b.gdn_commit_rows(n, grid)
    assert r % grid == 0 and 0 <= r <= n and n - r < grid


@SETTINGS
@given(n=st.integers(-(1 << 20), -1), grid=st.integers(-4096, 0))
def test_commit_rows_refuses_bad_arguments(n, grid):
    assert b.gdn_commit_rows(n, 512) == -1
    assert b.gdn_commit_rows(100, grid) == -1


@SETTINGS
@given(s=st.integers(0, 1 << 24), extra=st.integers(0, 1 << 20))
def test_shared_prefix_rows(s, extra):
    state_pos = 64 * s
    end = state_pos + extra
    run = b.gdn_shared_prefix_rows(state_pos, end)
    # runs whole sub-chunks from the state, never past the prefix, leaving less than 64 rows
    assert run >= 0 and run % 64 == 0 and state_pos + run <= end
    assert end - (state_pos + run) < 64
    # and the rows it runs end at an absolute multiple of 64
    assert (state_pos + run) % 64 == 0


@SETTINGS
@given(s=st.integers(0, 1 << 20), off=st.integers(1, 63), back=st.integers(1, 1000))
def test_shared_prefix_rows_refuses_bad_arguments(s, off, back):
    assert b.gdn_shared_prefix_rows(64 * s + off, 64 * s + 1000) == -1  # unaligned state
    assert b.gdn_shared_prefix_rows(64 * s + 64 * back, 64 * s) == -1  # prefix behind the state


class RingModel:
    """The ring's documented rules: the slot already holding pos, else the lowest empty slot,
    else the slot pushed longest ago; find = the largest pos <= d; drop = forget pos > d."""

    def __init__(self, cap):
        self.cap = cap
        self.pos = [-1] * cap
        self.stamp = [0] * cap
        self.clock = 0

    def push(self, p):
        if p in self.pos[:self.cap]:
            s = self.pos.index(p)
        elif -1 in self.pos:
            s = self.pos.index(-1)
        else:
            s = min(range(self.cap), key=lambda i: self.stamp[i])
        self.pos[s] = p
        self.clock += 1
        self.stamp[s] = self.clock
        return s

    def find(self, d):
        live = [(p, i) for i, p in enumerate(self.pos) if 0 <= p <= d]
        return max(live)[1] if live else -1

    def drop(self, d):
        n = 0
        for i, p in enumerate(self.pos):
            if p >= 0 and p > d:
                self.pos[i], self.stamp[i] = -1, 0
                n += 1
        return n


ops = st.lists(st.one_of(
    st.tuples(st.just("push"), st.integers(0, 40).map(lambda k: 512 * k)),
    st.tuples(st.just("find"), st.integers(-10, 21000)),
    st.tuples(st.just("drop"), st.integers(-10, 21000))), max_size=60)


@SETTINGS
@given(cap=st.integers(1, b.MAX_CHECKPOINTS), seq=ops)
def test_checkpoint_ring_follows_its_rules(cap, seq):
    ring, model = b.CkptRing(cap), RingModel(cap)
    for op, v in seq:
        if op == "push":
            assert ring.push(v) == model.push(v)
        elif op == "find":
            assert ring.find(v) == model.find(v)
        else:
            assert ring.drop_above(v) == model.drop(v)
        assert ring.positions() == model.pos
        assert ring.c.n == sum(p >= 0 for p in model.pos)


def _state_file(tmp_path, seed):
    d = b.make_desc(2, 4, 64, 64)
    r = np.random.default_rng(seed)
    S = r.standard_normal((d.n_v_heads, d.d_k, d.d_v)).astype(np.float32)
    conv = r.integers(0, 1 << 16, size=(d.conv_width - 1, d.channels), dtype=np.uint16)
    path = str(tmp_path / ("s%d.gdn" % seed))
    b.gdn_state_file_write(d, S, conv, 512 * (seed % 50), 0xABCDEF, path)
    return d, path


@settings(max_examples=150, deadline=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(seed=st.integers(0, 3), where=st.floats(0, 1, exclude_max=True), bit=st.integers(0, 7))
def test_any_flipped_bit_reads_as_missing_or_mismatch(tmp_path, seed, where, bit):
    d, path = _state_file(tmp_path, seed)
    raw = bytearray(open(path, "rb").read())
    i = int(where * len(raw))
    raw[i] ^= 1 << bit
    open(path, "wb").write(bytes(raw))
    with pytest.raises(b.GdnError) as e:
        b.gdn_state_file_read(d, 0xABCDEF, path)
    assert e.value.status in (b.GDN_EFILE, b.GDN_EMISMATCH)


@settings(max_examples=100, deadline=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(seed=st.integers(0, 3), keep=st.floats(0, 1, exclude_max=True))
def test_short_file_reads_as_missing(tmp_path, seed, keep):
    d, path = _state_file(tmp_path, seed)
    raw = open(path, "rb").read()
    open(path, "wb").write(raw[:int(keep * len(raw))])
    with pytest.raises(b.GdnError) as e:
        b.gdn_state_file_read(d, 0xABCDEF, path)
    assert e.value.status == b.GDN_EFILE


@SETTINGS
@given(rows=st.integers(0, 1 << 22), more=st.integers(0, 1 << 16), segs=st.integers(1, 64),
       d=st.sampled_from([64, 128]), ratio=st.sampled_from([1, 2, 4]))
def test_workspace_grows_with_rows_and_segments(rows, more, segs, d, ratio):
    desc = b.make_desc(4, 4 * ratio, d, d)
    w = b.gdn_workspace_bytes(desc, rows, segs)
    assert w > 0
    assert b.gdn_workspace_bytes(desc, rows + more, segs) >= w
    assert b.gdn_workspace_bytes(desc, rows, segs + 1) >= w


def _desc_ok(f):
    """The descriptor rules the library documents."""
    import math
    nk, nv, dk, dv, cw, sc, grid, act, out, silu, scale, eps = f
    if min(nk, nv, dk, dv) <= 0 or act not in (0, 1) or out not in (0, 1) or silu not in (0, 1):
        return False
    if not (math.isfinite(eps) and eps >= 0 and math.isfinite(scale)):
        return False
    if nv % nk or dk != dv or dk not in (64, 128) or cw not in (0, 4) or sc != 64:
        return False
    if grid <= 0 or grid % 64:
        return False
    return 2 * nk * dk + nv * dv <= 1 << 24


small = st.one_of(st.integers(-3, 300), st.sampled_from([-(1 << 31), (1 << 31) - 1, 1 << 20]))
f32 = st.floats(width=32, allow_nan=True, allow_infinity=True)


@SETTINGS
@given(nk=small, nv=small, dk=st.sampled_from([-1, 0, 32, 64, 100, 128, 256]),
       dv=st.sampled_from([0, 64, 128, 256]), cw=st.integers(-1, 5), sc=st.sampled_from([0, 32, 64, 128]),
       grid=st.sampled_from([-512, 0, 1, 64, 100, 512, 2048, 1 << 20]), act=st.integers(-1, 2),
       out=st.integers(-1, 2), silu=st.integers(-1, 2), scale=f32, eps=f32)
def test_descriptor_check_matches_its_rules(nk, nv, dk, dv, cw, sc, grid, act, out, silu, scale, eps):
    f = (nk, nv, dk, dv, cw, sc, grid, act, out, silu, scale, eps)
    d = b.gdn_desc(*f)
    ok = b.gdn_desc_check(d) == b.GDN_OK
    assert ok == _desc_ok(f)
    # the size queries answer only for valid descriptors
    assert (b.gdn_state_S_bytes(d) > 0) == ok
    assert (b.gdn_workspace_bytes(d, 1024, 1) > 0) == ok
