"""Grid-exact commit, fork, branches and state copies on the GPU, through the C ABI.

The pages' criteria: a turn-by-turn replay equals a fresh prefill on the same grid bit for
bit and a fork leaves everything below the committed length unchanged ("The shadow reader",
section "Exact on a grid"); a branch continued from a shared prefix state equals a plain pass
over its full prompt bit for bit (PR "qwen3_5: run prompts that share prefixes once per
prefix", sections Purpose and "Test Result"); states for another layer are refused and slot
copies are exact ("Long context and sessions", section "Sessions on one engine").
"""
import numpy as np
import pytest
import torch

from hybrid_linear_attention_prefill_amd import synth
from tests.helpers import assert_parity, new_state, oracle, run_fork, same_bits, to_dev

pytestmark = pytest.mark.gpu

SHAPE = synth.LAYER_16x32x128


@pytest.fixture(scope="module")
def b():
    from hybrid_linear_attention_prefill_amd import binding
    assert torch.cuda.is_available()
    return binding


@pytest.fixture(scope="module")
def desc(b):
    return b.make_desc(16, 32, 128, 128, conv_width=4, grid=512)


def _commit(b, desc, dinp, state, r0, r1, ws):
    T = r1 - r0
    o = torch.empty((T, desc.n_v_heads, desc.d_v), dtype=desc.out_torch, device="cuda")
    n = b.gdn_prefill_chunked(desc, dinp["x"][r0:r1], dinp["conv_w"], dinp["g"][r0:r1],
                              dinp["beta"][r0:r1], state, state, o, T, b.GDN_COMMIT, ws)
    return n, o[:n]


def test_commit_rows_and_pending_tail(b, desc):
    dinp = to_dev(synth.layer_inputs(SHAPE, 1300, seed=10))
    ws = b.workspace(desc, 1300)
    s = new_state(b, desc)
    n, _ = _commit(b, desc, dinp, s, 0, 1300, ws)
    assert n == 1024 and s.pos == 1024
    n, _ = _commit(b, desc, dinp, s, 1024, 1300, ws)  # 276 < 512: nothing absorbed
    assert n == 0 and s.pos == 1024


def test_replay_equals_fresh_bitwise(b, desc):
    """Turns of random length; after each, COMMIT whole 512-chunks; the pending tail waits.
    The committed state equals a fresh one-call COMMIT of the committed prefix, bit for bit."""
    total = 5000
    inp = synth.layer_inputs(SHAPE, total, seed=11)
    dinp = to_dev(inp)
    ws = b.workspace(desc, total)
    cuts = synth.turn_cuts(11, total, 6)
    live = new_state(b, desc)
    committed, outs = 0, []
    for end in cuts:
        n, o = _commit(b, desc, dinp, live, committed, end, ws)
        outs.append(o.clone())
        committed += n
        assert live.pos == committed and committed % 512 == 0
        fresh = new_state(b, desc)
        n2, o2 = _commit(b, desc, dinp, fresh, 0, committed, ws)
        torch.cuda.synchronize()
        assert n2 == committed
        assert same_bits(live.S, fresh.S) and same_bits(live.conv, fresh.conv)
        assert same_bits(torch.cat(outs), o2)


def test_fork_leaves_state_unchanged_and_matches_oracle(b, desc):
    total = 1100
    inp = synth.layer_inputs(SHAPE, total, seed=12)
    dinp = to_dev(inp)
    ws = b.workspace(desc, total)
    live = new_state(b, desc)
    n, _ = _commit(b, desc, dinp, live, 0, total, ws)
    assert n == 1024
    S_before, W_before = live.S.clone(), live.conv.clone()
    fork = b.State(desc)
    o, fork = run_fork(b, desc, dinp, live, rows=(1024, total), out_state=fork, ws=ws)
    torch.cuda.synchronize()
    assert same_bits(live.S, S_before) and same_bits(live.conv, W_before) and live.pos == 1024
    assert fork.pos == total
    # fork rows equal the oracle continued from the committed state
    part = {k: v[1024:total] for k, v in inp.items() if k != "conv_w"}
    part["conv_w"] = inp["conv_w"]
    o_ref, S_ref, _ = oracle(desc, part, S0=live.S.cpu().numpy().astype(np.float64),
                             window=synth.f64(live.conv))
    assert_parity(o, fork.S, o_ref, S_ref, label="fork")
    # and bitwise equal to one FORK over the whole prefix from zero (same 64-row grid)
    o_all, s_all = run_fork(b, desc, dinp, new_state(b, desc), ws=ws)
    torch.cuda.synchronize()
    assert same_bits(o_all[1024:], o) and same_bits(s_all.S, fork.S)


def test_split_at_multiples_of_64_bitwise(b, desc):
    dinp = to_dev(synth.layer_inputs(SHAPE, 777, seed=13))
    ws = b.workspace(desc, 777)
    o_all, s_all = run_fork(b, desc, dinp, new_state(b, desc), ws=ws)
    s = new_state(b, desc)
    parts = []
    for r0, r1 in [(0, 64), (64, 320), (320, 704), (704, 777)]:
        o, s = run_fork(b, desc, dinp, s, rows=(r0, r1), ws=ws)
        parts.append(o)
    torch.cuda.synchronize()
    assert same_bits(torch.cat(parts), o_all) and same_bits(s.S, s_all.S)
    assert same_bits(s.conv, s_all.conv)


def test_grid_512_equals_grid_2048(b):
    """The only arithmetic boundary is the multiple of 64, so two commit grids agree."""
    d512 = b.make_desc(16, 32, 128, 128, grid=512)
    d2048 = b.make_desc(16, 32, 128, 128, grid=2048)
    dinp = to_dev(synth.layer_inputs(SHAPE, 4096, seed=14))
    ws = b.workspace(d512, 4096)
    a = new_state(b, d512)
    for r0 in range(0, 4096, 512):
        _commit(b, d512, dinp, a, r0, r0 + 512, ws)
    c = new_state(b, d2048)
    _commit(b, d2048, dinp, c, 0, 4096, ws)
    torch.cuda.synchronize()
    assert same_bits(a.S, c.S) and same_bits(a.conv, c.conv)


def test_capture_restore_roundtrip_and_tag_refusal(b, desc):
    dinp = to_dev(synth.layer_inputs(SHAPE, 600, seed=15))
    ws = b.workspace(desc, 600)
    live = new_state(b, desc)
    _commit(b, desc, dinp, live, 0, 600, ws)
    snap = b.State(desc)
    b.gdn_state_capture(desc, live, snap)
    S0, W0 = live.S.clone(), live.conv.clone()
    run_fork(b, desc, dinp, live, rows=(512, 600), ws=ws)        # does not touch live
    live.S.add_(1.0)                                              # scribble on live
    b.gdn_state_restore(desc, live, snap)
    torch.cuda.synchronize()
    assert same_bits(live.S, S0) and same_bits(live.conv, W0) and live.pos == 512
    other = b.make_desc(16, 32, 128, 128, grid=1024)
    bad = new_state(b, other)
    with pytest.raises(b.GdnError) as e:
        b.gdn_state_restore(desc, live, bad)
    assert e.value.status == b.GDN_EMISMATCH
    torch.cuda.synchronize()
    assert same_bits(live.S, S0)


def test_interleaved_sessions_equal_uninterrupted(b, desc):
    """Three sessions time-share one live state through slot copies."""
    n_sess, turns = 3, 3
    inps = [to_dev(synth.layer_inputs(SHAPE, 512 * turns, seed=20 + i)) for i in range(n_sess)]
    ws = b.workspace(desc, 512)
    ref = []
    for i in range(n_sess):
        s = new_state(b, desc)
        for t in range(turns):
            _commit(b, desc, inps[i], s, 512 * t, 512 * (t + 1), ws)
        ref.append(s)
    slots = [new_state(b, desc) for _ in range(n_sess)]
    live = b.State(desc)
    for t in range(turns):
        for i in range(n_sess):
            b.gdn_state_restore(desc, live, slots[i])
            _commit(b, desc, inps[i], live, 512 * t, 512 * (t + 1), ws)
            b.gdn_state_capture(desc, live, slots[i])
    torch.cuda.synchronize()
    for i in range(n_sess):
        assert same_bits(slots[i].S, ref[i].S) and same_bits(slots[i].conv, ref[i].conv)


def test_branches_equal_full_prompt_prefill(b, desc):
    """Request prefix -> groups -> branches, each prefix run once up to its last multiple of
    64; every branch equals a single FORK over its full prompt, bit for bit."""
    P = 1000
    groups = [0, 1, 70, 128]
    per_group = 2
    lens = synth.branch_lengths(30, len(groups) * per_group)
    total = P + sum(groups) + sum(lens)
    inp = synth.layer_inputs(SHAPE, total, seed=30)
    dinp = to_dev(inp)
    ws = b.workspace(desc, total, 64)
    # token layout: request prefix, then each group's prefix, then its branches
    req = (0, P)
    gofs, bofs, cur, k = [], [], P, 0
    for gl in groups:
        gofs.append((cur, cur + gl))
        cur += gl
    for gi in range(len(groups)):
        for j in range(per_group):
            bofs.append((gi, cur, cur + lens[k]))
            cur += lens[k]
            k += 1
    assert cur == total
    # request prefix state
    run_req = b.gdn_shared_prefix_rows(0, P)
    req_state = b.State(desc)
    run_fork(b, desc, dinp, new_state(b, desc), rows=(0, run_req), out_state=req_state, ws=ws)
    # group states: rows = request remainder + group prefix, run to the last multiple of 64
    gstates, gcarry = [], []
    for (g0, g1) in gofs:
        idx = list(range(run_req, P)) + list(range(g0, g1))
        run = b.gdn_shared_prefix_rows(run_req, run_req + len(idx))
        if run == 0:
            gstates.append(req_state)
            gcarry.append(idx)
        else:
            sub = {kk: v[idx[:run]] for kk, v in dinp.items() if kk != "conv_w"}
            sub["conv_w"] = dinp["conv_w"]
            st = b.State(desc)
            run_fork(b, desc, sub, req_state, out_state=st, ws=ws)
            gstates.append(st)
            gcarry.append(idx[run:])
    # batched branches
    rows, inits, cu = [], [], [0]
    for (gi, b0, b1) in bofs:
        idx = gcarry[gi] + list(range(b0, b1))
        rows += idx
        inits.append(gstates[gi])
        cu.append(cu[-1] + len(idx))
    bx = {kk: v[rows] for kk, v in dinp.items() if kk != "conv_w"}
    o = torch.empty((cu[-1], 32, 128), dtype=torch.bfloat16, device="cuda")
    outs = [b.State(desc) for _ in bofs]
    b.gdn_prefill_branches(desc, cu, bx["x"], dinp["conv_w"], bx["g"], bx["beta"], inits, outs,
                           o, ws)
    torch.cuda.synchronize()
    for k, (gi, b0, b1) in enumerate(bofs):
        full = list(range(0, P)) + list(range(*gofs[gi])) + list(range(b0, b1))
        fx = {kk: v[full] for kk, v in dinp.items() if kk != "conv_w"}
        fx["conv_w"] = dinp["conv_w"]
        of, sf = run_fork(b, desc, fx, new_state(b, desc), ws=ws)
        torch.cuda.synchronize()
        nb = cu[k + 1] - cu[k]
        assert same_bits(o[cu[k]:cu[k + 1]], of[len(full) - nb:]), k
        assert same_bits(outs[k].S, sf.S) and same_bits(outs[k].conv, sf.conv), k
        assert outs[k].pos == len(full)


def test_batched_sequences_equal_single_calls(b, desc):
    """Eight whole sequences of 1 to 16 sub-chunks (ragged and whole), from a zero state and
    from a shared non-zero one, in one batched call: each equals its own single-sequence call
    bit for bit, and the longest matches the oracle.  A batch of eight has 2,048 chain
    workgroups at 32 value heads, so its chains run two workgroups per CU with a two-deep
    prefetch ring; a single sequence has 256 and runs one per CU with a three-deep ring."""
    lens = [64, 128, 192, 200, 256, 320, 1000, 1024]
    total = 128 + sum(lens)
    inp = synth.layer_inputs(SHAPE, total, seed=31)
    dinp = to_dev(inp)
    ws = b.workspace(desc, total, len(lens))
    shared = b.State(desc)
    run_fork(b, desc, dinp, new_state(b, desc), rows=(0, 128), out_state=shared, ws=ws)
    zero = new_state(b, desc)
    inits = [zero if k % 2 == 0 else shared for k in range(len(lens))]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    rows = slice(128, total)
    o = torch.empty((cu[-1], 32, 128), dtype=torch.bfloat16, device="cuda")
    outs = [b.State(desc) for _ in lens]
    b.gdn_prefill_branches(desc, cu, dinp["x"][rows], dinp["conv_w"], dinp["g"][rows],
                           dinp["beta"][rows], inits, outs, o, ws)
    torch.cuda.synchronize()
    for k, n in enumerate(lens):
        r0 = 128 + cu[k]
        of, sf = run_fork(b, desc, dinp, inits[k], rows=(r0, r0 + n), ws=ws)
        torch.cuda.synchronize()
        assert same_bits(o[cu[k]:cu[k + 1]], of), k
        assert same_bits(outs[k].S, sf.S) and same_bits(outs[k].conv, sf.conv), k
        assert outs[k].pos == inits[k].pos + n
    k = 7  # 1,024 rows from the shared state
    r0 = 128 + cu[k]
    sub = {kk: v[r0:r0 + lens[k]] for kk, v in inp.items() if kk != "conv_w"}
    sub["conv_w"] = inp["conv_w"]
    o_ref, S_ref, w_ref = oracle(desc, sub, S0=shared.S.double().cpu().numpy(),
                                 window=synth.f64(shared.conv.cpu()))
    assert_parity(o[cu[k]:cu[k + 1]], outs[k].S, o_ref, S_ref,
                  label="batched 1024 rows from a shared state")
    assert np.array_equal(synth.f64(outs[k].conv.cpu()), w_ref)


def test_more_branches_than_one_launch(b, desc):
    """Forty branches of 1 to 130 rows, from four different states: the host cuts them into
    launches of at most 32 sequences, and every branch still equals its own single call bit
    for bit (outputs, final state and window)."""
    rng = np.random.default_rng(5)
    lens = [int(n) for n in rng.integers(1, 131, size=40)]
    total = 256 + sum(lens)
    inp = synth.layer_inputs(SHAPE, total, seed=33)
    dinp = to_dev(inp)
    ws = b.workspace(desc, total, len(lens))
    starts = [new_state(b, desc)]
    for r in (64, 128, 256):
        starts.append(run_fork(b, desc, dinp, new_state(b, desc), rows=(0, r), ws=ws)[1])
    inits = [starts[k % 4] for k in range(len(lens))]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    rows = slice(256, total)
    o = torch.empty((cu[-1], 32, 128), dtype=torch.bfloat16, device="cuda")
    outs = [b.State(desc) for _ in lens]
    b.gdn_prefill_branches(desc, cu, dinp["x"][rows], dinp["conv_w"], dinp["g"][rows],
                           dinp["beta"][rows], inits, outs, o, ws)
    torch.cuda.synchronize()
    for k, n in enumerate(lens):
        r0 = 256 + cu[k]
        of, sf = run_fork(b, desc, dinp, inits[k], rows=(r0, r0 + n), ws=ws)
        torch.cuda.synchronize()
        assert same_bits(o[cu[k]:cu[k + 1]], of), k
        assert same_bits(outs[k].S, sf.S) and same_bits(outs[k].conv, sf.conv), k
        assert outs[k].pos == inits[k].pos + n


def test_refusals_enqueue_nothing(b, desc):
    dinp = to_dev(synth.layer_inputs(SHAPE, 128, seed=40))
    ws = b.workspace(desc, 128)
    live = new_state(b, desc)
    S0 = live.S.clone()
    o = torch.empty((128, 32, 128), dtype=torch.bfloat16, device="cuda")
    # FORK into itself
    with pytest.raises(b.GdnError) as e:
        b.gdn_prefill_chunked(desc, dinp["x"], dinp["conv_w"], dinp["g"], dinp["beta"], live,
                              live, o, 128, b.GDN_FORK, ws)
    assert e.value.status == b.GDN_EALIAS
    # too small a workspace
    with pytest.raises(b.GdnError) as e:
        b.gdn_prefill_chunked(desc, dinp["x"], dinp["conv_w"], dinp["g"], dinp["beta"], live,
                              b.State(desc), o, 128, b.GDN_FORK, ws[:100])
    assert e.value.status == b.GDN_EWORKSPACE
    # an empty branch
    with pytest.raises(b.GdnError) as e:
        b.gdn_prefill_branches(desc, [0, 64, 64], dinp["x"], dinp["conv_w"], dinp["g"],
                               dinp["beta"], [live, live], None, o, ws)
    assert e.value.status == b.GDN_EINVAL
    torch.cuda.synchronize()
    assert same_bits(live.S, S0) and live.pos == 0
    # and the path still gives the same results afterwards
    o1, s1 = run_fork(b, desc, dinp, live, ws=ws)
    o2, s2 = run_fork(b, desc, dinp, new_state(b, desc), ws=ws)
    torch.cuda.synchronize()
    assert same_bits(o1, o2) and same_bits(s1.S, s2.S)


def test_state_file_round_trip_continues_exactly(b, desc, tmp_path):
    """A session saved to a file and loaded into another slot continues bit for bit ("The
    shadow reader", section "Memory": it comes back exact); a file for other weights is
    refused and the slot keeps what it held."""
    weights = 0xABCDEF0123456789
    dinp = to_dev(synth.layer_inputs(SHAPE, 1536, seed=50))
    ws = b.workspace(desc, 1536)
    live = new_state(b, desc)
    _commit(b, desc, dinp, live, 0, 1024, ws)
    path = str(tmp_path / "session.gdn")
    b.gdn_state_save(desc, live, weights, path)
    slot = new_state(b, desc)
    b.gdn_state_load(desc, slot, weights, path)
    assert same_bits(slot.S, live.S) and same_bits(slot.conv, live.conv)
    assert slot.pos == live.pos == 1024 and slot.tag == live.tag
    _, o1 = _commit(b, desc, dinp, live, 1024, 1536, ws)
    _, o2 = _commit(b, desc, dinp, slot, 1024, 1536, ws)
    assert same_bits(o1, o2) and same_bits(slot.S, live.S)
    keep = slot.S.clone()
    with pytest.raises(b.GdnError) as e:
        b.gdn_state_load(desc, slot, weights + 1, path)
    assert e.value.status == b.GDN_EMISMATCH
    assert same_bits(slot.S, keep) and slot.pos == 1536


@pytest.mark.parametrize("cap", [256, 64])
def test_chained_launches_equal_one_launch(b, desc, monkeypatch, cap):
    """A sequence longer than the per-launch row cap runs as chained launches, each continuing
    from the state the previous one wrote; with the cap lowered (GDN_TEST_LAUNCH_ROWS) a
    1,000-row fork and a 1,536-row commit give the same bits as one launch each."""
    dinp = to_dev(synth.layer_inputs(SHAPE, 1536, seed=81))
    ws = b.workspace(desc, 1536)
    zero = new_state(b, desc)
    ref_o, ref_s = run_fork(b, desc, dinp, zero, rows=(0, 1000), ws=ws)
    ref_c = new_state(b, desc)
    _, ref_co = _commit(b, desc, dinp, ref_c, 0, 1536, ws)
    torch.cuda.synchronize()
    monkeypatch.setenv("GDN_TEST_LAUNCH_ROWS", str(cap))
    o, s = run_fork(b, desc, dinp, zero, rows=(0, 1000), ws=ws)
    live = new_state(b, desc)
    n, co = _commit(b, desc, dinp, live, 0, 1536, ws)
    torch.cuda.synchronize()
    assert n == 1536 and s.pos == 1000
    assert same_bits(o, ref_o) and same_bits(s.S, ref_s.S) and same_bits(s.conv, ref_s.conv)
    assert same_bits(co, ref_co) and same_bits(live.S, ref_c.S) and same_bits(live.conv, ref_c.conv)


def test_branches_without_final_states_give_the_same_outputs(b, desc):
    """gdn_prefill_branches with out=None (scratch final states inside the workspace sized by
    gdn_workspace_bytes(desc, rows, B)) writes the same o bits as with output states."""
    lens = [64, 130, 7, 200, 64, 91]
    total = sum(lens)
    dinp = to_dev(synth.layer_inputs(SHAPE, total, seed=82))
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    zero = new_state(b, desc)
    ws = b.workspace(desc, total, len(lens))
    assert ws.numel() == b.gdn_workspace_bytes(desc, total, len(lens))
    o1 = torch.empty((total, 32, 128), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    outs = [b.State(desc) for _ in lens]
    b.gdn_prefill_branches(desc, cu, dinp["x"], dinp["conv_w"], dinp["g"], dinp["beta"],
                           [zero] * len(lens), outs, o1, ws)
    b.gdn_prefill_branches(desc, cu, dinp["x"], dinp["conv_w"], dinp["g"], dinp["beta"],
                           [zero] * len(lens), None, o2, ws)
    torch.cuda.synchronize()
    assert same_bits(o1, o2)


def test_session_store_spill_and_reload_continue_exactly(b, desc, tmp_path):
    """Two sessions through a store with one resident slot: each acquire of the other session
    writes the resident one to its file; the reloaded session then continues its commits bit
    for bit as if it had never left the GPU."""
    dinp = to_dev(synth.layer_inputs(SHAPE, 2048, seed=83))
    other = to_dev(synth.layer_inputs(SHAPE, 1024, seed=84))
    ws = b.workspace(desc, 2048)
    store = b.SessionStore(desc, 1, b.gdn_state_S_bytes(desc) + b.gdn_state_conv_bytes(desc),
                           directory=str(tmp_path), weights_hash=0x5EED)
    a, origin = store.acquire(1)
    assert origin == b.GDN_STORE_FRESH
    _commit(b, desc, dinp, a, 0, 1024, ws)
    o_mid = None
    s2, origin = store.acquire(2)  # session 1 leaves for its file
    assert origin == b.GDN_STORE_FRESH and store.entry(1)["where"] == b.GDN_STORE_ON_DISK
    _commit(b, desc, other, s2, 0, 1024, ws)
    a, origin = store.acquire(1)  # session 2 leaves; session 1 comes back
    assert origin == b.GDN_STORE_FROM_DISK and a.pos == 1024
    n, o_mid = _commit(b, desc, dinp, a, 1024, 2048, ws)
    torch.cuda.synchronize()
    ref = new_state(b, desc)
    _, o_ref = _commit(b, desc, dinp, ref, 0, 2048, ws)
    torch.cuda.synchronize()
    assert n == 1024 and a.pos == 2048
    assert same_bits(o_mid, o_ref[1024:]) and same_bits(a.S, ref.S) and same_bits(a.conv, ref.conv)
