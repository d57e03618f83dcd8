"""Workload-shaped GPU tests through the C ABI.

- A multi-turn session of 41,802 tokens in 12 turns. After each turn the whole 512-row
  chunks are committed and the pending tail plus a 40-token question is forked. The
  committed state must equal a fresh one-call commit bit for bit, and the fork must leave it
  untouched ("The shadow reader", sections "Exact on a grid" and "Read rate").
- A long session of 24 independent layers at 100,000 tokens in 6 turns, with a checkpoint at
  every turn end. After a divergence the newest checkpoint at or below it is restored and
  the rest re-prefilled; the result must equal a fresh prefill of the changed prompt, bit for
  bit ("The shadow reader", section "One session's state"; "Long context and sessions",
  section Checkpoints).
- The prefix-sharing layout of 32 branches in 4 groups, for a sweep of request prefixes.
  Every branch must equal a plain pass over its full prompt, bit for bit (PR "qwen3_5: run
  prompts that share prefixes once per prefix", sections "Test Plan" and "Test Result").

Token ids index random embedding rows: x, beta and g of a token are rows of seeded tables.
The vocabulary sizes here (4,096 and 1,024 rows) are stand-ins; the pages fix none.
"""
import numpy as np
import pytest
import torch

from hybrid_linear_attention_prefill_amd import synth
from tests.helpers import assert_parity, new_state, oracle, run_fork, same_bits

pytestmark = pytest.mark.gpu

SHAPE = synth.LAYER_16x32x128
HEADS = [0, 7, 18, 31]  # value heads the oracle checks in the long runs


@pytest.fixture(scope="module")
def b():
    from hybrid_linear_attention_prefill_amd import binding
    assert torch.cuda.is_available()
    return binding


@pytest.fixture(scope="module")
def desc(b):
    return b.make_desc(16, 32, 128, 128, conv_width=4, grid=512)


class DevTables:
    """Token tables on the device (for gathering inputs) and on the host (for the oracle)."""

    def __init__(self, vocab, seed):
        self.host = synth.TokenTables(SHAPE, vocab, seed)
        self.E = self.host.E.cuda()
        self.g = self.host.g.cuda()
        self.beta = self.host.beta.cuda()
        self.conv_w = self.host.conv_w.cuda()

    def dev(self, ids):
        i = torch.as_tensor(np.asarray(ids, dtype=np.int64), device="cuda")
        return {"x": self.E[i], "g": self.g[i], "beta": self.beta[i], "conv_w": self.conv_w}

    def host_rows(self, ids):
        r = self.host.rows(ids)
        r["conv_w"] = self.host.conv_w
        return r


def _commit(b, desc, inp, state, ws):
    T = inp["x"].shape[0]
    o = torch.empty((T, desc.n_v_heads, desc.d_v), dtype=desc.out_torch, device="cuda")
    n = b.gdn_prefill_chunked(desc, inp["x"], inp["conv_w"], inp["g"], inp["beta"], state, state,
                              o, T, b.GDN_COMMIT, ws)
    return n, o[:n]


def _check_oracle(desc, host_inp, o_gpu, S_gpu, S0=None, window=None, heads=HEADS):
    o_ref, S_ref, w_ref = oracle(desc, host_inp, S0=S0, window=window, heads=heads)
    assert_parity(o_gpu[:, heads], S_gpu[heads], o_ref[:, heads], S_ref[heads])
    return w_ref


def test_multi_turn_replay_41802(b, desc):
    total, n_turns, n_question, vocab, seed = 41802, 12, 40, 4096, 50
    tab = DevTables(vocab, seed)
    ids = synth.token_ids(seed, total, vocab)
    cuts = synth.turn_cuts(seed, total, n_turns)
    ws = b.workspace(desc, total)
    live = new_state(b, desc)
    committed = 0
    for t, end in enumerate(cuts):
        n, _ = _commit(b, desc, tab.dev(ids[committed:end]), live, ws)
        committed += n
        assert live.pos == committed and committed % 512 == 0
        # the pending tail plus a question, forked from the committed state
        q = synth.question_ids(seed, t, n_question, vocab)
        fork_ids = np.concatenate([ids[committed:end], q])
        S_before, W_before = live.S.clone(), live.conv.clone()
        fork = b.State(desc)
        o, fork = run_fork(b, desc, tab.dev(fork_ids), live, out_state=fork, ws=ws)
        torch.cuda.synchronize()
        assert same_bits(live.S, S_before) and same_bits(live.conv, W_before)
        assert live.pos == committed and fork.pos == committed + len(fork_ids)
        if t % 4 == 3 or t == n_turns - 1:
            w_ref = _check_oracle(desc, tab.host_rows(fork_ids), o, fork.S,
                                  S0=live.S.cpu().numpy().astype(np.float64),
                                  window=synth.f64(live.conv))
            assert np.array_equal(synth.f64(fork.conv), w_ref)
        # the committed state equals a fresh one-call commit of the committed prefix
        fresh = new_state(b, desc)
        n2, _ = _commit(b, desc, tab.dev(ids[:committed]), fresh, ws)
        torch.cuda.synchronize()
        assert n2 == committed
        assert same_bits(live.S, fresh.S) and same_bits(live.conv, fresh.conv)
    assert committed == 41472 and total - committed == 330
    # the last fork equals one FORK over the whole prompt plus the question, bit for bit
    whole = np.concatenate([ids, q])
    o_all, s_all = run_fork(b, desc, tab.dev(whole), new_state(b, desc), ws=ws)
    torch.cuda.synchronize()
    assert same_bits(o_all[committed:], o) and same_bits(s_all.S, fork.S)
    assert same_bits(s_all.conv, fork.conv)


def test_long_session_checkpoints_and_divergence(b, desc):
    n_layers, total, n_turns, vocab, seed = 24, 100_000, 6, 1024, 60
    tabs = [DevTables(vocab, 1000 + l) for l in range(n_layers)]
    ids = synth.token_ids(seed, total, vocab)
    cuts = synth.turn_cuts(seed, total, n_turns)
    ws = b.workspace(desc, total)
    ring = b.CkptRing()
    live = [new_state(b, desc) for _ in range(n_layers)]
    slots = [[b.State(desc) for _ in range(b.MAX_CHECKPOINTS)] for _ in range(n_layers)]
    committed = 0
    for end in cuts:
        n = None
        for l in range(n_layers):
            nl, _ = _commit(b, desc, tabs[l].dev(ids[committed:end]), live[l], ws)
            assert n is None or nl == n
            n = nl
        committed += n
        k = ring.push(committed)
        assert k >= 0
        for l in range(n_layers):
            b.gdn_state_capture(desc, live[l], slots[l][k])
    assert committed == (total // 512) * 512
    # a divergence: every token from d on is replaced
    d = synth.divergence_point(seed, 1, total)
    ids2 = ids.copy()
    ids2[d:] = synth.token_ids(seed + 1, total - d, vocab)
    k = ring.find(d)
    ring.drop_above(d)
    p = ring.c.pos[k] if k >= 0 else 0
    assert p <= d and p % 512 == 0
    for l in range(n_layers):
        if k >= 0:
            b.gdn_state_restore(desc, live[l], slots[l][k])
        else:
            b.gdn_state_init(desc, live[l])
        assert live[l].pos == p
        _commit(b, desc, tabs[l].dev(ids2[p:]), live[l], ws)
        fresh = new_state(b, desc)
        _commit(b, desc, tabs[l].dev(ids2), fresh, ws)
        torch.cuda.synchronize()
        assert live[l].pos == fresh.pos == committed
        assert same_bits(live[l].S, fresh.S) and same_bits(live[l].conv, fresh.conv), l
    # two layers against the oracle: 2,048 rows continued from the restored checkpoint
    for l in (0, n_layers - 1):
        st = b.State(desc)
        if k >= 0:
            b.gdn_state_restore(desc, st, slots[l][k])
        else:
            b.gdn_state_init(desc, st)
        rows = ids2[p:p + 2048]
        o, fk = run_fork(b, desc, tabs[l].dev(rows), st, ws=ws)
        torch.cuda.synchronize()
        _check_oracle(desc, tabs[l].host_rows(rows), o, fk.S,
                      S0=st.S.cpu().numpy().astype(np.float64), window=synth.f64(st.conv))


def _sub(dinp, idx):
    i = torch.as_tensor(np.asarray(idx, dtype=np.int64), device="cuda")
    out = {k: v[i] for k, v in dinp.items() if k != "conv_w"}
    out["conv_w"] = dinp["conv_w"]
    return out


@pytest.mark.parametrize("P", [0, 1, 63, 64, 65, 300, 1000])
def test_32_branches_prefix_sweep(b, desc, P):
    """Request prefix P; groups with 0, 1, 70 and 128 rows of their own; 8 branches per group
    of 1-200 rows each.  Each prefix runs once up to its last multiple of 64; the remainder
    runs at the head of every branch."""
    groups, per_group = [0, 1, 70, 128], 8
    lens = synth.branch_lengths(31 + P, len(groups) * per_group)
    total = P + sum(groups) + sum(lens)
    host = synth.layer_inputs(SHAPE, total, seed=31 + P)
    dinp = {k: v.cuda() for k, v in host.items()}
    ws = b.workspace(desc, total, 64)
    gofs, bofs, cur, k = [], [], P, 0
    for gl in groups:
        gofs.append((cur, cur + gl))
        cur += gl
    for gi in range(len(groups)):
        for _ in range(per_group):
            bofs.append((gi, cur, cur + lens[k]))
            cur += lens[k]
            k += 1
    run_req = b.gdn_shared_prefix_rows(0, P)
    assert run_req == (P // 64) * 64
    req_state = new_state(b, desc)
    if run_req > 0:
        req_state = b.State(desc)
        run_fork(b, desc, _sub(dinp, range(run_req)), new_state(b, desc), out_state=req_state,
                 ws=ws)
    gstates, gcarry = [], []
    for (g0, g1) in gofs:
        idx = list(range(run_req, P)) + list(range(g0, g1))
        run = b.gdn_shared_prefix_rows(run_req, run_req + len(idx))
        if run == 0:
            gstates.append(req_state)
            gcarry.append(idx)
        else:
            st = b.State(desc)
            run_fork(b, desc, _sub(dinp, idx[:run]), req_state, out_state=st, ws=ws)
            gstates.append(st)
            gcarry.append(idx[run:])
    rows, inits, cu = [], [], [0]
    for (gi, b0, b1) in bofs:
        idx = gcarry[gi] + list(range(b0, b1))
        rows += idx
        inits.append(gstates[gi])
        cu.append(cu[-1] + len(idx))
    bx = _sub(dinp, rows)
    o = torch.empty((cu[-1], 32, 128), dtype=torch.bfloat16, device="cuda")
    outs = [b.State(desc) for _ in bofs]
    b.gdn_prefill_branches(desc, cu, bx["x"], bx["conv_w"], bx["g"], bx["beta"], inits, outs, o,
                           ws)
    torch.cuda.synchronize()
    for k, (gi, b0, b1) in enumerate(bofs):
        full = list(range(0, P)) + list(range(*gofs[gi])) + list(range(b0, b1))
        of, sf = run_fork(b, desc, _sub(dinp, full), new_state(b, desc), ws=ws)
        torch.cuda.synchronize()
        nb = cu[k + 1] - cu[k]
        assert same_bits(o[cu[k]:cu[k + 1]], of[len(full) - nb:]), k
        assert same_bits(outs[k].S, sf.S) and same_bits(outs[k].conv, sf.conv), k
        assert outs[k].pos == len(full)
        if k in (0, 13, 31):  # a few branches against the oracle over their full prompts
            hf = {kk: v[full] for kk, v in host.items() if kk != "conv_w"}
            hf["conv_w"] = host["conv_w"]
            o_ref, S_ref, _ = oracle(desc, hf, heads=HEADS)
            assert_parity(o[cu[k]:cu[k + 1]][:, HEADS], outs[k].S[HEADS],
                          o_ref[len(full) - nb:, HEADS], S_ref[HEADS], label="branch %d" % k)


def test_bf16_output_is_rounded_fp32_output(b):
    """The same call with fp32 and bf16 outputs: the bf16 values are the fp32 ones rounded to
    nearest even (the state does not depend on the output type)."""
    d32 = b.make_desc(16, 32, 128, 128, out_dtype=torch.float32)
    d16 = b.make_desc(16, 32, 128, 128, out_dtype=torch.bfloat16)
    dinp = {k: v.cuda() for k, v in synth.layer_inputs(SHAPE, 700, seed=70).items()}
    o32, s32 = run_fork(b, d32, dinp, new_state(b, d32))
    o16, s16 = run_fork(b, d16, dinp, new_state(b, d16))
    torch.cuda.synchronize()
    assert same_bits(o32.to(torch.bfloat16), o16)
    assert same_bits(s32.S, s16.S) and same_bits(s32.conv, s16.conv)
