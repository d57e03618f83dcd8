"""One-token decode steps on the GPU, through the C ABI.

After a fork's prefill the small model writes its answer token by token on top of the session
("The shadow reader", section "Who asks": the fork decodes eagerly).  Each decode step is the
per-token gated delta rule, which is exactly what the float64 oracle runs, so a run of decode
steps is checked against the oracle over the same rows from the same starting state (the
GPU's own state, downloaded, so only the steps' rounding is measured).
"""
import numpy as np
import pytest
import torch

from hybrid_linear_attention_prefill_amd import synth
from tests.helpers import TOL, desc_kwargs, new_state, rel_l2, run_fork, same_bits, to_dev

pytestmark = pytest.mark.gpu

SHAPE = synth.LAYER_16x32x128
DECODE_TOL = 1e-5  # the step is fp32 throughout: it must sit far inside the 2e-3 bar


@pytest.fixture(scope="module")
def b():
    from hybrid_linear_attention_prefill_amd import binding
    assert torch.cuda.is_available()
    return binding


def _commit(b, desc, dinp, n):
    s = new_state(b, desc)
    o = torch.empty((n, desc.n_v_heads, desc.d_v), dtype=desc.out_torch, device="cuda")
    ws = b.workspace(desc, n)
    assert b.gdn_prefill_chunked(desc, dinp["x"][:n], dinp.get("conv_w"), dinp["g"][:n],
                                 dinp["beta"][:n], s, s, o, n, b.GDN_COMMIT, ws) == n
    return s


def _decode_rows(b, desc, dinp, state, r0, r1, out_state=None):
    """Decode rows r0 .. r1-1 one at a time from `state` (in place unless out_state)."""
    outs = []
    cur = state
    for r in range(r0, r1):
        o = torch.empty((1, desc.n_v_heads, desc.d_v), dtype=desc.out_torch, device="cuda")
        dst = out_state if (out_state is not None and r == r0) else cur
        b.gdn_decode_step(desc, dinp["x"][r:r + 1], dinp.get("conv_w"), dinp["g"][r:r + 1],
                          dinp["beta"][r:r + 1], [cur], [dst], o)
        cur = dst
        outs.append(o)
    return torch.cat(outs), cur


def _oracle_from(desc, inp, r0, r1, S0, win0):
    from oracle import c_oracle
    x = synth.f64(inp["x"][r0:r1])
    conv_w = synth.f64(inp["conv_w"]) if desc.conv_width > 0 else None
    return c_oracle.gdn_layer(x, conv_w, win0, synth.f64(inp["g"][r0:r1]),
                              synth.f64(inp["beta"][r0:r1]), S0, **desc_kwargs(desc))


def _host_state(state):
    S = state.S.detach().cpu().to(torch.float64).numpy()
    win = None if state.conv is None else state.conv.detach().cpu().to(torch.float64).numpy()
    return S, win


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_steps_match_oracle(b, out_dtype):
    """24 tokens decoded in place after a 1,024-row commit, against the per-token oracle."""
    desc = b.make_desc(16, 32, 128, 128, out_dtype=out_dtype)
    inp = synth.layer_inputs(SHAPE, 1024 + 24, seed=40)
    dinp = to_dev(inp)
    live = _commit(b, desc, dinp, 1024)
    S0, win0 = _host_state(live)
    o, live = _decode_rows(b, desc, dinp, live, 1024, 1048)
    torch.cuda.synchronize()
    o_ref, S_ref, win_ref = _oracle_from(desc, inp, 1024, 1048, S0, win0)
    eo = rel_l2(o.float().cpu().numpy(), o_ref)
    es = rel_l2(live.S.cpu().numpy(), S_ref)
    print("decode rel_l2 o=%.3e S=%.3e" % (eo, es), flush=True)
    assert es < DECODE_TOL
    assert eo < (DECODE_TOL if out_dtype == torch.float32 else TOL)
    # the window holds the last three inputs, bit for bit
    assert same_bits(live.conv, dinp["x"][1045:1048])
    assert live.pos == 1048


def test_decode_gqa_silu_d64(b):
    """Four value heads per key head, width 64, SiLU after the conv, fp32 activations."""
    shape = synth.Shape(2, 8, 64, 64, 4)
    desc = b.make_desc(2, 8, 64, 64, conv_silu=True, act_dtype=torch.float32,
                       out_dtype=torch.float32)
    inp = synth.layer_inputs(shape, 512 + 9, seed=41, act_dtype=torch.float32)
    dinp = to_dev(inp)
    live = _commit(b, desc, dinp, 512)
    S0, win0 = _host_state(live)
    o, live = _decode_rows(b, desc, dinp, live, 512, 521)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = _oracle_from(desc, inp, 512, 521, S0, win0)
    eo, es = rel_l2(o.cpu().numpy(), o_ref), rel_l2(live.S.cpu().numpy(), S_ref)
    print("decode gqa rel_l2 o=%.3e S=%.3e" % (eo, es), flush=True)
    assert eo < DECODE_TOL and es < DECODE_TOL


def test_decode_without_conv_one_head(b):
    """The one-head fp32 recipe (inputs already post-conv, unit q/k rows), from a zero state."""
    desc = b.make_desc(1, 1, 64, 64, conv_width=0, act_dtype=torch.float32,
                       out_dtype=torch.float32)
    inp = synth.layer_inputs(synth.ONE_HEAD, 40, seed=42, act_dtype=torch.float32, unit_qk=True)
    dinp = to_dev(inp)
    live = new_state(b, desc)
    o, live = _decode_rows(b, desc, dinp, live, 0, 40)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = _oracle_from(desc, inp, 0, 40, np.zeros((1, 64, 64)), None)
    assert rel_l2(o.cpu().numpy(), o_ref) < DECODE_TOL
    assert rel_l2(live.S.cpu().numpy(), S_ref) < DECODE_TOL


def test_decode_batch_equals_single_sequences_bitwise(b):
    """Five sequences in one call: three own states and two that read one shared state.  Each
    equals the same step run alone, bit for bit; the shared input state is not touched."""
    desc = b.make_desc(16, 32, 128, 128)
    inp = synth.layer_inputs(SHAPE, 1536, seed=43)
    dinp = to_dev(inp)
    def rows_from(r):
        return {"x": dinp["x"][r:], "g": dinp["g"][r:], "beta": dinp["beta"][r:],
                "conv_w": dinp["conv_w"]}

    base = [_commit(b, desc, rows_from(r), 512) for r in (0, 256, 512)]
    shared = base[2]
    shared_S = shared.S.clone()
    ins = [base[0], base[1], shared, shared, shared]
    rows = [1000, 1001, 1002, 1003, 1004]
    # batched: sequences 0, 1 in place; 2, 3, 4 into fresh states
    snaps = []
    for s in ins[:2]:
        c = b.State(desc)
        b.gdn_state_capture(desc, s, c)
        snaps.append(c)
    outs = [ins[0], ins[1], b.State(desc), b.State(desc), b.State(desc)]
    x = torch.stack([dinp["x"][r] for r in rows])
    g = torch.stack([dinp["g"][r] for r in rows])
    beta = torch.stack([dinp["beta"][r] for r in rows])
    o = torch.empty((5, 32, 128), dtype=desc.out_torch, device="cuda")
    b.gdn_decode_step(desc, x, dinp["conv_w"], g, beta, ins, outs, o)
    assert same_bits(shared.S, shared_S)
    singles_in = snaps + [shared, shared, shared]
    for i, r in enumerate(rows):
        so = torch.empty((1, 32, 128), dtype=desc.out_torch, device="cuda")
        dst = b.State(desc)
        b.gdn_decode_step(desc, dinp["x"][r:r + 1], dinp["conv_w"], dinp["g"][r:r + 1],
                          dinp["beta"][r:r + 1], [singles_in[i]], [dst], so)
        assert same_bits(so[0], o[i]), i
        assert same_bits(dst.S, outs[i].S) and same_bits(dst.conv, outs[i].conv), i
        assert outs[i].pos == singles_in[i].pos + 1


def test_decode_in_place_equals_out_of_place(b):
    desc = b.make_desc(16, 32, 128, 128)
    inp = synth.layer_inputs(SHAPE, 520, seed=44)
    dinp = to_dev(inp)
    a = _commit(b, desc, dinp, 512)
    c = b.State(desc)
    b.gdn_state_capture(desc, a, c)
    fresh = b.State(desc)
    o1, _ = _decode_rows(b, desc, dinp, c, 512, 513, out_state=fresh)
    o2, _ = _decode_rows(b, desc, dinp, a, 512, 513)
    assert same_bits(o1, o2) and same_bits(fresh.S, a.S) and same_bits(fresh.conv, a.conv)


def test_decode_agrees_with_fork_prefill_and_is_off_grid(b):
    """Five decode steps and a FORK prefill of the same five rows reach the same state within
    the bar (different rounding: per-token rule against chunk algebra).  The decoded state is
    off the 64-row grid, so a prefill from it is refused; another decode step continues it."""
    desc = b.make_desc(16, 32, 128, 128, out_dtype=torch.float32)
    inp = synth.layer_inputs(SHAPE, 512 + 6, seed=45)
    dinp = to_dev(inp)
    live = _commit(b, desc, dinp, 512)
    o_f, st_f = run_fork(b, desc, dinp, live, rows=(512, 517))
    dec = b.State(desc)
    o_d, dec = _decode_rows(b, desc, dinp, live, 512, 517, out_state=dec)
    torch.cuda.synchronize()
    assert rel_l2(o_d.cpu().numpy(), o_f.cpu().numpy()) < TOL
    assert rel_l2(dec.S.cpu().numpy(), st_f.S.cpu().numpy()) < TOL
    assert same_bits(dec.conv, st_f.conv)
    assert dec.pos == 517 and live.pos == 512
    with pytest.raises(b.GdnError) as e:
        run_fork(b, desc, dinp, dec, rows=(517, 518))
    assert e.value.status == b.GDN_EGRID
    _decode_rows(b, desc, dinp, dec, 517, 518)
    assert dec.pos == 518


def test_decode_more_sequences_than_one_launch(b):
    """40 sequences (two launch groups) equal the steps run one at a time, bit for bit."""
    shape = synth.Shape(1, 2, 64, 64, 4)
    desc = b.make_desc(1, 2, 64, 64)
    inp = synth.layer_inputs(shape, 40, seed=46)
    dinp = to_dev(inp)
    states = []
    for i in range(40):
        s = new_state(b, desc)
        states.append(s)
    o = torch.empty((40, 2, 64), dtype=desc.out_torch, device="cuda")
    outs = [b.State(desc) for _ in range(40)]
    b.gdn_decode_step(desc, dinp["x"], dinp["conv_w"], dinp["g"], dinp["beta"], states, outs, o)
    for i in (0, 31, 32, 39):
        so = torch.empty((1, 2, 64), dtype=desc.out_torch, device="cuda")
        dst = b.State(desc)
        b.gdn_decode_step(desc, dinp["x"][i:i + 1], dinp["conv_w"], dinp["g"][i:i + 1],
                          dinp["beta"][i:i + 1], [states[i]], [dst], so)
        assert same_bits(so[0], o[i]) and same_bits(dst.S, outs[i].S), i
