"""Calls captured in a HIP graph (through torch.cuda.graph) and replayed.

- gdn_prefill_chunked_noalloc: each replay, with new inputs written into the captured buffers by
  eager work in between, equals an eager call of gdn_prefill_chunked with a caller workspace
  bit for bit.
- gdn_decode_step: a run of one-token steps captured once equals the same steps run eagerly, bit
  for bit, on every replay.
"""
import pytest
import torch

from hybrid_linear_attention_prefill_amd import synth
from tests.helpers import new_state, run_fork, same_bits, to_dev

pytestmark = pytest.mark.gpu

SHAPE = synth.LAYER_16x32x128


@pytest.fixture(scope="module")
def b():
    from hybrid_linear_attention_prefill_amd import binding
    assert torch.cuda.is_available()
    return binding


def test_noalloc_fork_replays_in_a_graph_exactly(b):
    desc = b.make_desc(16, 32, 128, 128)
    T = 300
    pre = to_dev(synth.layer_inputs(SHAPE, 128, seed=94))
    _, s0 = run_fork(b, desc, pre, new_state(b, desc))  # a read-only starting state at pos 128
    buf = to_dev(synth.layer_inputs(SHAPE, T, seed=95))   # the buffers the graph reads
    out = b.State(desc)
    o = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")

    def call():
        return b.gdn_prefill_chunked_noalloc(desc, buf["x"], buf["conv_w"], buf["g"], buf["beta"],
                                             s0, out, o, T, b.GDN_FORK)

    assert call() == T  # eager first call: the static array's address is looked up here
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.synchronize()
    for i in range(3):
        new = to_dev(synth.layer_inputs(SHAPE, T, seed=96 + i))
        for k in ("x", "conv_w", "g", "beta"):
            buf[k].copy_(new[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref = run_fork(b, desc, new, s0)
        torch.cuda.synchronize()
        assert same_bits(o, ref_o), i
        assert same_bits(out.S, ref.S) and same_bits(out.conv, ref.conv), i


@pytest.mark.parametrize("B", [1, 3])
def test_decode_steps_replay_in_a_graph_exactly(b, B):
    """A serving loop's decode steps captured once and replayed: sixteen one-token steps of B
    sessions (states stepped back and forth between two sets) equal the same steps run eagerly,
    bit for bit, on every replay, with other eager decode work between the replays."""
    desc = b.make_desc(16, 32, 128, 128)
    N = 16
    pre = to_dev(synth.layer_inputs(SHAPE, 128, seed=97))
    _, s0 = run_fork(b, desc, pre, new_state(b, desc))  # the sessions' starting state (pos 128)
    inp = to_dev(synth.layer_inputs(SHAPE, N * B, seed=98))
    ping = [b.State(desc) for _ in range(B)]
    pong = [b.State(desc) for _ in range(B)]
    o = torch.empty((N, B, 32, 128), dtype=torch.bfloat16, device="cuda")

    def reset():
        for st in ping:
            b.gdn_state_capture(desc, s0, st)

    def steps(out):
        for i in range(N):
            src, dst = (ping, pong) if i % 2 == 0 else (pong, ping)
            r = slice(i * B, (i + 1) * B)
            b.gdn_decode_step(desc, inp["x"][r], inp["conv_w"], inp["g"][r], inp["beta"][r], src,
                              dst, out[i])

    reset()
    steps(o)
    torch.cuda.synchronize()
    ref_o = o.clone()
    ref = [(st.S.clone(), st.conv.clone()) for st in ping]  # N even: the last step wrote ping
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            steps(o)
    torch.cuda.synchronize()
    scratch_o = torch.empty_like(o)
    for rep in range(3):
        reset()
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert same_bits(o, ref_o), rep
        for st, (S, conv) in zip(ping, ref):
            assert same_bits(st.S, S) and same_bits(st.conv, conv), rep
        reset()  # eager decode work between the replays
        steps(scratch_o)
        torch.cuda.synchronize()
        assert same_bits(scratch_o, ref_o), rep
