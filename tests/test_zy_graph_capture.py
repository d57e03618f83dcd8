"""gdn_prefill_chunked_noalloc captured in a HIP graph (through torch.cuda.graph) and replayed:
each replay, with new inputs written into the captured buffers by eager work in between,
equals an eager call of gdn_prefill_chunked with a caller workspace bit for bit."""
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
