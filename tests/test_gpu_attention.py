"""Causal prefill attention of the full-attention layers on the GPU, through the C ABI.

The pages run these layers as split-K flash attention whose merge order depends only on
absolute position, so that cutting a prompt into calls or running branches over a cached prefix
gives exactly the same output ("Long context and sessions", section "The KV cache"); cache rows
below a cut stay valid, so rewinding needs no checkpoint ("The shadow reader", section "Exact
on a grid").  Tested here: parity with the float64 oracle (plain softmax attention on the exact
bf16 inputs) over head ratios 1 to 16, head dims 128 and 256, ragged tiles and cached prefixes
that start off any split boundary; bitwise equality between one call and the same rows cut
into calls, batched into branches, or recomputed after a rewind; the layer's shape at 8,192
rows on sampled rows.
"""
import numpy as np
import pytest
import torch

from hybrid_linear_attention_prefill_amd import synth
from tests.helpers import TOL, rel_l2, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    from hybrid_linear_attention_prefill_amd import binding
    assert torch.cuda.is_available()
    return binding


def _oracle(q, k, v, pos0, scale, rows=None):
    from oracle import numpy_ref
    qs = synth.f64(q)
    if rows is not None:
        out = []
        for t in rows:
            out.append(numpy_ref.attention(qs[t:t + 1], synth.f64(k), synth.f64(v), pos0 + t,
                                           scale)[0])
        return np.stack(out)
    return numpy_ref.attention(qs, synth.f64(k), synth.f64(v), pos0, scale)


def _run(b, desc, q, k, v, pos0, dtype):
    o = torch.empty(q.shape, dtype=dtype, device="cuda")
    b.gdn_attention_prefill(desc, [(q, k, v, o, pos0)])
    return o


@pytest.mark.parametrize("T,pos0,Hq,Hkv,D,dtype", [
    (300, 0, 4, 1, 128, torch.bfloat16),   # ratio 4: two row tiles per workgroup, ragged tail
    (77, 700, 8, 1, 256, torch.float32),   # cached prefix starting inside a split
    (200, 0, 2, 2, 128, torch.float32),    # one query head per key head
    (130, 320, 16, 2, 256, torch.bfloat16),
    (70, 0, 4, 2, 256, torch.float32),     # ratio 2
    (90, 40, 16, 1, 128, torch.float32),   # ratio 16: two workgroups per key head
    (1, 0, 8, 1, 128, torch.float32),      # a single row at position 0
    (5, 1023, 8, 1, 256, torch.float32),   # rows right after a split boundary
])
def test_attention_matches_oracle(b, T, pos0, Hq, Hkv, D, dtype):
    q_all, k, v = synth.attention_inputs(pos0 + T, Hq, Hkv, D, seed=T + pos0 + D)
    q = q_all[pos0:].contiguous()
    desc = b.make_attn_desc(Hq, Hkv, D, out_dtype=dtype)
    o = _run(b, desc, q.cuda(), k.cuda(), v.cuda(), pos0, dtype)
    torch.cuda.synchronize()
    ref = _oracle(q, k, v, pos0, desc.scale)
    err = rel_l2(o.float().cpu().numpy(), ref)
    print("attention T=%d pos0=%d Hq=%d Hkv=%d D=%d %s rel_l2=%.3e"
          % (T, pos0, Hq, Hkv, D, dtype, err), flush=True)
    assert err < TOL


@pytest.mark.parametrize("D", [128, 256])
def test_cut_into_calls_is_bitwise_one_call(b, D):
    """One call over 1,000 rows equals the same rows cut at 333, or at 256 and 600, bit for
    bit: the cuts fall inside splits and inside row tiles."""
    T, Hq, Hkv = 1000, 8, 1
    q, k, v = (t.cuda() for t in synth.attention_inputs(T, Hq, Hkv, D, seed=21))
    desc = b.make_attn_desc(Hq, Hkv, D)
    full = _run(b, desc, q, k, v, 0, torch.bfloat16)
    for cuts in ((0, 333, T), (0, 256, 600, T), (0, 1, 2, 999, T)):
        parts = [_run(b, desc, q[a:e].contiguous(), k, v, a, torch.bfloat16)
                 for a, e in zip(cuts[:-1], cuts[1:])]
        assert same_bits(torch.cat(parts), full), cuts


def test_branches_over_a_shared_prefix_are_bitwise_full_prompts(b):
    """Three branches continue one cached 600-row prefix, in one batched call; each branch's
    rows equal those rows of a single call over its whole prompt, and the batched call equals
    the branches run one at a time."""
    Hq, Hkv, D = 16, 2, 256
    desc = b.make_attn_desc(Hq, Hkv, D)
    P = 600
    lens = (37, 200, 1)
    prompts = []
    for i, n in enumerate(lens):
        q, k, v = synth.attention_inputs(P + n, Hq, Hkv, D, seed=30 + i)
        if prompts:  # the shared prefix: identical rows 0 .. P-1
            q0, k0, v0 = prompts[0]
            q[:P], k[:P], v[:P] = q0[:P], k0[:P], v0[:P]
        prompts.append((q.cuda(), k.cuda(), v.cuda()))
    outs = [torch.empty((n, Hq, D), dtype=torch.bfloat16, device="cuda") for n in lens]
    b.gdn_attention_prefill(desc, [(q[P:].contiguous(), k, v, o, P)
                                   for (q, k, v), o in zip(prompts, outs)])
    for (q, k, v), o, n in zip(prompts, outs, lens):
        full = _run(b, desc, q, k, v, 0, torch.bfloat16)
        assert same_bits(o, full[P:]), n
        alone = _run(b, desc, q[P:].contiguous(), k, v, P, torch.bfloat16)
        assert same_bits(o, alone), n


def test_rewind_reuses_cache_rows_below_the_cut(b):
    """A second continuation from row 512 over the same cache rows 0 .. 511 (new rows above)
    equals a fresh call over the new prompt: no state besides the cache rows is needed."""
    Hq, Hkv, D, T = 8, 1, 128, 900
    q, k, v = (t.cuda() for t in synth.attention_inputs(T, Hq, Hkv, D, seed=40))
    desc = b.make_attn_desc(Hq, Hkv, D)
    _run(b, desc, q, k, v, 0, torch.bfloat16)
    q2, k2, v2 = (t.cuda() for t in synth.attention_inputs(T, Hq, Hkv, D, seed=41))
    q2[:512], k2[:512], v2[:512] = q[:512], k[:512], v[:512]
    kc, vc = k.clone(), v.clone()
    kc[512:], vc[512:] = k2[512:], v2[512:]  # the cache after the rewind: new rows above 512
    cont = _run(b, desc, q2[512:].contiguous(), kc, vc, 512, torch.bfloat16)
    fresh = _run(b, desc, q2, k2, v2, 0, torch.bfloat16)
    assert same_bits(cont, fresh[512:])


def test_empty_calls_touch_nothing(b):
    desc = b.make_attn_desc(4, 1, 128, out_dtype=torch.float32)
    q, k, v = (t.cuda() for t in synth.attention_inputs(16, 4, 1, 128, seed=50))
    o = torch.full((16, 4, 128), 5.0, device="cuda")
    b.gdn_attention_prefill(desc, [])
    b.gdn_attention_prefill(desc, [(q[:0], k, v, o[:0], 3)])
    torch.cuda.synchronize()
    assert (o == 5.0).all()


def test_more_sequences_than_one_launch(b):
    """40 one-row sequences (two launches) equal the same rows run one at a time."""
    Hq, Hkv, D = 4, 1, 128
    desc = b.make_attn_desc(Hq, Hkv, D)
    q, k, v = (t.cuda() for t in synth.attention_inputs(300, Hq, Hkv, D, seed=60))
    outs = [torch.empty((1, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(40)]
    b.gdn_attention_prefill(desc, [(q[250 + i:251 + i].contiguous(), k, v, outs[i], 250 + i)
                                   for i in range(40)])
    full = _run(b, desc, q, k, v, 0, torch.bfloat16)
    for i in range(40):
        assert same_bits(outs[i], full[250 + i:251 + i]), i


def test_layer_shape_8192_rows_sampled(b):
    """16 query heads over 2 key heads of width 256 at 8,192 rows: sampled rows against the
    oracle, and a tail call from row 8,000 against the same rows of the full call."""
    T, Hq, Hkv, D = 8192, 16, 2, 256
    q, k, v = synth.attention_inputs(T, Hq, Hkv, D, seed=70)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    desc = b.make_attn_desc(Hq, Hkv, D)
    o = _run(b, desc, qd, kd, vd, 0, torch.bfloat16)
    torch.cuda.synchronize()
    rows = [0, 255, 256, 4000, 6143, 8191]
    ref = _oracle(q, k, v, 0, desc.scale, rows=rows)
    err = rel_l2(o[rows].float().cpu().numpy(), ref)
    print("attention 8192 sampled rel_l2=%.3e" % err, flush=True)
    assert err < TOL
    tail = _run(b, desc, qd[8000:].contiguous(), kd, vd, 8000, torch.bfloat16)
    assert same_bits(tail, o[8000:])
