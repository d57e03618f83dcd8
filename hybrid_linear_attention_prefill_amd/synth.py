"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and casts them; it holds none of the layer's arithmetic.
Both the HIP path and the float64 oracle receive exactly the arrays made here: the device
gets a copy of the cast tensor, the oracle gets the same tensor upcast to float64.

Draws use numpy's PCG64 seeded with ``[seed, stream]``; the stream ids are fixed:

  0 q channels | 1 k channels | 2 v channels / embedding table | 3 beta logits |
  4 g logits | 5 conv weights | 6 token ids | 7 turn cuts | 8 question ids |
  9 branch lengths | 10 divergence point | 11 projection inputs | 12 projection weights |
  13 attention queries | 14 attention keys | 15 attention values

Value recipes (the pages print no data; these are stated stand-ins):
  x ~ N(0,1) cast to the activation dtype with round-to-nearest-even;
  conv weights ~ U(-1/2, 1/2); beta = sigmoid(N(0,1)); g = -softplus(N(0,1)) (times an
  optional factor for slow-decay stress inputs); all fp32.
"""
from dataclasses import dataclass

import numpy as np
import torch

STREAM_Q, STREAM_K, STREAM_V, STREAM_BETA, STREAM_G, STREAM_W = 0, 1, 2, 3, 4, 5
STREAM_IDS, STREAM_CUTS, STREAM_QUESTION, STREAM_BRANCH, STREAM_DIVERGE = 6, 7, 8, 9, 10
STREAM_PROJ_X, STREAM_PROJ_W = 11, 12
STREAM_ATT_Q, STREAM_ATT_K, STREAM_ATT_V = 13, 14, 15


@dataclass(frozen=True)
class Shape:
    n_k_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    conv_width: int = 4

    @property
    def channels(self):
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v


# One value head of width 64, fp32, inputs already post-conv.
ONE_HEAD = Shape(1, 1, 64, 64, 0)
# One layer: 16 key heads, 32 value heads, head dim 128, width-4 conv.
LAYER_16x32x128 = Shape(16, 32, 128, 128, 4)


def rng(seed, stream):
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def cast(a, dtype):
    """float64 numpy -> CPU torch tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dtype)


def f64(t):
    """CPU float64 numpy copy of a tensor (exact upcast)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z):
    return np.logaddexp(0.0, z)


def gates_from_logits(beta_logit, g_logit, g_scale=1.0):
    """beta = sigmoid(logit), g = -softplus(logit) * g_scale, both cast to fp32."""
    beta = cast(_sigmoid(beta_logit), torch.float32)
    g = cast(-_softplus(g_logit) * g_scale, torch.float32)
    return beta, g


def layer_inputs(shape, T, seed=0, act_dtype=torch.bfloat16, g_scale=1.0, unit_qk=False,
                 v_scale=1.0, beta_shift=0.0):
    """Random layer inputs for T rows.

    Returns a dict of CPU tensors: x [T, C] (act dtype), conv_w [C, W] (act dtype, absent
    when W == 0), g, beta [T, Hv] fp32.  ``unit_qk`` scales each q and k head row to unit
    length in float64 before the cast (the one-head fp32 recipe).
    ``v_scale`` multiplies the v channels (a power of two keeps the cast exact relative to the
    unscaled draw); ``beta_shift`` is added to the beta logits (a large shift drives beta
    towards 1).  Both serve stress inputs beyond the stated recipe.
    """
    a = shape.n_k_heads * shape.d_k
    q = rng(seed, STREAM_Q).standard_normal((T, a))
    k = rng(seed, STREAM_K).standard_normal((T, a))
    v = rng(seed, STREAM_V).standard_normal((T, shape.n_v_heads * shape.d_v)) * v_scale
    if unit_qk:
        for m in (q, k):
            r = m.reshape(T, shape.n_k_heads, shape.d_k)
            r /= np.sqrt((r * r).sum(-1, keepdims=True))
    x = cast(np.concatenate([q, k, v], axis=1), act_dtype)
    beta, g = gates_from_logits(rng(seed, STREAM_BETA).standard_normal((T, shape.n_v_heads))
                                + beta_shift,
                                rng(seed, STREAM_G).standard_normal((T, shape.n_v_heads)),
                                g_scale)
    out = {"x": x, "g": g, "beta": beta}
    if shape.conv_width > 0:
        out["conv_w"] = cast(rng(seed, STREAM_W).uniform(-0.5, 0.5,
                                                          (shape.channels, shape.conv_width)),
                             act_dtype)
    return out


class TokenTables:
    """Per-id random rows: ids -> (x row, beta, g), i.e. "ids -> random embeddings".

    E [V, C] ~ N(0,1) in the activation dtype; beta/g logits [V, Hv] ~ N(0,1).
    """

    def __init__(self, shape, vocab, seed, act_dtype=torch.bfloat16):
        self.shape, self.vocab = shape, vocab
        self.E = cast(rng(seed, STREAM_V).standard_normal((vocab, shape.channels)), act_dtype)
        self.beta, self.g = gates_from_logits(
            rng(seed, STREAM_BETA).standard_normal((vocab, shape.n_v_heads)),
            rng(seed, STREAM_G).standard_normal((vocab, shape.n_v_heads)))
        self.conv_w = cast(rng(seed, STREAM_W).uniform(-0.5, 0.5,
                                                        (shape.channels, shape.conv_width)),
                           act_dtype)

    def rows(self, ids):
        ids = torch.as_tensor(np.asarray(ids, dtype=np.int64))
        return {"x": self.E[ids], "g": self.g[ids], "beta": self.beta[ids]}


def token_ids(seed, n, vocab, stream=STREAM_IDS):
    return rng(seed, stream).integers(0, vocab, size=n, dtype=np.int64)


def turn_cuts(seed, total, n_turns):
    """n_turns - 1 distinct uniform cut points in (0, total), sorted; turn ends follow."""
    r = rng(seed, STREAM_CUTS)
    cuts = np.sort(r.choice(np.arange(1, total), size=n_turns - 1, replace=False))
    return [int(c) for c in cuts] + [int(total)]


def question_ids(seed, turn, n, vocab):
    return rng(seed * 1000 + turn, STREAM_QUESTION).integers(0, vocab, size=n, dtype=np.int64)


def branch_lengths(seed, n, lo=1, hi=200):
    return [int(v) for v in rng(seed, STREAM_BRANCH).integers(lo, hi + 1, size=n)]


def divergence_point(seed, lo, hi):
    return int(rng(seed, STREAM_DIVERGE).integers(lo, hi))


def linear_inputs(T, K, N, seed=0):
    """Inputs of a projection y = x w^T: x [T, K] ~ N(0,1) and w [N, K] ~ N(0, 1/K) (the usual
    1/sqrt(fan-in) init), both cast to bf16 with round-to-nearest-even."""
    x = cast(rng(seed, STREAM_PROJ_X).standard_normal((T, K)), torch.bfloat16)
    w = cast(rng(seed, STREAM_PROJ_W).standard_normal((N, K)) / np.sqrt(K), torch.bfloat16)
    return x, w


def attention_inputs(T, Hq, Hkv, D, seed=0):
    """Queries [T, Hq, D] and key / value caches [T, Hkv, D] for T positions, bf16.  q and k are
    N(0, 1) with a per-head scale drawn from [0.5, 2) (so that some heads attend sharply and
    others broadly at the usual 1/sqrt(D) score scale); v is N(0, 1)."""
    r = rng(seed, STREAM_ATT_Q)
    qs = 0.5 + 1.5 * r.random((1, Hq, 1))
    q = cast(r.standard_normal((T, Hq, D)) * qs, torch.bfloat16)
    r = rng(seed, STREAM_ATT_K)
    ks = 0.5 + 1.5 * r.random((1, Hkv, 1))
    k = cast(r.standard_normal((T, Hkv, D)) * ks, torch.bfloat16)
    v = cast(rng(seed, STREAM_ATT_V).standard_normal((T, Hkv, D)), torch.bfloat16)
    return q, k, v
