"""numpy float64 twin of the oracle, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each function restates, in float64 and one token at a time, a step of the layer whose state
the pages keep: the conv window holding the three most recent conv inputs (PR "qwen3_5: run prompts
that share prefixes once per prefix", section Purpose), and the gated delta rule's fp32
recurrent state (named in "The shadow reader", section "One session's state", and in "Long
context and sessions", section Checkpoints; its update equation is not printed on the pages:
the standard gated delta rule is used, read as decay first, then the delta-rule write).
"""
import numpy as np


def causal_conv(x, w, window, silu=False):
    """Causal depthwise conv, width W = w.shape[1], state = the last W-1 inputs.

    x [T, C], w [C, W], window [W-1, C] (oldest row first).  With xt = window ++ x,
    y[t, c] = sum_j w[c, j] * xt[t + j, c] (tap W-1 is the current token).
    Returns (y [T, C], new window = last W-1 rows of xt).
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    window = np.asarray(window, np.float64)
    T, C = x.shape
    W = w.shape[1]
    xt = np.concatenate([window, x], axis=0)
    y = np.zeros((T, C))
    for t in range(T):
        for j in range(W):
            y[t] += w[:, j] * xt[t + j]
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y, xt[xt.shape[0] - (W - 1):].copy()


def l2norm(x, eps):
    """Row-wise x / sqrt(sum x^2 + eps) over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def gated_delta_rule(q, k, v, g, beta, S0, scale):
    """One value head, token by token.

    q, k [T, dk] (already normalised), v [T, dv], g, beta [T], S0 [dk, dv].
    S <- exp(g_t) S;  e <- v_t - S^T k_t;  S <- S + beta_t k_t e^T;  o_t <- scale S^T q_t.
    Returns (o [T, dv], S_T).
    """
    S = np.array(S0, np.float64, copy=True)
    T = q.shape[0]
    o = np.zeros((T, S.shape[1]))
    for t in range(T):
        S *= np.exp(g[t])
        e = v[t] - S.T @ k[t]
        S += beta[t] * np.outer(k[t], e)
        o[t] = scale * (S.T @ q[t])
    return o, S


def split_qkv(y, n_k_heads, n_v_heads, d_k, d_v):
    """Split channels [T, C] into q, k [T, Hk, dk] and v [T, Hv, dv] (q | k | v order)."""
    T = y.shape[0]
    a = n_k_heads * d_k
    q = y[:, :a].reshape(T, n_k_heads, d_k)
    k = y[:, a:2 * a].reshape(T, n_k_heads, d_k)
    v = y[:, 2 * a:2 * a + n_v_heads * d_v].reshape(T, n_v_heads, d_v)
    return q, k, v


def gdn_layer(x, conv_w, window, g, beta, S0, *, n_k_heads, n_v_heads, d_k, d_v,
              scale, l2_eps, conv_silu=False):
    """Whole layer: conv (skipped when conv_w is None) -> L2 norm -> gated delta rule.

    x [T, C]; g, beta [T, Hv]; S0 [Hv, dk, dv].  Value head h reads key head
    h // (Hv // Hk).  Returns (o [T, Hv, dv], S [Hv, dk, dv], new window or None).
    """
    x = np.asarray(x, np.float64)
    if conv_w is not None:
        y, win = causal_conv(x, conv_w, window, conv_silu)
    else:
        y, win = x, None
    q, k, v = split_qkv(y, n_k_heads, n_v_heads, d_k, d_v)
    qn, kn = l2norm(q, l2_eps), l2norm(k, l2_eps)
    group = n_v_heads // n_k_heads
    T = x.shape[0]
    o = np.zeros((T, n_v_heads, d_v))
    S = np.zeros((n_v_heads, d_k, d_v))
    for h in range(n_v_heads):
        kh = h // group
        o[:, h], S[h] = gated_delta_rule(qn[:, kh], kn[:, kh], v[:, h], np.asarray(g)[:, h],
                                         np.asarray(beta)[:, h], S0[h], scale)
    return o, S, win


def linear(x, w):
    """The projections around the layer: y[t, n] = sum_k x[t, k] w[n, k] (w as stored by a
    linear layer, one row per output), in float64.  The pages fix one summation order per
    weight shape so that grouped runs equal a plain pass (PR "qwen3_5: run prompts that share
    prefixes once per prefix", section Purpose, "GEMMs"); the exact sum has no order."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    return x @ w.T


def attention(q, k, v, pos0, scale):
    """Causal softmax attention of the full-attention layers, in float64: the query at absolute
    position p = pos0 + t attends to keys 0 .. p, and query head h reads key head
    h // (Hq / Hkv).  o[t, h] = sum_j softmax_j(scale q[t, h] . k[j, h']) v[j, h'].  The pages
    compute it as split-K flash attention with an online softmax ("Long context and sessions",
    section "The KV cache"); rescaling by a running max changes only rounding, so the exact
    result is the plain definition written here.

    q [T, Hq, D]; k, v [>= pos0 + T, Hkv, D]; returns o [T, Hq, D]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    R = Hq // Hkv
    o = np.zeros((T, Hq, D))
    for h in range(Hq):
        kh, vh = k[:, h // R, :], v[:, h // R, :]
        for t in range(T):
            n = pos0 + t + 1
            s = scale * (kh[:n] @ q[t, h])
            w = np.exp(s - s.max())
            o[t, h] = (w / w.sum()) @ vh[:n]
    return o
