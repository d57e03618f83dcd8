"""Pins of the float64 oracle against facts fixed outside it (CPU only).

Each check is chosen so that a plausible mistake in the oracle fails at least one of them:
a dropped decay (beta=0 closed form), a wrong sign or placement of the delta correction
(retrieval invariant, hand-derived example), a transposed state (orthonormal keys with
d_k != d_v), output read before the update (single-token closed form), a wrong GQA map, a
wrong conv tap order or window (numpy.convolve, identity and shift taps), a wrong L2 eps.
Both oracle implementations (C and numpy) are pinned.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import c_oracle, numpy_ref
from tests.chunk_model import chunk_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, n, d):
    a = rng.standard_normal((n, d))
    return a / np.linalg.norm(a, axis=1, keepdims=True)


def run_head(impl, q, k, v, g, beta, S0, scale=1.0, eps=0.0):
    """One value head through the whole-layer entry (no conv) of either implementation."""
    T, dk = q.shape
    dv = v.shape[1]
    x = np.concatenate([q, k, v], axis=1)
    kw = dict(n_k_heads=1, n_v_heads=1, d_k=dk, d_v=dv, scale=scale, l2_eps=eps)
    if impl == "c":
        o, S, _ = c_oracle.gdn_layer(x, None, None, g[:, None], beta[:, None], S0[None], **kw)
    else:
        o, S, _ = numpy_ref.gdn_layer(x, None, None, g[:, None], beta[:, None], S0[None], **kw)
    return o[:, 0], S[0]


IMPLS = ["c", "np"]


def _load_golden():
    rows = {}
    with open(os.path.join(GOLDEN, "gdr_hand_2d.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = [float(Fraction(v)) for v in vals]
    return rows


@pytest.mark.parametrize("impl", IMPLS)
def test_hand_derived_example(impl):
    r = _load_golden()
    k = np.array(r["k"]).reshape(3, 2)
    v = np.array(r["v"]).reshape(3, 2)
    g = np.log(np.array(r["a"]))
    beta = np.array(r["b"])
    o, S = run_head(impl, k, k, v, g, beta, np.zeros((2, 2)))
    np.testing.assert_allclose(o, np.array(r["o"]).reshape(3, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, np.array(r["S"]).reshape(2, 2), rtol=0, atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS)
def test_beta_zero_is_pure_decay(impl):
    rng = np.random.default_rng(1)
    T, dk, dv = 9, 5, 3
    q = _unit(rng, T, dk)
    k = _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g = -rng.uniform(0.0, 0.7, T)
    S0 = rng.standard_normal((dk, dv))
    o, S = run_head(impl, q, k, v, g, np.zeros(T), S0, scale=0.7)
    G = np.cumsum(g)
    np.testing.assert_allclose(S, np.exp(G[-1]) * S0, rtol=1e-13, atol=0)
    np.testing.assert_allclose(o, 0.7 * np.exp(G)[:, None] * (q @ S0), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("impl", IMPLS)
def test_single_token_no_decay(impl):
    rng = np.random.default_rng(2)
    dk, dv = 6, 4
    q = _unit(rng, 1, dk)
    k = _unit(rng, 1, dk)
    v = rng.standard_normal((1, dv))
    o, S = run_head(impl, q, k, v, np.zeros(1), np.array([0.3]), np.zeros((dk, dv)), scale=0.5)
    np.testing.assert_allclose(S, 0.3 * np.outer(k[0], v[0]), rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(o[0], 0.5 * 0.3 * (q[0] @ k[0]) * v[0], rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("impl", IMPLS)
def test_beta_one_unit_key_retrieves_value(impl):
    """With beta=1 and a unit key the write is exact: S_t^T k_t = v_t whatever the decay."""
    rng = np.random.default_rng(3)
    T, dk, dv = 7, 5, 4
    k = _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g = -rng.uniform(0.1, 1.0, T)
    S0 = rng.standard_normal((dk, dv))
    for t in range(1, T + 1):
        # reading with q = k_t at the last token returns v_t
        q = k.copy()
        o, S = run_head(impl, q[:t], k[:t], v[:t], g[:t], np.ones(t), S0)
        np.testing.assert_allclose(o[t - 1], v[t - 1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S.T @ k[t - 1], v[t - 1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS)
def test_orthonormal_keys_store_outer_products(impl):
    """Orthonormal keys, g=0, beta=1, S0=0: S = sum_t e_t v_t^T (d_k != d_v catches a transpose)."""
    rng = np.random.default_rng(4)
    dk, dv, T = 6, 3, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T]
    v = rng.standard_normal((T, dv))
    o, S = run_head(impl, k, k, v, np.zeros(T), np.ones(T), np.zeros((dk, dv)))
    np.testing.assert_allclose(S, k.T @ v, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS)
def test_zero_key_is_decay_only(impl):
    rng = np.random.default_rng(5)
    T, dk, dv = 5, 4, 4
    q = _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g = -rng.uniform(0.0, 1.0, T)
    S0 = rng.standard_normal((dk, dv))
    o, S = run_head(impl, q, np.zeros((T, dk)), v, g, rng.uniform(0, 1, T), S0, eps=1e-6)
    np.testing.assert_allclose(S, np.exp(g.sum()) * S0, rtol=1e-13)


def _explicit_products(q, k, v, g, beta, S0, scale):
    """Brute force: S_T = P_T..P_1 S0 + sum_t (P_T..P_{t+1}) b_t k_t v_t^T, P_t = a_t(I - b_t k k^T)."""
    T, dk = k.shape
    outs = []
    for n in range(1, T + 1):
        P = [np.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(n)]
        S = np.linalg.multi_dot([*reversed(P), S0]) if n > 1 else P[0] @ S0
        for t in range(n):
            tail = np.eye(dk)
            for s in range(t + 1, n):
                tail = P[s] @ tail
            S = S + tail @ (beta[t] * np.outer(k[t], v[t]))
        outs.append((scale * S.T @ q[n - 1], S))
    return np.array([a for a, _ in outs]), outs[-1][1]


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("T,dk,dv", [(1, 3, 2), (4, 5, 3), (8, 8, 8), (6, 2, 7)])
def test_brute_force_matrix_products(impl, T, dk, dv):
    rng = np.random.default_rng(10 + T + dk)
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    g = -np.logaddexp(0, rng.standard_normal(T))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((dk, dv))
    o_ref, S_ref = _explicit_products(q, k, v, g, beta, S0, 0.8)
    o, S = run_head(impl, q, k, v, g, beta, S0, scale=0.8)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("impl", IMPLS)
def test_linear_in_state_and_values(impl):
    rng = np.random.default_rng(6)
    T, dk, dv = 12, 6, 5
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    g = -np.logaddexp(0, rng.standard_normal(T))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    v1, v2 = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    S1, S2 = rng.standard_normal((dk, dv)), rng.standard_normal((dk, dv))
    a, b = 0.7, -1.3
    o1, F1 = run_head(impl, q, k, v1, g, beta, S1)
    o2, F2 = run_head(impl, q, k, v2, g, beta, S2)
    o3, F3 = run_head(impl, q, k, a * v1 + b * v2, g, beta, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(F3, a * F1 + b * F2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS)
def test_value_columns_independent(impl):
    """Column j of S and o depends only on column j of S0 and v (permutation equivariance)."""
    rng = np.random.default_rng(7)
    T, dk, dv = 10, 4, 6
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    g = -np.logaddexp(0, rng.standard_normal(T))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    v = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((dk, dv))
    perm = rng.permutation(dv)
    o, S = run_head(impl, q, k, v, g, beta, S0)
    op, Sp = run_head(impl, q, k, v[:, perm], g, beta, S0[:, perm])
    np.testing.assert_allclose(op, o[:, perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sp, S[:, perm], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("C", [1, 3, 64, 100])
def test_chunk_form_equals_per_token(C):
    """The chunked (WY/UT) algebra, derived separately, reaches the per-token result."""
    rng = np.random.default_rng(8)
    T, d = 300, 64
    q, k = _unit(rng, T, d), _unit(rng, T, d)
    v = rng.standard_normal((T, d))
    g = -np.logaddexp(0, rng.standard_normal(T))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((d, d)) * 0.1
    o_ref, S_ref = run_head("c", q, k, v, g, beta, S0, scale=d ** -0.5)
    o, S = chunk_forward(q, k, v, g, beta, S0, d ** -0.5, C)
    assert np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref) < 1e-13
    assert np.linalg.norm(S - S_ref) / np.linalg.norm(S_ref) < 1e-13


# ---------------------------------------------------------------- conv and L2 norm


def _conv_impl(impl, x, w, window, silu=False):
    if impl == "c":
        return c_oracle.causal_conv(x, w, window, silu)
    return numpy_ref.causal_conv(x, w, window, silu)


@pytest.mark.parametrize("impl", IMPLS)
def test_conv_matches_numpy_convolve(impl):
    rng = np.random.default_rng(20)
    T, C, W = 17, 5, 4
    x, w = rng.standard_normal((T, C)), rng.uniform(-0.5, 0.5, (C, W))
    win = rng.standard_normal((W - 1, C))
    y, wo = _conv_impl(impl, x, w, win)
    xt = np.concatenate([win, x])
    for c in range(C):
        np.testing.assert_allclose(y[:, c], np.convolve(xt[:, c], w[c, ::-1], "valid"),
                                   rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(wo, x[-3:])


@pytest.mark.parametrize("impl", IMPLS)
def test_conv_identity_and_shift_taps(impl):
    rng = np.random.default_rng(21)
    T, C = 6, 3
    x, win = rng.standard_normal((T, C)), rng.standard_normal((3, C))
    y, _ = _conv_impl(impl, x, np.tile([0.0, 0.0, 0.0, 1.0], (C, 1)), win)
    np.testing.assert_array_equal(y, x)
    y, _ = _conv_impl(impl, x, np.tile([1.0, 0.0, 0.0, 0.0], (C, 1)), win)
    np.testing.assert_array_equal(y, np.concatenate([win, x])[:T])


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("T", [0, 1, 2, 3, 5])
def test_conv_window_carries_across_splits(impl, T):
    """Splitting the stream anywhere and carrying the window equals one call (also T < 3)."""
    rng = np.random.default_rng(22 + T)
    C = 4
    x = rng.standard_normal((T + 7, C))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    win = rng.standard_normal((3, C))
    y_all, wo_all = _conv_impl(impl, x, w, win)
    y1, wo1 = _conv_impl(impl, x[:T], w, win)
    y2, wo2 = _conv_impl(impl, x[T:], w, wo1)
    np.testing.assert_array_equal(np.concatenate([y1, y2]), y_all)
    np.testing.assert_array_equal(wo2, wo_all)
    if T < 3:  # the window shifts: old rows then new inputs
        np.testing.assert_array_equal(wo1, np.concatenate([win, x[:T]])[-3:])


def test_conv_silu_flag():
    rng = np.random.default_rng(23)
    x, w, win = rng.standard_normal((9, 3)), rng.uniform(-1, 1, (3, 4)), np.zeros((3, 3))
    y0, _ = c_oracle.causal_conv(x, w, win, False)
    y1, _ = c_oracle.causal_conv(x, w, win, True)
    np.testing.assert_allclose(y1, y0 * 0.5 * (1 + np.tanh(y0 / 2)), rtol=1e-13, atol=1e-15)


def test_l2norm_closed_form():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((11, 7)) * rng.uniform(0.01, 10, (11, 1))
    eps = 1e-3
    y = numpy_ref.l2norm(x, eps)
    n2 = (x * x).sum(1)
    np.testing.assert_allclose((y * y).sum(1), n2 / (n2 + eps), rtol=1e-13)
    # same direction
    np.testing.assert_allclose(y / np.linalg.norm(y, axis=1, keepdims=True),
                               x / np.linalg.norm(x, axis=1, keepdims=True), rtol=1e-13)


def test_layer_l2norm_eps_and_scale():
    """The layer normalises q and k with eps inside the root, and o is linear in scale."""
    rng = np.random.default_rng(25)
    T, d = 3, 4
    q = rng.standard_normal((T, d)) * 0.01   # small norms make eps visible
    k = np.zeros((T, d))
    k[:, 0] = 0.02
    v = rng.standard_normal((T, d))
    eps = 1e-4
    o, S = run_head("c", q, k, v, np.zeros(T), np.ones(T), np.zeros((d, d)), scale=2.0, eps=eps)
    kn = k / np.sqrt((k * k).sum(1, keepdims=True) + eps)
    qn = q / np.sqrt((q * q).sum(1, keepdims=True) + eps)
    on, Sn = numpy_ref.gated_delta_rule(qn, kn, v, np.zeros(T), np.ones(T), np.zeros((d, d)), 2.0)
    np.testing.assert_allclose(o, on, rtol=1e-12, atol=1e-15)
    o1, _ = run_head("c", q, k, v, np.zeros(T), np.ones(T), np.zeros((d, d)), scale=1.0, eps=eps)
    np.testing.assert_allclose(o, 2.0 * o1, rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("impl", IMPLS)
def test_gqa_value_head_uses_key_head_h_div_group(impl):
    """Hv = 2 Hk: value heads 2j and 2j+1 read key head j."""
    rng = np.random.default_rng(26)
    T, Hk, Hv, d = 6, 2, 4, 3
    x = rng.standard_normal((T, 2 * Hk * d + Hv * d))
    g = -np.logaddexp(0, rng.standard_normal((T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    S0 = rng.standard_normal((Hv, d, d))
    kw = dict(n_k_heads=Hk, n_v_heads=Hv, d_k=d, d_v=d, scale=0.9, l2_eps=1e-6)
    f = c_oracle.gdn_layer if impl == "c" else numpy_ref.gdn_layer
    o, S, _ = f(x, None, None, g, beta, S0, **kw)
    for h in range(Hv):
        j = h // 2
        qh = x[:, j * d:(j + 1) * d]
        kh = x[:, (Hk + j) * d:(Hk + j + 1) * d]
        vh = x[:, 2 * Hk * d + h * d:2 * Hk * d + (h + 1) * d]
        oh, Sh = run_head(impl, qh, kh, vh, g[:, h], beta[:, h], S0[h], scale=0.9, eps=1e-6)
        np.testing.assert_allclose(o[:, h], oh, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(S[h], Sh, rtol=1e-13, atol=1e-15)


def test_c_and_numpy_implementations_agree_with_conv():
    rng = np.random.default_rng(27)
    T, Hk, Hv, d = 21, 2, 4, 8
    C = 2 * Hk * d + Hv * d
    x = rng.standard_normal((T, C))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    win = rng.standard_normal((3, C))
    g = -np.logaddexp(0, rng.standard_normal((T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    S0 = rng.standard_normal((Hv, d, d))
    kw = dict(n_k_heads=Hk, n_v_heads=Hv, d_k=d, d_v=d, scale=d ** -0.5, l2_eps=1e-6)
    a = c_oracle.gdn_layer(x, w, win, g, beta, S0, **kw)
    b = numpy_ref.gdn_layer(x, w, win, g, beta, S0, **kw)
    for u, v in zip(a, b):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-14)


def test_oracle_bitwise_invariant_to_call_splits():
    """The per-token oracle runs the same operations however the rows are split into calls."""
    rng = np.random.default_rng(28)
    T, Hk, Hv, d = 40, 1, 2, 8
    C = 2 * Hk * d + Hv * d
    x = rng.standard_normal((T, C))
    w = rng.uniform(-0.5, 0.5, (C, 4))
    g = -np.logaddexp(0, rng.standard_normal((T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    kw = dict(n_k_heads=Hk, n_v_heads=Hv, d_k=d, d_v=d, scale=0.3, l2_eps=1e-6)
    S0 = np.zeros((Hv, d, d))
    o, S, wo = c_oracle.gdn_layer(x, w, np.zeros((3, C)), g, beta, S0, **kw)
    cut = 13
    o1, S1, w1 = c_oracle.gdn_layer(x[:cut], w, np.zeros((3, C)), g[:cut], beta[:cut], S0, **kw)
    o2, S2, w2 = c_oracle.gdn_layer(x[cut:], w, w1, g[cut:], beta[cut:], S1, **kw)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(S2, S)
    assert np.array_equal(w2, wo)


def test_head_subset_matches_full_run():
    rng = np.random.default_rng(29)
    T, Hk, Hv, d = 10, 2, 4, 4
    C = 2 * Hk * d + Hv * d
    x = rng.standard_normal((T, C))
    g = -np.logaddexp(0, rng.standard_normal((T, Hv)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Hv))))
    S0 = rng.standard_normal((Hv, d, d))
    kw = dict(n_k_heads=Hk, n_v_heads=Hv, d_k=d, d_v=d, scale=0.5, l2_eps=1e-6)
    o, S, _ = c_oracle.gdn_layer(x, None, None, g, beta, S0, **kw)
    os_, Ss, _ = c_oracle.gdn_layer(x, None, None, g, beta, S0, heads=[3, 1], **kw)
    for h in (1, 3):
        assert np.array_equal(os_[:, h], o[:, h]) and np.array_equal(Ss[h], S[h])


def test_linear_against_brute_force_and_closed_forms():
    """The projection's oracle against a triple loop, identity and permutation weights, and
    linearity: a transposed operand or a dropped term fails one of these."""
    from oracle import numpy_ref
    r = np.random.default_rng(7)
    x = r.standard_normal((5, 8))
    w = r.standard_normal((3, 8))
    y = numpy_ref.linear(x, w)
    for t in range(5):
        for n in range(3):
            s = 0.0
            for k in range(8):
                s += x[t, k] * w[n, k]
            assert abs(y[t, n] - s) < 1e-12
    assert np.array_equal(numpy_ref.linear(x, np.eye(8)), x)
    perm = np.eye(8)[[3, 1, 7]]  # rows pick input columns 3, 1, 7
    assert np.array_equal(numpy_ref.linear(x, perm), x[:, [3, 1, 7]])
    x2 = r.standard_normal((5, 8))
    assert np.allclose(numpy_ref.linear(2 * x + x2, w), 2 * y + numpy_ref.linear(x2, w), atol=1e-12)
    assert numpy_ref.linear(x, w).shape == (5, 3)


def test_attention_against_brute_force_loops():
    """Explicit loops with math.exp on a tiny case with grouped heads and cached rows."""
    import math
    from oracle import numpy_ref
    r = np.random.default_rng(11)
    T, Hq, Hkv, D, pos0 = 3, 4, 2, 5, 2
    q = r.standard_normal((T, Hq, D))
    k = r.standard_normal((pos0 + T, Hkv, D))
    v = r.standard_normal((pos0 + T, Hkv, D))
    scale = 0.37
    o = numpy_ref.attention(q, k, v, pos0, scale)
    for t in range(T):
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            w = []
            for j in range(pos0 + t + 1):
                w.append(math.exp(scale * sum(q[t, h, d] * k[j, kv, d] for d in range(D))))
            for d in range(D):
                ref = sum(w[j] * v[j, kv, d] for j in range(len(w))) / sum(w)
                assert abs(o[t, h, d] - ref) < 1e-12


def test_attention_closed_forms():
    """The first position sees only itself; a zero query averages the values it can see; a key
    far ahead of the others in score takes all the weight; heads read key head h // ratio."""
    from oracle import numpy_ref
    r = np.random.default_rng(12)
    T, Hq, Hkv, D = 6, 4, 2, 8
    q = r.standard_normal((T, Hq, D))
    k = r.standard_normal((T, Hkv, D))
    v = r.standard_normal((T, Hkv, D))
    o = numpy_ref.attention(q, k, v, 0, 0.3)
    for h in range(Hq):
        assert np.array_equal(o[0, h], v[0, h // 2])
    oz = numpy_ref.attention(np.zeros_like(q), k, v, 0, 0.3)
    for t in range(T):
        assert np.allclose(oz[t, 0], v[:t + 1, 0].mean(axis=0), atol=1e-14)
        assert np.allclose(oz[t, 3], v[:t + 1, 1].mean(axis=0), atol=1e-14)
    k2 = k.copy()
    k2[2, 0] = 50.0 * q[5, 1] / np.linalg.norm(q[5, 1])  # head 1 reads key head 0
    o2 = numpy_ref.attention(q, k2, v, 0, 1.0)
    assert np.allclose(o2[5, 1], v[2, 0], atol=1e-9)
    # grouped heads: each query head alone against its own key head
    for h in range(Hq):
        alone = numpy_ref.attention(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1],
                                    0, 0.3)
        assert np.allclose(alone[:, 0], o[:, h], atol=1e-14)


def test_attention_continuation_from_cached_rows():
    """Rows a .. T-1 run from position a over the same cache equal those rows of one pass."""
    from oracle import numpy_ref
    r = np.random.default_rng(13)
    T, D = 9, 4
    q = r.standard_normal((T, 2, D))
    k = r.standard_normal((T, 1, D))
    v = r.standard_normal((T, 1, D))
    full = numpy_ref.attention(q, k, v, 0, 0.5)
    for a in (1, 4, 8):
        part = numpy_ref.attention(q[a:], k, v, a, 0.5)
        assert np.allclose(part, full[a:], atol=1e-14)
