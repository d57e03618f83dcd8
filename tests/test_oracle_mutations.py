"""The pins catch plausible oracle mistakes (CPU only).

Each mutant below is a wrong variant of the per-token recurrence, planted in a local copy on
the CPU; the checks are the same closed forms and brute-force products that pin the real
oracle.  Every mutant must fail at least one check, and the correct rule must pass them all.
"""
import numpy as np
import pytest

from oracle import numpy_ref


def rule(q, k, v, g, beta, S0, scale, variant=None):
    S = np.array(S0, dtype=np.float64, copy=True)
    T = q.shape[0]
    o = np.zeros((T, S.shape[1]))
    for t in range(T):
        a = np.exp(g[t])
        if variant == "no_decay_on_correction":       # a S + b k (v - S^T k)^T, S undecayed in e
            e = v[t] - S.T @ k[t]
            S = a * S + beta[t] * np.outer(k[t], e)
        elif variant == "plus_sign":                  # e = v + S^T k
            S *= a
            S += beta[t] * np.outer(k[t], v[t] + S.T @ k[t])
        elif variant == "output_before_update":
            o[t] = scale * (a * S).T @ q[t]
            S *= a
            S += beta[t] * np.outer(k[t], v[t] - S.T @ k[t])
            continue
        elif variant == "decay_after_write":
            S += beta[t] * np.outer(k[t], v[t] - S.T @ k[t])
            S *= a
        elif variant == "missing_beta_on_correction":
            S *= a
            S += np.outer(k[t], beta[t] * v[t] - S.T @ k[t])
        elif variant == "transposed_state":           # state read as [d_v][d_k] (square dims)
            S *= a
            S += beta[t] * np.outer(k[t], v[t] - S @ k[t])
            o[t] = scale * (S @ q[t])
            continue
        else:
            S *= a
            S += beta[t] * np.outer(k[t], v[t] - S.T @ k[t])
        o[t] = scale * (S.T @ q[t])
    return o, S


def _unit(rng, n, d):
    a = rng.standard_normal((n, d))
    return a / np.linalg.norm(a, axis=1, keepdims=True)


def checks(f):
    """Return the names of the pin checks that the rule f fails (a shape error is a failure)."""
    failed = []
    rng = np.random.default_rng(0)
    T, dk, dv = 6, 5, 3
    q, k, v = _unit(rng, T, dk), _unit(rng, T, dk), rng.standard_normal((T, dv))
    g = -rng.uniform(0.1, 0.7, T)
    S0 = rng.standard_normal((dk, dv))
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    d = 4
    kq = _unit(rng, 5, d)
    vs = rng.standard_normal((5, d))
    S0s = rng.standard_normal((d, d))
    gs = -rng.uniform(0.1, 0.7, 5)

    def beta0():            # beta = 0: pure decay
        o, S = f(q, k, v, g, np.zeros(T), S0, 1.0)
        return np.allclose(S, np.exp(g.sum()) * S0, rtol=1e-12)

    def retrieval():        # beta = 1, unit key, q = k: the output is the value
        o, S = f(k, k, v, g, np.ones(T), S0, 1.0)
        return np.allclose(o, v, rtol=1e-10, atol=1e-10)

    def single_token():     # one token, g = 0: S = beta k v^T
        o, S = f(q[:1], k[:1], v[:1], np.zeros(1), np.array([0.3]), np.zeros((dk, dv)), 0.5)
        return np.allclose(o[0], 0.5 * 0.3 * (q[0] @ k[0]) * v[0], rtol=1e-12, atol=1e-14)

    def orthonormal():      # orthonormal keys, beta = 1, d_k != d_v: S = K^T V
        o, S = f(Qm[:3], Qm[:3], v[:3], np.zeros(3), np.ones(3), np.zeros((dk, dv)), 1.0)
        return np.allclose(S, Qm[:3].T @ v[:3], rtol=1e-12, atol=1e-12)

    def retrieval_square(): # square dims, non-symmetric start state: retrieval still exact
        o, S = f(kq, kq, vs, gs, np.ones(5), S0s, 1.0)
        return np.allclose(o, vs, rtol=1e-10, atol=1e-10)

    for check in (beta0, retrieval, single_token, orthonormal, retrieval_square):
        try:
            ok = check()
        except ValueError:
            ok = False
        if not ok:
            failed.append(check.__name__)
    return failed


def test_correct_rule_passes_every_check():
    assert checks(lambda *a: rule(*a)) == []
    assert checks(lambda q, k, v, g, b, S0, sc: numpy_ref.gated_delta_rule(q, k, v, g, b, S0, sc)) == []


@pytest.mark.parametrize("variant", ["no_decay_on_correction", "plus_sign", "output_before_update",
                                     "decay_after_write", "missing_beta_on_correction",
                                     "transposed_state"])
def test_each_mutant_fails_some_check(variant):
    assert checks(lambda *a: rule(*a, variant=variant)), variant
