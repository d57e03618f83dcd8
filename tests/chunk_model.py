"""float64 model of the chunked (WY/UT) form of the gated delta rule.

Used only by tests: it is an independent formulation of the same recurrence, so its
agreement with the per-token oracle (to float64 rounding) pins the oracle, and its
intermediates (cumulative gates, the triangular factor, the corrected values) describe what
the GPU kernels compute per 64-row sub-chunk.

For a sub-chunk of n rows (K, Q, V, beta, g) entered with state S:
    G_r = sum_{i<=r} g_i,  gamma_r = exp(G_r),  Gam_ri = exp(G_r - G_i) (i <= r)
    A = strict_lower(diag(beta) (K K^T) * Gam),   Tinv = (I + A)^-1
    D = Tinv diag(beta) (V - diag(gamma) K S)
    O = scale (diag(gamma) Q S + (lower(Q K^T) * Gam) D)
    S' = gamma_n S + (diag(exp(G_n - G)) K)^T D
"""
import numpy as np


def chunk_forward(q, k, v, g, beta, S0, scale, C):
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, S.shape[1]))
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C]
        b, gg = beta[c0:c0 + C], g[c0:c0 + C]
        n = Q.shape[0]
        G = np.cumsum(gg)
        diff = G[:, None] - G[None, :]
        low = np.tril(np.ones((n, n)))
        Gam = np.where(low > 0, np.exp(np.where(low > 0, diff, 0.0)), 0.0)
        A = np.tril(b[:, None] * (K @ K.T) * Gam, -1)
        Tinv = np.linalg.solve(np.eye(n) + A, np.eye(n))
        D = Tinv @ (b[:, None] * (V - np.exp(G)[:, None] * (K @ S)))
        O = scale * (np.exp(G)[:, None] * (Q @ S) + (np.tril(Q @ K.T) * Gam) @ D)
        S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * K).T @ D
        o[c0:c0 + n] = O
    return o, S
