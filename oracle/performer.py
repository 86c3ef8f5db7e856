"""Performer (FAVOR+) coupling in fp64 -- test infrastructure only.

The pages compare the exact coupling with two linearized ones, linear
attention and Performer (ai4snews digest, "Synopsis"; project page,
"Abstract").  They print no formula for the latter; the reading taken here
is the published FAVOR+ estimator of the softmax kernel with positive random
features: for a softmax scale c (1/sqrt(d) as in the exact coupling) and m
random directions w_1..w_m (rows of W, m x d, drawn by the caller),

    phi(x)_i = exp(sqrt(c) w_i . x - c |x|^2 / 2) / sqrt(m),

so that E[phi(q) . phi(k)] = exp(c q . k) for w_i ~ N(0, I).  The coupling
is the linear-attention formula with these features:

    den_q = phi(q) . sum_j phi(k_j),   O_q = phi(q) (sum_j phi(k_j) v_j^T) / den_q.

The backward (W held fixed) is the chain rule written out, with
d phi_i / dx = phi_i (sqrt(c) w_i - c x).
"""

from __future__ import annotations

import numpy as np

__all__ = ["favor_features", "performer_fwd", "performer_bwd"]


def favor_features(X, W, scale) -> np.ndarray:
    """phi(X) [n x m] for rows X [n x d], directions W [m x d]."""
    X = np.asarray(X, np.float64)
    W = np.asarray(W, np.float64)
    sq = np.sqrt(scale)
    return np.exp(sq * (X @ W.T) - 0.5 * scale * np.sum(X * X, axis=1, keepdims=True)) / np.sqrt(W.shape[0])


def performer_fwd(Q, K, V, W, scale):
    """O [n_N x k] and ln(den) [n_N]."""
    V = np.asarray(V, np.float64)
    fQ, fK = favor_features(Q, W, scale), favor_features(K, W, scale)
    KV = fK.T @ V
    z = fK.sum(axis=0)
    den = fQ @ z
    return (fQ @ KV) / den[:, None], np.log(den)


def performer_bwd(Q, K, V, W, dO, scale):
    """dQ, dK, dV of sum(dO * O) for the forward above."""
    Q, K, V, W, dO = (np.asarray(a, np.float64) for a in (Q, K, V, W, dO))
    sq = np.sqrt(scale)
    fQ, fK = favor_features(Q, W, scale), favor_features(K, W, scale)
    KV = fK.T @ V
    z = fK.sum(axis=0)
    den = fQ @ z
    O = (fQ @ KV) / den[:, None]
    g = dO / den[:, None]                     # d/dA of O = A / den
    s = np.sum(dO * O, axis=1) / den          # -d/dden
    dfQ = g @ KV.T - s[:, None] * z[None, :]
    dKV = fQ.T @ g
    dz = -(fQ.T @ s)
    dV = fK @ dKV
    dfK = V @ dKV.T + dz[None, :]

    def through(dF, F, X):
        G = dF * F
        return sq * (G @ W) - scale * X * G.sum(axis=1, keepdims=True)

    return through(dfQ, fQ, Q), through(dfK, fK, K), dV
