"""Linear-attention coupling (ELU feature map) in fp64 -- test infrastructure only.

The pages compare the exact coupling with linearized couplings that replace
the softmax by a low-rank feature map (ai4snews digest, "Interpretation";
project page, "Runtime and memory", Table 1 row "Linear attention (ELU)").
The pages give no formula beyond that; the reading taken here is the
standard ELU linear attention (Katharopoulos et al. 2020), applied to the raw
descriptors with no score scale:

    phi(x) = elu(x) + 1  = x + 1 if x > 0 else exp(x)      (elementwise, > 0)
    W_ij   = phi(q_i) . phi(k_j) / sum_j' phi(q_i) . phi(k_j')
    O      = W V                                            (n_N x k)

computed through the associativity that makes it linear in n:

    KV  = phi(K)^T V      (d x k),      z = phi(K)^T 1      (d)
    den_i = phi(q_i) . z,                O_i = phi(q_i) KV / den_i

Backward for an upstream gradient dO (chain rule written out):

    g_i   = dO_i / den_i,                s_i = (dO_i . O_i) / den_i
    dA_i  = KV g_i - s_i z               (gradient w.r.t. phi(q_i))
    dKV   = sum_i phi(q_i) g_i^T,        dz = -sum_i s_i phi(q_i)
    dQ    = phi'(Q) * dA,                phi'(x) = 1 if x > 0 else exp(x)
    dK_j  = phi'(k_j) * (dKV v_j + dz),  dV_j = dKV^T phi(k_j)

`linear_weights` materialises W for small inputs (a second route, used by
the tests to pin the factorised form).
"""

from __future__ import annotations

import numpy as np

from .dense import upcast

__all__ = ["elu1", "elu1_grad", "linear_fwd", "linear_bwd", "linear_weights"]


def elu1(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def elu1_grad(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def linear_fwd(Q, K, V):
    """O [n_N x k] and den [n_N] (fp64) of the ELU linear coupling."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    fK = elu1(K)
    KV = fK.T @ V
    z = fK.sum(axis=0)
    fQ = elu1(Q)
    den = fQ @ z
    return (fQ @ KV) / den[:, None], den


def linear_bwd(Q, K, V, dO):
    """dQ, dK, dV (fp64) of <dO, O> for the ELU linear coupling."""
    Q, K, V, dO = (np.asarray(x, np.float64) for x in (Q, K, V, dO))
    fK, fQ = elu1(K), elu1(Q)
    KV = fK.T @ V
    z = fK.sum(axis=0)
    den = fQ @ z
    O = (fQ @ KV) / den[:, None]
    g = dO / den[:, None]
    s = np.sum(dO * O, axis=1) / den
    dA = g @ KV.T - s[:, None] * z[None, :]
    dKV = fQ.T @ g
    dz = -(fQ.T @ s)
    dQ = elu1_grad(Q) * dA
    dK = elu1_grad(K) * (V @ dKV.T + dz[None, :])
    dV = fK @ dKV
    return dQ, dK, dV


def linear_weights(Q, K):
    """The coupling matrix W [n_N x n_M] itself (small inputs only)."""
    A = elu1(Q) @ elu1(K).T
    return A / A.sum(axis=1, keepdims=True)
