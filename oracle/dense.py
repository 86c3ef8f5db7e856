"""Dense spatial-spectral coupling in fp64 -- test infrastructure only.

Definition (spatial-spectral-attention.github.io, "How it works": the product
Pi_NM Phi_M written out is scaled dot-product attention with Q = F_N,
K = F_M, V = Phi_M; "The bottleneck": Pi_NM has one row per target vertex and
one column per source vertex):

    S    = Q K^T * scale                    (n_N x n_M), scale = 1/sqrt(d)
    Pi   = row-wise softmax of S            (each row sums to 1)
    O    = Pi V                             (n_N x k)
    lse_i = log sum_j exp(S_ij)             (natural log; kept for backward)

Backward for an upstream gradient dO of O (chain rule through the softmax):

    D_i  = sum_c dO_ic O_ic
    dP   = dO V^T
    dS   = Pi * (dP - D)                    (elementwise, D broadcast per row)
    dQ   = scale * dS K,   dK = scale * dS^T Q,   dV = Pi^T dO

Rows are processed in blocks of whole rows, so no running max or rescaling
is needed: each block is the textbook softmax of complete rows.
"""

from __future__ import annotations

import numpy as np

__all__ = ["upcast", "dense_fwd", "dense_bwd", "dense_rows", "rowdot"]


def upcast(a, dtype: str) -> np.ndarray:
    """Stored input -> exact fp64.  bf16 arrives as uint16 bit patterns."""
    a = np.asarray(a)
    if dtype == "bf16":
        bits = a.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return a.astype(np.float64)
    raise ValueError(dtype)


def _softmax_rows(S: np.ndarray):
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    ell = E.sum(axis=1, keepdims=True)
    return E / ell, m[:, 0] + np.log(ell[:, 0])


def dense_fwd(Q, K, V, scale, block: int = 1024, return_P: bool = False):
    """O = softmax(Q K^T * scale) V and lse, in fp64.

    With return_P the whole map Pi (n_N x n_M) is also returned; only for
    small inputs.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n_N, n_M = Q.shape[0], K.shape[0]
    if n_M < 1:
        raise ValueError("the softmax needs at least one source vertex")
    O = np.zeros((n_N, V.shape[1]))
    lse = np.zeros(n_N)
    Ps = []
    for r0 in range(0, n_N, block):
        r1 = min(n_N, r0 + block)
        P, lse[r0:r1] = _softmax_rows((Q[r0:r1] @ K.T) * scale)
        O[r0:r1] = P @ V
        if return_P:
            Ps.append(P)
    if return_P:
        Pm = np.concatenate(Ps, axis=0) if Ps else np.zeros((0, n_M))
        return O, lse, Pm
    return O, lse


def dense_rows(Q, K, V, scale, rows):
    """O and lse for the listed target rows only (each row is independent)."""
    rows = np.asarray(rows, dtype=np.int64)
    return dense_fwd(np.asarray(Q, np.float64)[rows], K, V, scale)


def rowdot(dO, O):
    """D_i = sum_c dO_ic O_ic."""
    return np.einsum("ic,ic->i", np.asarray(dO, np.float64), np.asarray(O, np.float64))


def dense_bwd(Q, K, V, dO, scale, block: int = 1024, rows=None):
    """dQ, dK, dV of <dO, softmax(Q K^T scale) V>, in fp64.

    `rows` (optional) restricts the upstream gradient to those target rows,
    i.e. dO is taken as zero elsewhere: then only those rows contribute to dK
    and dV, and dQ is zero on every other row.  The forward quantities (Pi,
    O, D) are the oracle's own.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    n_N, n_M = Q.shape[0], K.shape[0]
    dQ = np.zeros_like(Q)
    dK = np.zeros((n_M, K.shape[1]))
    dV = np.zeros((n_M, V.shape[1]))
    sel = np.arange(n_N) if rows is None else np.unique(np.asarray(rows, np.int64))
    for b0 in range(0, len(sel), block):
        r = sel[b0:b0 + block]
        P, _ = _softmax_rows((Q[r] @ K.T) * scale)
        O = P @ V
        D = rowdot(dO[r], O)
        dP = dO[r] @ V.T
        dS = P * (dP - D[:, None])
        dQ[r] = scale * (dS @ K)
        dK += scale * (dS.T @ Q[r])
        dV += P.T @ dO[r]
    return dQ, dK, dV
