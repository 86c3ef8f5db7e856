"""Geo-FlashAttention coupling in fp64 -- test infrastructure only.

The pipeline (spatial-spectral-attention.github.io, "Geo-FlashAttention" and
its pipeline figure; ai4snews digest, "Interpretation"): partition both
shapes into geodesic patches, pool the source keys per patch, score the
source patches from the descriptors, keep the top R (here s) source patches
per target patch, and take the exact softmax of every target row over the
union of its patch's selected source patches only.

Readings where the pages are silent (each is listed in the design notes):
* pooling is the patch mean, on both shapes; the score of (target patch p,
  source patch q) is the unscaled dot product of the two means;
* the top-s order is (score descending, source index ascending), so ties go
  to the lower index and the selection is unique;
* the backward treats the selection as fixed (it is piecewise constant);
* an empty patch has a zero mean; a target row whose support is empty gets
  O = 0, lse = -inf and zero gradients.

Everything runs in the ORIGINAL vertex order from per-vertex labels, so a
patch-sorted implementation is checked against an independent layout.
"""

from __future__ import annotations

import numpy as np

__all__ = ["patch_means", "patch_scores", "topk", "cut_gaps", "geo_support",
           "geo_fwd", "geo_bwd", "executed_pairs"]


def patch_means(X, labels, P: int) -> np.ndarray:
    """Mean descriptor of each patch (fp64 [P, d]); empty patch -> 0."""
    X = np.asarray(X, np.float64)
    labels = np.asarray(labels, np.int64)
    sums = np.zeros((P, X.shape[1]))
    np.add.at(sums, labels, X)
    cnt = np.bincount(labels, minlength=P).astype(np.float64)
    out = np.zeros_like(sums)
    nz = cnt > 0
    out[nz] = sums[nz] / cnt[nz, None]
    return out


def patch_scores(Qbar, Kbar) -> np.ndarray:
    """C[p, q] = <Qbar_p, Kbar_q>  (fp64 [P_N, P_M])."""
    return np.asarray(Qbar, np.float64) @ np.asarray(Kbar, np.float64).T


def topk(C, s: int) -> np.ndarray:
    """Row-wise top-s source indices ordered by (score desc, index asc)."""
    C = np.asarray(C, np.float64)
    P_N, P_M = C.shape
    if not (1 <= s <= P_M):
        raise ValueError("need 1 <= s <= P_M")
    q = np.arange(P_M)
    out = np.empty((P_N, s), dtype=np.int32)
    for p in range(P_N):
        out[p] = np.lexsort((q, -C[p]))[:s]
    return out


def cut_gaps(C, s: int) -> np.ndarray:
    """Per row: (s-th largest score) - ((s+1)-th largest); +inf when s = P_M."""
    C = np.asarray(C, np.float64)
    srt = -np.sort(-C, axis=1)
    if s >= C.shape[1]:
        return np.full(C.shape[0], np.inf)
    return srt[:, s - 1] - srt[:, s]


def geo_support(labN, labM, idx):
    """For each target patch p: (rows T_p, source rows J_p), ascending."""
    labN = np.asarray(labN, np.int64)
    labM = np.asarray(labM, np.int64)
    out = []
    for p in range(idx.shape[0]):
        T = np.nonzero(labN == p)[0]
        J = np.nonzero(np.isin(labM, idx[p]))[0]
        out.append((T, J))
    return out


def executed_pairs(labN, labM, idx) -> int:
    """sum_p |T_p| * |J_p|: the (target, source) pairs the softmax visits."""
    return int(sum(len(T) * len(J) for T, J in geo_support(labN, labM, idx)))


def geo_fwd(Q, K, V, labN, labM, idx, scale):
    """O, lse of the selected-support coupling (fp64, original order)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    O = np.zeros((Q.shape[0], V.shape[1]))
    lse = np.full(Q.shape[0], -np.inf)
    for T, J in geo_support(labN, labM, idx):
        if len(T) == 0 or len(J) == 0:
            continue
        S = (Q[T] @ K[J].T) * scale
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        ell = E.sum(axis=1, keepdims=True)
        O[T] = (E / ell) @ V[J]
        lse[T] = m[:, 0] + np.log(ell[:, 0])
    return O, lse


def geo_bwd(Q, K, V, dO, labN, labM, idx, scale):
    """dQ, dK, dV of <dO, O_geo> for a fixed selection (fp64, original order).

    Source rows outside every selected support get zero dK and dV.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros((K.shape[0], V.shape[1]))
    for T, J in geo_support(labN, labM, idx):
        if len(T) == 0 or len(J) == 0:
            continue
        S = (Q[T] @ K[J].T) * scale
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        P = E / E.sum(axis=1, keepdims=True)
        O = P @ V[J]
        D = np.einsum("ic,ic->i", dO[T], O)
        dS = P * (dO[T] @ V[J].T - D[:, None])
        dQ[T] = scale * (dS @ K[J])
        dK[J] += scale * (dS.T @ Q[T])
        dV[J] += P.T @ dO[T]
    return dQ, dK, dV
