"""Pins of the Geo-FlashAttention fp64 oracle.

Pipeline (spatial-spectral-attention.github.io, "Geo-FlashAttention"):
patches -> pooled keys -> patch scores -> top-s per target patch -> exact
softmax on the selected support.  Pins: brute-force means and dot products,
Python's `sorted` on (-score, index) with constructed exact ties, the
special cases s = P_M (geo == dense) and one patch per shape, torch's CPU
scaled_dot_product_attention with a boolean support mask (fp64, autograd),
central finite differences at a fixed selection, and the zero gradient of
source rows outside every support.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (cut_gaps, dense_bwd, dense_fwd, executed_pairs, geo_bwd, geo_fwd,
                    patch_means, patch_scores, topk)


def rnd(seed, *shape, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def labels(seed, n, P):
    lab = np.random.default_rng(seed).integers(0, P, n)
    lab[:P] = np.arange(P)  # every patch non-empty
    return np.random.default_rng(seed + 1).permutation(lab).astype(np.int32)


def test_patch_means_brute_force():
    X = rnd(1, 40, 5)
    lab = labels(2, 40, 6)
    M = patch_means(X, lab, 7)  # patch 6 is empty
    for p in range(6):
        rows = [i for i in range(40) if lab[i] == p]
        for c in range(5):
            assert M[p, c] == pytest.approx(math.fsum(X[i, c] for i in rows) / len(rows), abs=1e-15)
    assert np.all(M[6] == 0)


def test_patch_scores_brute_force():
    A, B = rnd(3, 4, 6), rnd(4, 5, 6)
    C = patch_scores(A, B)
    for p in range(4):
        for q in range(5):
            assert C[p, q] == pytest.approx(math.fsum(A[p, c] * B[q, c] for c in range(6)), abs=1e-14)


def test_topk_matches_sorted_and_breaks_ties_low():
    C = rnd(5, 9, 13)
    C[2, 7] = C[2, 3] = C[2, 11] = C[2].max() + 1.0   # exact three-way tie at the top
    C[4, :] = 0.5                                       # whole row tied
    C[6, 5] = C[6, 0] = np.sort(C[6])[-4]               # tie straddling the cut region
    for s in (1, 4, 13):
        idx = topk(C, s)
        for p in range(9):
            expect = [q for _, q in sorted((-C[p, q], q) for q in range(13))][:s]
            assert list(idx[p]) == expect
    assert list(topk(C, 3)[2]) == [3, 7, 11]
    assert list(topk(C, 5)[4]) == [0, 1, 2, 3, 4]
    assert sorted(topk(C, 13)[0]) == list(range(13))
    with pytest.raises(ValueError):
        topk(C, 0)
    with pytest.raises(ValueError):
        topk(C, 14)


def test_cut_gaps():
    C = np.array([[3.0, 1.0, 2.0, 2.0], [0.0, 5.0, 4.0, 1.0]])
    np.testing.assert_array_equal(cut_gaps(C, 2), [0.0, 3.0])
    np.testing.assert_array_equal(cut_gaps(C, 4), [np.inf, np.inf])


def _dense_problem(seed, nN=30, nM=36, d=6, k=4, PN=5, PM=6):
    Q, K, V, dO = (rnd(seed, nN, d, scale=1.5), rnd(seed + 1, nM, d, scale=1.5),
                   rnd(seed + 2, nM, k), rnd(seed + 3, nN, k))
    return Q, K, V, dO, labels(seed + 4, nN, PN), labels(seed + 6, nM, PM)


def test_full_selection_equals_dense():
    Q, K, V, dO, lN, lM = _dense_problem(10)
    sc = 1 / math.sqrt(6)
    C = patch_scores(patch_means(Q, lN, 5), patch_means(K, lM, 6))
    idx = topk(C, 6)
    O, lse = geo_fwd(Q, K, V, lN, lM, idx, sc)
    Od, lsed = dense_fwd(Q, K, V, sc)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=0, atol=1e-12)
    for g, gd in zip(geo_bwd(Q, K, V, dO, lN, lM, idx, sc), dense_bwd(Q, K, V, dO, sc)):
        np.testing.assert_allclose(g, gd, rtol=0, atol=1e-12)
    assert executed_pairs(lN, lM, idx) == 30 * 36


def test_one_patch_per_shape_equals_dense():
    Q, K, V, dO, _, _ = _dense_problem(20)
    z30, z36 = np.zeros(30, np.int32), np.zeros(36, np.int32)
    idx = topk(patch_scores(patch_means(Q, z30, 1), patch_means(K, z36, 1)), 1)
    np.testing.assert_allclose(geo_fwd(Q, K, V, z30, z36, idx, 0.4)[0], dense_fwd(Q, K, V, 0.4)[0],
                               rtol=0, atol=1e-13)


def _mask(lN, lM, idx):
    return np.array([[lM[j] in set(idx[lN[i]]) for j in range(len(lM))] for i in range(len(lN))])


@pytest.mark.parametrize("s", [1, 2, 4])
def test_against_torch_masked_sdpa_fp64(s):
    Q, K, V, dO, lN, lM = _dense_problem(30 + s)
    sc = 1 / math.sqrt(6)
    idx = topk(patch_scores(patch_means(Q, lN, 5), patch_means(K, lM, 6)), s)
    mask = torch.tensor(_mask(lN, lM, idx))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    to = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                          attn_mask=mask[None], scale=sc)[0]
    to.backward(torch.tensor(dO))
    O, lse = geo_fwd(Q, K, V, lN, lM, idx, sc)
    np.testing.assert_allclose(O, to.detach().numpy(), rtol=0, atol=1e-13)
    dQ, dK, dV = geo_bwd(Q, K, V, dO, lN, lM, idx, sc)
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-12)
    # lse against a direct log-sum-exp over each row's support
    S = (Q @ K.T) * sc
    for i in range(len(Q)):
        row = S[i][mask[i].numpy()]
        assert lse[i] == pytest.approx(np.log(np.sum(np.exp(row))), abs=1e-12)


def test_geo_backward_finite_differences_fixed_selection():
    Q, K, V, dO, lN, lM = _dense_problem(40, nN=8, nM=9, d=3, k=2, PN=3, PM=3)
    idx = topk(patch_scores(patch_means(Q, lN, 3), patch_means(K, lM, 3)), 2)
    sc = 0.9
    G = geo_bwd(Q, K, V, dO, lN, lM, idx, sc)
    h = 1e-6

    def loss(Q_, K_, V_):
        return float(np.sum(dO * geo_fwd(Q_, K_, V_, lN, lM, idx, sc)[0]))

    for which, X in enumerate((Q, K, V)):
        num = np.zeros_like(X)
        for ij in np.ndindex(X.shape):
            args_p = [Q.copy(), K.copy(), V.copy()]
            args_m = [Q.copy(), K.copy(), V.copy()]
            args_p[which][ij] += h
            args_m[which][ij] -= h
            num[ij] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        rel = np.linalg.norm(num - G[which]) / max(np.linalg.norm(G[which]), 1e-300)
        assert rel < 1e-7, (which, rel)


def test_unselected_source_rows_get_zero_gradient_and_empty_support():
    Q, K, V, dO, lN, lM = _dense_problem(50)
    idx = np.array([[0], [0], [1], [1], [0]], dtype=np.int32)  # patches 2..5 never selected
    dQ, dK, dV = geo_bwd(Q, K, V, dO, lN, lM, idx, 0.5)
    off = ~np.isin(lM, [0, 1])
    assert np.all(dK[off] == 0) and np.all(dV[off] == 0)
    assert np.abs(dK[~off]).sum() > 0
    # an empty selected patch gives an empty support
    lM2 = lM.copy()
    lM2[lM2 == 1] = 2
    O, lse = geo_fwd(Q, K, V, lN, lM2, idx, 0.5)
    rows = np.isin(lN, [2, 3])
    assert np.all(O[rows] == 0) and np.all(np.isneginf(lse[rows]))
    assert np.all(np.isfinite(lse[~rows]))


def test_singleton_patches_against_torch_masked_sdpa():
    Q, K, V, dO, lN, lM = _dense_problem(60)
    lN = lN.copy()
    lN[lN == 4] = 3
    lN[7] = 4                     # target patch 4 holds exactly one vertex
    lM = lM.copy()
    lM[lM == 5] = 0
    lM[11] = 5                    # source patch 5 holds exactly one vertex
    sc = 0.45
    idx = topk(patch_scores(patch_means(Q, lN, 5), patch_means(K, lM, 6)), 3)
    idx[4] = [5, 1, 2]            # make sure the singleton source patch is used
    mask = torch.tensor(_mask(lN, lM, idx))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    to = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                          attn_mask=mask[None], scale=sc)[0]
    to.backward(torch.tensor(dO))
    np.testing.assert_allclose(geo_fwd(Q, K, V, lN, lM, idx, sc)[0], to.detach().numpy(), atol=1e-13)
    for g, t in zip(geo_bwd(Q, K, V, dO, lN, lM, idx, sc), (tq, tk, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=0, atol=1e-12)
