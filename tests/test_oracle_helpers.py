"""Pins of the oracle's helper routines that the GPU tests and the benchmark
lean on: `dense_rows` (the coupling on listed target rows only), `linear_weights`
(the ELU coupling matrix itself) and `executed_pairs` (the (target, source)
pairs a geo selection visits).

Each is checked against a route that shares none of its code: the full dense
coupling indexed afterwards and a pure-Python brute force (project page,
"How it works": each row of the coupling depends on its own target row only);
the factorised linear coupling and a per-entry Python loop (ai4snews digest,
"Interpretation"); and a plain count over vertex labels at s < P_M, where the
count depends on which source patches were selected (project page,
"Geo-FlashAttention": each target patch attends to its selected source
patches only).  The inputs are chosen so that a swapped operand, a dropped
normaliser or an ignored selection changes the result.
"""

import math

import numpy as np

from oracle import dense_fwd, dense_rows, executed_pairs, linear_fwd, linear_weights
from oracle.brute import brute_fwd


def rnd(seed, *shape, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def test_dense_rows_equals_full_coupling_on_those_rows():
    # n_N != n_M != k and unsorted rows with a repeat: a transposed operand,
    # a sorted or de-duplicated row list, or rows taken from K would differ
    Q, K, V = rnd(1, 9, 4, scale=1.5), rnd(2, 13, 4, scale=1.5), rnd(3, 13, 3)
    rows = np.array([7, 0, 7, 4, 8])
    O, lse = dense_rows(Q, K, V, 0.7, rows)
    assert O.shape == (5, 3) and lse.shape == (5,)
    Of, lsef = dense_fwd(Q, K, V, 0.7)
    np.testing.assert_array_equal(O, Of[rows])
    np.testing.assert_array_equal(lse, lsef[rows])
    Ob = brute_fwd(Q[rows].tolist(), K.tolist(), V.tolist(), 0.7)[0]
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)


def test_dense_rows_scale_enters():
    Q, K, V = rnd(4, 3, 5), rnd(5, 6, 5), rnd(6, 6, 2)
    a = dense_rows(Q, K, V, 0.5, [0, 2])[0]
    b = dense_rows(Q, K, V, 1.0, [0, 2])[0]
    assert np.max(np.abs(a - b)) > 1e-3


def _python_weights(Q, K):
    def phi(x):
        return x + 1.0 if x > 0 else math.exp(x)
    W = []
    for q in Q:
        a = [math.fsum(phi(x) * phi(y) for x, y in zip(q, k)) for k in K]
        tot = math.fsum(a)
        W.append([v / tot for v in a])
    return np.array(W)


def test_linear_weights_shape_values_and_product():
    # n_N = 4, n_M = 7: swapping Q and K gives a 7 x 4 matrix, a missing row
    # normalisation breaks the row sums, and W V must be the factorised O
    Q, K, V = rnd(7, 4, 3, scale=1.3), rnd(8, 7, 3, scale=1.3), rnd(9, 7, 5)
    W = linear_weights(Q, K)
    assert W.shape == (4, 7)
    np.testing.assert_allclose(W, _python_weights(Q.tolist(), K.tolist()), rtol=0, atol=1e-14)
    np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    O, _ = linear_fwd(Q, K, V)
    np.testing.assert_allclose(W @ V, O, rtol=0, atol=1e-13)


def test_linear_weights_not_symmetric_in_operands():
    Q, K = rnd(10, 5, 3, scale=2.0), rnd(11, 5, 3, scale=2.0)
    assert np.max(np.abs(linear_weights(Q, K) - linear_weights(K, Q).T)) > 1e-3


def _count_pairs(labN, labM, idx):
    total = 0
    for p in range(idx.shape[0]):
        rows = sum(1 for l in labN if l == p)
        sel = set(int(q) for q in idx[p])
        keys = sum(1 for l in labM if l in sel)
        total += rows * keys
    return total


def test_executed_pairs_plain_loop_with_partial_selection():
    rng = np.random.default_rng(12)
    P_N, P_M, s = 6, 9, 3
    labN = rng.integers(0, P_N, 200)
    labM = rng.integers(0, P_M, 170)
    labN[:3] = 5  # keep every target patch non-empty
    idx = np.stack([rng.permutation(P_M)[:s] for _ in range(P_N)]).astype(np.int32)
    got = executed_pairs(labN, labM, idx)
    assert got == _count_pairs(labN, labM, idx)
    # the selection matters: another selection of the same size counts differently,
    # and the full selection counts n_N x n_M
    idx2 = ((idx + 1) % P_M).astype(np.int32)
    assert executed_pairs(labN, labM, idx2) == _count_pairs(labN, labM, idx2)
    assert executed_pairs(labN, labM, idx2) != got
    full = np.tile(np.arange(P_M, dtype=np.int32), (P_N, 1))
    assert executed_pairs(labN, labM, full) == 200 * 170


def test_executed_pairs_empty_patches():
    labN = np.array([0, 0, 2, 2, 2])          # target patch 1 is empty
    labM = np.array([1, 1, 1, 0, 3, 3])       # source patch 2 is empty
    idx = np.array([[1, 2], [0, 3], [3, 2]], np.int32)
    # patch 0: 2 rows x (3 + 0) keys; patch 1: 0 rows; patch 2: 3 rows x (2 + 0)
    assert executed_pairs(labN, labM, idx) == 2 * 3 + 3 * 2
