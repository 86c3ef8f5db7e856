"""Pins of the dense fp64 oracle against things other than itself.

The coupling is scaled dot-product attention with Q = F_N, K = F_M, V = Phi_M
(spatial-spectral-attention.github.io, "How it works").  Pins: the
pure-Python brute force (different backward route: the explicit softmax
Jacobian), closed forms (one-hot permutation, uniform logits, single key),
invariants (row sums, shift/permutation invariance, linearity, gradient
identities), library routines (scipy logsumexp / softmax, torch's CPU
scaled_dot_product_attention and autograd in fp64) and central finite
differences.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import dense_bwd, dense_fwd, rowdot, upcast
from oracle.brute import brute_bwd, brute_fwd


def rnd(seed, *shape, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("nN,nM,d,k", [(1, 1, 1, 1), (5, 7, 4, 3), (8, 3, 2, 5), (3, 9, 6, 2)])
def test_brute_force_agrees(nN, nM, d, k):
    Q, K, V, dO = rnd(1, nN, d, scale=1.5), rnd(2, nM, d, scale=1.5), rnd(3, nM, k), rnd(4, nN, k)
    sc = 1.0 / math.sqrt(d)
    O, lse, P = dense_fwd(Q, K, V, sc, return_P=True)
    Ob, lseb, Pb = brute_fwd(Q, K, V, sc)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-13)
    np.testing.assert_allclose(P, Pb, rtol=0, atol=1e-14)
    dQ, dK, dV = dense_bwd(Q, K, V, dO, sc)
    bQ, bK, bV = brute_bwd(Q, K, V, dO, sc)
    np.testing.assert_allclose(dQ, bQ, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, bK, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, bV, rtol=0, atol=1e-12)


def test_rows_of_map_sum_to_one():
    Q, K, V = rnd(5, 40, 16, scale=3), rnd(6, 70, 16, scale=3), rnd(7, 70, 4)
    _, _, P = dense_fwd(Q, K, V, 0.25, block=7, return_P=True)
    assert P.shape == (40, 70)
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_map_matches_scipy_softmax_and_logsumexp():
    Q, K, V = rnd(8, 33, 8, scale=2), rnd(9, 51, 8, scale=2), rnd(10, 51, 6)
    sc = 1 / math.sqrt(8)
    O, lse, P = dense_fwd(Q, K, V, sc, block=10, return_P=True)
    S = (Q @ K.T) * sc
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=1), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(S, axis=1), rtol=1e-14, atol=1e-13)


@pytest.mark.parametrize("alpha,n,d", [(1.0, 6, 8), (3.0, 12, 12), (16.0, 128, 128)])
def test_one_hot_permutation_closed_form(alpha, n, d):
    rng = np.random.default_rng(11)
    pi = rng.permutation(n)
    FN = np.zeros((n, d))
    FN[np.arange(n), pi] = alpha
    FM = np.zeros((n, d))
    FM[np.arange(n), np.arange(n)] = alpha
    Phi = rnd(12, n, 5)
    sc = 1 / math.sqrt(d)
    a = alpha * alpha * sc
    O, lse = dense_fwd(FN, FM, Phi, sc)
    expect = ((math.expm1(a)) * Phi[pi] + Phi.sum(axis=0)) / (math.exp(a) + n - 1)
    np.testing.assert_allclose(O, expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(math.exp(a) + n - 1), rtol=1e-14)
    if alpha == 16.0:
        # large logit gap: the coupling returns the permuted basis rows
        assert np.max(np.abs(O - Phi[pi])) < 1e-7


def test_uniform_logits_give_mean_of_basis():
    K, V = rnd(13, 25, 6), rnd(14, 25, 4)
    O, lse = dense_fwd(np.zeros((3, 6)), K, V, 0.7)
    np.testing.assert_allclose(O, np.tile(V.mean(axis=0), (3, 1)), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(25), rtol=1e-15)


def test_single_source_vertex():
    Q, K, V, dO = rnd(15, 9, 4), rnd(16, 1, 4), rnd(17, 1, 3), rnd(18, 9, 3)
    O, lse = dense_fwd(Q, K, V, 0.5)
    np.testing.assert_allclose(O, np.tile(V[0], (9, 1)), rtol=0, atol=0)
    np.testing.assert_allclose(lse, 0.5 * (Q @ K[0]), rtol=1e-15)
    dQ, dK, dV = dense_bwd(Q, K, V, dO, 0.5)
    assert np.max(np.abs(dQ)) < 1e-15 and np.max(np.abs(dK)) < 1e-14
    np.testing.assert_allclose(dV[0], dO.sum(axis=0), rtol=1e-14)


def test_shift_permutation_and_linearity_invariants():
    Q, K, V, V2 = rnd(19, 20, 8, scale=2), rnd(20, 30, 8, scale=2), rnd(21, 30, 5), rnd(22, 30, 5)
    sc = 0.3
    O, lse = dense_fwd(Q, K, V, sc)
    c = rnd(23, 8)
    O2, lse2 = dense_fwd(Q, K + c, V, sc)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + sc * (Q @ c), rtol=0, atol=1e-12)
    perm = np.random.default_rng(24).permutation(30)
    O3, _ = dense_fwd(Q, K[perm], V[perm], sc)
    np.testing.assert_allclose(O3, O, rtol=0, atol=1e-13)
    rp = np.random.default_rng(25).permutation(20)
    O4, _ = dense_fwd(Q[rp], K, V, sc)
    np.testing.assert_allclose(O4, O[rp], rtol=0, atol=1e-13)
    Oa, _ = dense_fwd(Q, K, 2.0 * V - 3.0 * V2, sc)
    Ob, _ = dense_fwd(Q, K, V2, sc)
    np.testing.assert_allclose(Oa, 2.0 * O - 3.0 * Ob, rtol=0, atol=1e-12)


def test_against_torch_sdpa_and_autograd_fp64():
    Q, K, V, dO = rnd(26, 37, 16, scale=2), rnd(27, 45, 16, scale=2), rnd(28, 45, 7), rnd(29, 37, 7)
    sc = 1 / math.sqrt(16)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V))
    to = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], scale=sc)[0]
    to.backward(torch.tensor(dO))
    O, _ = dense_fwd(Q, K, V, sc, block=8)
    dQ, dK, dV = dense_bwd(Q, K, V, dO, sc, block=8)
    np.testing.assert_allclose(O, to.detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_central_finite_differences():
    Q, K, V, dO = rnd(30, 4, 3), rnd(31, 5, 3), rnd(32, 5, 2), rnd(33, 4, 2)
    sc = 0.8
    dQ, dK, dV = dense_bwd(Q, K, V, dO, sc)
    h = 1e-6

    def loss(Q_, K_, V_):
        return float(np.sum(dO * dense_fwd(Q_, K_, V_, sc)[0]))

    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = {"Q": (Xp, K, V), "K": (Q, Xp, V), "V": (Q, K, Xp)}[name]
            args_m = {"Q": (Xm, K, V), "K": (Q, Xm, V), "V": (Q, K, Xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        rel = np.linalg.norm(num - G) / np.linalg.norm(G)
        assert rel < 1e-7, (name, rel)


def test_gradient_identities():
    Q, K, V, dO = rnd(34, 50, 8, scale=2), rnd(35, 60, 8, scale=2), rnd(36, 60, 6), rnd(37, 50, 6)
    dQ, dK, dV = dense_bwd(Q, K, V, dO, 0.35, block=16)
    # sum_j dS_ij = 0 for each row  =>  sum_j dK_j = 0
    np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-12)
    # rows of the map sum to one  =>  sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dV.sum(axis=0), dO.sum(axis=0), atol=1e-12)
    # both traces equal scale * sum_ij dS_ij q_i.k_j
    assert abs(np.sum(Q * dQ) - np.sum(K * dK)) < 1e-11


def test_row_restricted_backward_equals_masked_upstream():
    Q, K, V, dO = rnd(38, 30, 8), rnd(39, 40, 8), rnd(40, 40, 5), rnd(41, 30, 5)
    rows = np.array([0, 3, 17, 29])
    dOm = np.zeros_like(dO)
    dOm[rows] = dO[rows]
    a = dense_bwd(Q, K, V, dOm, 0.4)
    b = dense_bwd(Q, K, V, dO, 0.4, rows=rows, block=3)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-14)


def test_empty_target_set_and_bad_source():
    O, lse = dense_fwd(np.zeros((0, 4)), rnd(42, 5, 4), rnd(43, 5, 3), 0.5)
    assert O.shape == (0, 3) and lse.shape == (0,)
    with pytest.raises(ValueError):
        dense_fwd(rnd(44, 2, 4), np.zeros((0, 4)), np.zeros((0, 3)), 0.5)


def test_upcast_bf16_bits_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    got = upcast(bits, "bf16")
    expect = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -0.0]
    assert list(got) == expect
    t = torch.tensor(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, t)


def test_rowdot():
    a, b = rnd(45, 6, 4), rnd(46, 6, 4)
    np.testing.assert_allclose(rowdot(a, b), [math.fsum(x * y for x, y in zip(r, s)) for r, s in zip(a, b)],
                               rtol=1e-15)
