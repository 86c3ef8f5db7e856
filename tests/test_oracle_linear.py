"""Pins of the fp64 linear-attention (ELU feature map) oracle.

The linearized coupling replaces the softmax by the feature map
phi(x) = elu(x) + 1 (ai4snews digest, "Interpretation"; project page,
"Runtime and memory", Table 1 row "Linear attention (ELU)").  Pins: a
pure-Python brute force of the coupling matrix (no factorisation), torch's
elu and autograd in fp64 on the unfactorised formula, closed forms
(identical keys, constant basis), positivity and row sums of the coupling
matrix, and central finite differences.
"""

import math

import numpy as np
import pytest
import torch

from oracle import elu1, elu1_grad, linear_bwd, linear_fwd, linear_weights


def rnd(seed, *shape, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def brute_fwd(Q, K, V):
    """Pure Python: W_ij = phi(q_i).phi(k_j) / sum_j, O = W V."""
    def phi(x):
        return x + 1.0 if x > 0 else math.exp(x)
    nN, nM, k = len(Q), len(K), len(V[0])
    O = [[0.0] * k for _ in range(nN)]
    for i in range(nN):
        a = [math.fsum(phi(qi) * phi(kj) for qi, kj in zip(Q[i], K[j])) for j in range(nM)]
        tot = math.fsum(a)
        for c in range(k):
            O[i][c] = math.fsum(a[j] * V[j][c] for j in range(nM)) / tot
    return np.array(O)


@pytest.mark.parametrize("nN,nM,d,k", [(1, 1, 1, 1), (4, 6, 3, 2), (7, 3, 5, 4)])
def test_brute_force_agrees(nN, nM, d, k):
    Q, K, V = rnd(1, nN, d, scale=1.5), rnd(2, nM, d, scale=1.5), rnd(3, nM, k)
    O, den = linear_fwd(Q, K, V)
    np.testing.assert_allclose(O, brute_fwd(Q.tolist(), K.tolist(), V.tolist()), rtol=0, atol=1e-13)
    np.testing.assert_allclose(den, (elu1(Q) @ elu1(K).T).sum(axis=1), rtol=1e-14)


def test_feature_map_matches_torch_elu():
    x = np.array([-30.0, -2.5, -1e-3, 0.0, 1e-3, 0.7, 12.0])
    t = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.elu(t) + 1.0
    y.sum().backward()
    np.testing.assert_allclose(elu1(x), y.detach().numpy(), rtol=0, atol=1e-15)
    np.testing.assert_allclose(elu1_grad(x), t.grad.numpy(), rtol=0, atol=1e-15)
    assert elu1(0.0) == 1.0 and elu1_grad(0.0) == 1.0


def test_against_torch_autograd_unfactorised():
    Q, K, V, dO = rnd(5, 6, 4, scale=1.2), rnd(6, 9, 4, scale=1.2), rnd(7, 9, 3), rnd(8, 6, 3)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    A = (torch.nn.functional.elu(tq) + 1) @ (torch.nn.functional.elu(tk) + 1).T
    O = (A / A.sum(dim=1, keepdim=True)) @ tv
    O.backward(torch.tensor(dO))
    Of, _ = linear_fwd(Q, K, V)
    np.testing.assert_allclose(Of, O.detach().numpy(), rtol=0, atol=1e-13)
    dQ, dK, dV = linear_bwd(Q, K, V, dO)
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_coupling_matrix_positive_rows_sum_to_one():
    W = linear_weights(rnd(9, 5, 3, scale=3.0), rnd(10, 8, 3, scale=3.0))
    assert np.all(W > 0)
    np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_basis():
    Q = rnd(11, 4, 5)
    K = np.tile(rnd(12, 1, 5), (7, 1))
    V = rnd(13, 7, 3)
    O, _ = linear_fwd(Q, K, V)
    np.testing.assert_allclose(O, np.tile(V.mean(axis=0), (4, 1)), rtol=0, atol=1e-14)


def test_constant_basis_is_reproduced():
    O, _ = linear_fwd(rnd(14, 3, 4), rnd(15, 6, 4), np.full((6, 2), 2.5))
    np.testing.assert_allclose(O, 2.5, rtol=0, atol=1e-14)
    dQ, dK, dV = linear_bwd(rnd(14, 3, 4), rnd(15, 6, 4), np.full((6, 2), 2.5), rnd(16, 3, 2))
    # O does not depend on Q or K when every basis row is the same
    np.testing.assert_allclose(dQ, 0.0, atol=1e-13)
    np.testing.assert_allclose(dK, 0.0, atol=1e-13)


def test_backward_central_finite_differences():
    Q, K, V, dO = rnd(17, 3, 4), rnd(18, 5, 4), rnd(19, 5, 2), rnd(20, 3, 2)
    dQ, dK, dV = linear_bwd(Q, K, V, dO)
    h = 1e-6

    def loss(Q_, K_, V_):
        return float(np.sum(linear_fwd(Q_, K_, V_)[0] * dO))

    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[which], args_m[which] = Xp, Xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-8)
