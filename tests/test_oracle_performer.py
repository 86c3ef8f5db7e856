"""Pins of the fp64 Performer (FAVOR+) coupling (oracle.performer): the
estimator's expectation exp(c q.k) (Monte Carlo with many directions), its
convergence to the exact softmax coupling, the one-direction closed form,
torch autograd of an independent torch forward and central finite
differences for the backward, and the zero row sum the GPU side relies on."""

import numpy as np
import torch

import gen
from oracle import dense_fwd, favor_features, performer_bwd, performer_fwd


def test_unbiased_softmax_kernel():
    rng = np.random.default_rng(0)
    d, m, c = 4, 400000, 0.5
    q, k = 0.6 * rng.standard_normal(d), 0.6 * rng.standard_normal(d)
    W = rng.standard_normal((m, d))
    est = (favor_features(q[None], W, c) @ favor_features(k[None], W, c).T).item()
    want = np.exp(c * q @ k)
    # the per-feature variance is below exp(4c(|q|^2+|k|^2)/2) * want^2 / m
    assert abs(est / want - 1.0) < 0.01, (est, want)


def test_converges_to_the_softmax_coupling():
    rng = np.random.default_rng(1)
    n, d, k = 12, 4, 3
    Q, K, V = 0.5 * rng.standard_normal((n, d)), 0.5 * rng.standard_normal((n, d)), rng.standard_normal((n, k))
    c = 1.0 / np.sqrt(d)
    W = rng.standard_normal((300000, d))
    O, lnden = performer_fwd(Q, K, V, W, c)
    Od, _ = dense_fwd(Q, K, V, c)
    assert np.max(np.abs(O - Od)) < 1e-2
    # ln den estimates the log partition function ln sum_j exp(c q.k_j)
    lse = np.log(np.exp(c * Q @ K.T).sum(axis=1))
    assert np.max(np.abs(lnden - lse)) < 1e-2


def test_one_direction_closed_form():
    rng = np.random.default_rng(2)
    Q, K, V = rng.standard_normal((5, 3)), rng.standard_normal((7, 3)), rng.standard_normal((7, 2))
    w = rng.standard_normal((1, 3))
    c = 0.3
    O, lnden = performer_fwd(Q, K, V, w, c)
    a = np.exp(np.sqrt(c) * K @ w[0] - 0.5 * c * np.sum(K * K, axis=1))
    want = (a @ V) / a.sum()
    np.testing.assert_allclose(O, np.tile(want, (5, 1)), rtol=1e-13, atol=0)
    b = np.exp(np.sqrt(c) * Q @ w[0] - 0.5 * c * np.sum(Q * Q, axis=1))
    np.testing.assert_allclose(lnden, np.log(b * a.sum()), rtol=1e-13, atol=0)


def torch_forward(Q, K, V, W, c):
    def feats(X):
        return torch.exp(c ** 0.5 * X @ W.T - 0.5 * c * (X * X).sum(1, keepdim=True)) / W.shape[0] ** 0.5
    fQ, fK = feats(Q), feats(K)
    num = fQ @ (fK.T @ V)
    den = fQ @ fK.sum(0)
    return num / den[:, None]


def test_backward_matches_autograd_and_finite_differences():
    rng = np.random.default_rng(3)
    n_N, n_M, d, k, m = 6, 9, 5, 4, 11
    Q, K = 0.7 * rng.standard_normal((n_N, d)), 0.7 * rng.standard_normal((n_M, d))
    V, W, dO = rng.standard_normal((n_M, k)), rng.standard_normal((m, d)), rng.standard_normal((n_N, k))
    c = 1 / np.sqrt(d)
    dQ, dK, dV = performer_bwd(Q, K, V, W, dO, c)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V)]
    O = torch_forward(*t, torch.tensor(W), c)
    (O * torch.tensor(dO)).sum().backward()
    for g, tt in zip((dQ, dK, dV), t):
        np.testing.assert_allclose(g, tt.grad.numpy(), rtol=1e-10, atol=1e-12)
    # central differences on a few entries of each input
    h = 1e-6
    f = lambda Q_, K_, V_: float(np.sum(performer_fwd(Q_, K_, V_, W, c)[0] * dO))
    for which, G in ((0, dQ), (1, dK), (2, dV)):
        args = [Q.copy(), K.copy(), V.copy()]
        for idx in [(0, 0), (2, 1), (-1, -1)]:
            p, mm = [a.copy() for a in args], [a.copy() for a in args]
            p[which][idx] += h
            mm[which][idx] -= h
            fd = (f(*p) - f(*mm)) / (2 * h)
            assert abs(fd - G[idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, G[idx])


def test_query_row_sum_vanishes():
    # sum_i dphi(q)_i phi(q)_i = dO . O - dO . O = 0: the query gradient has no
    # c q term
    rng = np.random.default_rng(4)
    Q, K, V = rng.standard_normal((8, 4)), rng.standard_normal((10, 4)), rng.standard_normal((10, 3))
    W, dO = rng.standard_normal((6, 4)), rng.standard_normal((8, 3))
    c = 0.5
    fQ, fK = favor_features(Q, W, c), favor_features(K, W, c)
    KV, z = fK.T @ V, fK.sum(0)
    den = fQ @ z
    O = fQ @ KV / den[:, None]
    dfQ = (dO / den[:, None]) @ KV.T - (np.sum(dO * O, 1) / den)[:, None] * z[None]
    np.testing.assert_allclose(np.sum(dfQ * fQ, axis=1), 0.0, atol=1e-12)


def test_orthogonal_directions_generator():
    W = gen.bf16_bits_to_f32(gen.make_favor_directions(256, 128, seed=1)).astype(np.float64)
    assert W.shape == (256, 128)
    # rows within a block of d are orthogonal (up to bf16 rounding)
    B = W[:128]
    G = B @ B.T
    off = G - np.diag(np.diag(G))
    assert np.max(np.abs(off)) < 0.05 * np.max(np.diag(G))
