"""Pins of the fp64 functional-map solve (oracle.fmap) against facts fixed by
the mathematics: exact recovery of a planted map, the orthonormal-basis closed
form, an SVD least-squares routine, the reparametrisation rule, the normal
equations, torch autograd (fp64, CPU) and finite differences for the backward."""

import numpy as np
import pytest
import torch

from oracle import fmap_solve, fmap_solve_bwd


def _basis(n, k, seed, cond=1.0):
    rng = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    scales = np.geomspace(1.0, cond, k)
    W = np.linalg.qr(rng.standard_normal((k, k)))[0]
    return np.sqrt(n) * Q @ np.diag(scales) @ W.T


def test_recovers_a_planted_map():
    Phi = _basis(300, 20, 1, cond=10.0)
    C = np.random.default_rng(2).standard_normal((20, 20))
    np.testing.assert_allclose(fmap_solve(Phi, Phi @ C), C, atol=1e-10, rtol=0)


def test_orthonormal_basis_closed_form():
    rng = np.random.default_rng(3)
    Q, _ = np.linalg.qr(rng.standard_normal((250, 16)))
    O = rng.standard_normal((250, 16))
    np.testing.assert_allclose(fmap_solve(Q, O), Q.T @ O, atol=1e-12, rtol=0)


def test_matches_svd_least_squares():
    Phi = _basis(200, 30, 4, cond=30.0)
    O = np.random.default_rng(5).standard_normal((200, 30))
    ref = np.linalg.lstsq(Phi, O, rcond=None)[0]
    np.testing.assert_allclose(fmap_solve(Phi, O), ref, atol=1e-10, rtol=1e-9)


def test_reparametrisation_and_normal_equations():
    rng = np.random.default_rng(6)
    Phi = _basis(180, 12, 7, cond=5.0)
    O = rng.standard_normal((180, 12))
    M = rng.standard_normal((12, 12)) + 4 * np.eye(12)
    C = fmap_solve(Phi, O)
    # basis Phi M: the map in the new coordinates is M^-1 C
    np.testing.assert_allclose(fmap_solve(Phi @ M, O), np.linalg.solve(M, C), atol=1e-9, rtol=0)
    # the residual is orthogonal to the basis
    np.testing.assert_allclose(Phi.T @ (Phi @ C - O), 0.0, atol=1e-8)


def test_backward_identities_and_autograd():
    rng = np.random.default_rng(8)
    Phi = _basis(150, 10, 9, cond=8.0)
    O = rng.standard_normal((150, 10))
    dC = rng.standard_normal((10, 10))
    dO = fmap_solve_bwd(Phi, dC)
    # Phi^T dO = dC and dO lies in the span of the basis
    np.testing.assert_allclose(Phi.T @ dO, dC, atol=1e-9, rtol=0)
    Pt = torch.tensor(Phi, dtype=torch.float64)
    Ot = torch.tensor(O, dtype=torch.float64, requires_grad=True)
    Ct = torch.linalg.lstsq(Pt, Ot).solution
    (Ct * torch.tensor(dC, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(dO, Ot.grad.numpy(), atol=1e-9, rtol=1e-9)


@pytest.mark.parametrize("entry", [(0, 0), (37, 4), (149, 9)])
def test_backward_finite_differences(entry):
    rng = np.random.default_rng(10)
    Phi = _basis(150, 10, 11, cond=3.0)
    O = rng.standard_normal((150, 10))
    dC = rng.standard_normal((10, 10))
    g = fmap_solve_bwd(Phi, dC)[entry]
    h = 1e-6
    Op, Om = O.copy(), O.copy()
    Op[entry] += h
    Om[entry] -= h
    fd = (np.sum(dC * fmap_solve(Phi, Op)) - np.sum(dC * fmap_solve(Phi, Om))) / (2 * h)
    assert abs(fd - g) < 1e-6 * max(1.0, abs(g))
