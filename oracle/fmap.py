"""Functional-map solve after the coupling, in fp64 -- test infrastructure only.

The coupled functional-map pipelines use only the product Pi_NM Phi_M
(project page, "How it works"): a functional-map solver turns it into the
k x k map between the two spectral bases.  The pages do not print the
solver; the reading taken here is the plain least-squares map

    C = argmin_C || Phi_N C - O ||_F = (Phi_N^T Phi_N)^{-1} Phi_N^T O,

with O = Pi_NM Phi_M (n_N x k) and Phi_N the target basis (n_N x k, full
column rank).  Its backward for an upstream gradient dC (k x k), with the
basis held fixed (no gradient for Phi_N):

    dO = Phi_N (Phi_N^T Phi_N)^{-1} dC.

Both are written out with the normal equations and a library solve.
"""

from __future__ import annotations

import numpy as np

__all__ = ["fmap_solve", "fmap_solve_bwd"]


def fmap_solve(PhiN: np.ndarray, O: np.ndarray) -> np.ndarray:
    """C (k x k) = (Phi_N^T Phi_N)^{-1} Phi_N^T O, fp64."""
    PhiN = np.asarray(PhiN, np.float64)
    O = np.asarray(O, np.float64)
    G = PhiN.T @ PhiN
    R = PhiN.T @ O
    return np.linalg.solve(G, R)


def fmap_solve_bwd(PhiN: np.ndarray, dC: np.ndarray) -> np.ndarray:
    """dO (n_N x k) = Phi_N (Phi_N^T Phi_N)^{-1} dC, fp64."""
    PhiN = np.asarray(PhiN, np.float64)
    dC = np.asarray(dC, np.float64)
    G = PhiN.T @ PhiN
    return PhiN @ np.linalg.solve(G, dC)
