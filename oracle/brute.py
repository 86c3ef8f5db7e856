"""Pure-Python brute force of the dense coupling for tiny inputs.

Test infrastructure only.  Lists of floats, `math.exp` / `math.log` and
`math.fsum` (exactly rounded sums); no NumPy in the arithmetic.  It is the
definition of scaled dot-product attention (spatial-spectral-attention.github.io,
"How it works") evaluated entry by entry, with the backward obtained from the
softmax Jacobian dPi_ij/dS_ik = Pi_ij (delta_jk - Pi_ik) summed explicitly,
i.e. a different route from the D-trick used by `oracle.dense`.
"""

from __future__ import annotations

import math

__all__ = ["brute_fwd", "brute_bwd"]


def _rows(a):
    return [[float(v) for v in row] for row in a]


def brute_fwd(Q, K, V, scale):
    Q, K, V = _rows(Q), _rows(K), _rows(V)
    k = len(V[0]) if V else 0
    O, lse, Pi = [], [], []
    for q in Q:
        s = [scale * math.fsum(a * b for a, b in zip(q, kk)) for kk in K]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = math.fsum(e)
        p = [v / z for v in e]
        Pi.append(p)
        O.append([math.fsum(p[j] * V[j][c] for j in range(len(K))) for c in range(k)])
        lse.append(m + math.log(z))
    return O, lse, Pi


def brute_bwd(Q, K, V, dO, scale):
    """dQ, dK, dV via the explicit softmax Jacobian (O(n_M^2) per row)."""
    Qr, Kr, Vr, dOr = _rows(Q), _rows(K), _rows(V), _rows(dO)
    _, _, Pi = brute_fwd(Qr, Kr, Vr, scale)
    n_N, n_M = len(Qr), len(Kr)
    d, k = len(Qr[0]), len(Vr[0])
    dQ = [[0.0] * d for _ in range(n_N)]
    dK = [[0.0] * d for _ in range(n_M)]
    dV = [[0.0] * k for _ in range(n_M)]
    for i in range(n_N):
        p = Pi[i]
        # g_j = dL/dPi_ij = <dO_i, V_j>
        g = [math.fsum(dOr[i][c] * Vr[j][c] for c in range(k)) for j in range(n_M)]
        # dL/dS_ik = sum_j g_j Pi_ij (delta_jk - Pi_ik)
        ds = [math.fsum([g[kk] * p[kk]] + [-g[j] * p[j] * p[kk] for j in range(n_M)])
              for kk in range(n_M)]
        for j in range(n_M):
            for c in range(d):
                dQ[i][c] += scale * ds[j] * Kr[j][c]
                dK[j][c] += scale * ds[j] * Qr[i][c]
            for c in range(k):
                dV[j][c] += p[j] * dOr[i][c]
    return dQ, dK, dV
