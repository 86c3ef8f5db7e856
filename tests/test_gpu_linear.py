"""GPU parity of the linear-attention (ELU feature map) coupling against the
fp64 oracle, through the C ABI.

Same bars as the exact coupling: O max-abs <= 2e-2 and rel-Frobenius <= 5e-3;
dQ, dK, dV rel-Frobenius <= 1e-2 (bf16 inputs; phi(K)^T V and its backward
counterpart are rounded to bf16 once before the second product); the
normaliser den to rel 5e-3.  Every output is checked in full, also at 60k:
the oracle is O(n d k) here.
"""

import numpy as np
import pytest
import torch

import gen
import spatial_spectral_coupling_amd as ssc
from oracle import elu1, elu1_grad, linear_bwd, linear_fwd
from tests._util import check_fwd, check_grads, f64, rel_f, say, to_dev

pytestmark = pytest.mark.gpu


def run_linear(c):
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    O, den = ssc.coupling_linear_fwd(Q, K, V)
    dQ, dK, dV = ssc.coupling_linear_bwd(Q, K, V, O, dO, den)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (O, den, dQ, dK, dV)]


def check_all(c, what):
    O, den, dQ, dK, dV = run_linear(c)
    Q, K, V, dO = (f64(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    Or, denr = linear_fwd(Q, K, V)
    check_fwd(O, Or, what=what)
    rd = float(np.max(np.abs(den - denr) / denr))
    say(f"{what} den max-rel {rd:.3e}")
    assert rd <= 5e-3, (what, rd)
    ref = linear_bwd(Q, K, V, dO)
    if K.shape[0] == 1:
        # one source row: O = V[0] whatever Q and K are, so dQ and dK are
        # exactly 0, each the difference of two equal terms; they are checked
        # against the size of those terms (relative 1e-2), dV as usual.
        fK, fQ = elu1(K), elu1(Q)
        g = dO / denr[:, None]
        tQ = elu1_grad(Q) * (np.abs(g) @ np.abs(fK.T @ V).T)
        tK = elu1_grad(K) * (np.abs(V) @ np.abs(fQ.T @ g).T)
        for name, x, t in (("dQ", dQ, tQ), ("dK", dK, tK)):
            err = float(np.max(np.abs(x)) / max(float(np.max(t)), 1e-300))
            say(f"{what} {name} (exactly 0) max / term {err:.3e}")
            assert err <= 1e-2, (what, name, err)
        rf = rel_f(dV, ref[2])
        say(f"{what} dV rel-F {rf:.3e}")
        assert rf <= 1e-2, (what, rf)
    else:
        check_grads((dQ, dK, dV), ref, what=what)


SHAPES = [
    (300, 517, 128, 200),
    (1, 1, 128, 200),
    (129, 1000, 128, 200),
    (77, 33, 64, 30),
    (513, 1100, 128, 7),
    (200, 150, 128, 255),
    (64, 96, 64, 64),
    (260, 700, 64, 128),
]


@pytest.mark.parametrize("nN,nM,d,k", SHAPES)
def test_linear_parity_small(nN, nM, d, k):
    say("linear small", nN, nM, d, k)
    c = gen.make_small(nN, nM, d, k, "bf16", seed=3 * nN + nM)
    check_all(c, f"linear {nN}x{nM} d{d} k{k}")


def test_linear_parity_60k():
    c = gen.cached_config(2)
    say("linear 60k", c["n"], c["d"], c["k"])
    check_all(c, "linear 60k")


def test_linear_autograd_and_determinism():
    c = gen.make_small(200, 300, 128, 200, "bf16", seed=11)
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    Qr, Kr, Vr = (t.clone().requires_grad_(True) for t in (Q, K, V))
    O = ssc.linear_coupling(Qr, Kr, Vr)
    O.backward(dO.float())
    O2, den2 = ssc.coupling_linear_fwd(Q, K, V)
    g2 = ssc.coupling_linear_bwd(Q, K, V, O2, dO, den2)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    for a, b in zip((Qr.grad, Kr.grad, Vr.grad), g2):
        assert torch.equal(a.float(), b.to(a.dtype).float())
    O3, _ = ssc.coupling_linear_fwd(Q, K, V)
    assert torch.equal(O2, O3)


def test_linear_rejects_unsupported():
    Q = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    V = torch.zeros(4, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ssc.CouplingError):
        ssc.coupling_linear_fwd(Q, Q, V)           # k = 256 leaves no column for the normaliser
    Qf = torch.zeros(4, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(ssc.CouplingError):
        ssc.coupling_linear_fwd(Qf, Qf, Qf[:, :8].contiguous())


def test_linear_without_target_rows():
    """n_N = 0: the backward writes dK = dV = 0 (the query-side Gram sum is
    empty; nothing reads the empty Q, O, dO, den)."""
    say("linear without target rows")
    c = gen.make_small(1, 300, 128, 200, "bf16", seed=7)
    K, V = to_dev(c["K"], "bf16"), to_dev(c["V"], "bf16")
    Q = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    dO = torch.empty(0, 200, dtype=torch.bfloat16, device="cuda")
    O, den = ssc.coupling_linear_fwd(Q, K, V)
    assert O.shape == (0, 200) and den.shape == (0,)
    dQ, dK, dV = ssc.coupling_linear_bwd(Q, K, V, O, dO, den)
    torch.cuda.synchronize()
    assert dQ.shape == (0, 128)
    assert torch.count_nonzero(dK).item() == 0 and torch.count_nonzero(dV).item() == 0
