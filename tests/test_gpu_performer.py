"""GPU parity of the Performer (FAVOR+) coupling against the fp64 oracle,
through the C ABI.

Same bars as the other couplings: O max-abs <= 2e-2 and rel-Frobenius <=
5e-3; dQ, dK, dV rel-Frobenius <= 1e-2; ln den max-abs <= 1e-2 (natural
log).  The arithmetic behind them: bf16 inputs and directions, the feature
exponents in fp32, the shifted features rounded to bf16 once (2^-9), the
d x k products rounded to bf16 once before the row products.  Both sides use
the same directions W (drawn by the generator); the comparison is with the
oracle's estimator, not with the softmax it approximates.  Every output is
checked in full, also at 60k rows (the oracle is O(n d (d + k)) here).
"""

import numpy as np
import pytest
import torch

import gen
import spatial_spectral_coupling_amd as ssc
from oracle import performer_bwd, performer_fwd
from tests._util import check_fwd, check_grads, f64, rel_f, say, to_dev

pytestmark = pytest.mark.gpu


def run(c, Wb, scale):
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    W = to_dev(Wb, "bf16")
    O, lnden = ssc.coupling_performer_fwd(Q, K, V, W, scale)
    dQ, dK, dV = ssc.coupling_performer_bwd(Q, K, V, W, O, dO, lnden, scale)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (O, lnden, dQ, dK, dV)]


def check_all(c, what, wseed=0, m=None):
    d = c["d"]
    Wb = gen.make_favor_directions(d if m is None else m, d, seed=wseed)
    scale = 1.0 / np.sqrt(d)
    O, lnden, dQ, dK, dV = run(c, Wb, scale)
    Q, K, V, dO = (f64(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    W = f64(Wb, "bf16")
    Or, lr = performer_fwd(Q, K, V, W, scale)
    check_fwd(O, Or, what=what)
    e = float(np.max(np.abs(lnden - lr)))
    say(f"{what} ln den max-abs {e:.3e}")
    assert np.all(np.isfinite(lnden)) and e <= 1e-2, (what, e)
    ref = performer_bwd(Q, K, V, W, dO, scale)
    if K.shape[0] == 1:
        # one source row: O = V[0] whatever Q and K are, so dQ and dK are 0
        # up to rounding; checked against the size of dV's terms
        for name, x in (("dQ", dQ), ("dK", dK)):
            m = float(np.max(np.abs(x)))
            say(f"{what} {name} (exactly 0) max {m:.3e}")
            assert m <= 1e-2 * max(1.0, float(np.max(np.abs(dO)))), (what, name, m)
        rf = rel_f(dV, ref[2])
        say(f"{what} dV rel-F {rf:.3e}")
        assert rf <= 1e-2, (what, rf)
    else:
        check_grads((dQ, dK, dV), ref, what=what)


SHAPES = [
    (300, 517, 128, 200, 1.0),
    (1, 1, 128, 200, 1.0),
    (129, 1000, 128, 200, 1.0),
    (77, 33, 64, 30, 1.0),
    (513, 1100, 128, 7, 1.0),
    (200, 150, 128, 255, 1.0),
    (260, 700, 64, 128, 1.0),
    (400, 600, 128, 200, 6.0),   # large exponents: would overflow fp32 unshifted
]


@pytest.mark.parametrize("nN,nM,d,k,spread", SHAPES)
def test_performer_parity_small(nN, nM, d, k, spread):
    say("performer small", nN, nM, d, k, spread)
    c = gen.make_small(nN, nM, d, k, "bf16", seed=5 * nN + nM, spread=spread)
    check_all(c, f"performer {nN}x{nM} d{d} k{k} spread{spread}", wseed=nN)


@pytest.mark.parametrize("nN,nM,d,k,m", [(300, 517, 128, 200, 64), (260, 700, 64, 128, 128),
                                         (129, 1000, 64, 30, 64), (400, 600, 128, 200, 64)])
def test_performer_feature_count(nN, nM, d, k, m):
    """m random features other than d (fewer, or more than the row width):
    the directions W are m x d and every output matches the oracle's
    estimator with the same W."""
    say("performer m", nN, nM, d, k, m)
    c = gen.make_small(nN, nM, d, k, "bf16", seed=7 * nN + nM + m)
    check_all(c, f"performer {nN}x{nM} d{d} k{k} m{m}", wseed=m, m=m)


def test_performer_parity_60k():
    c = gen.cached_config(2)
    say("performer 60k", c["n"], c["d"], c["k"])
    check_all(c, "performer 60k")


def test_performer_autograd_and_determinism():
    c = gen.make_small(200, 300, 128, 200, "bf16", seed=12)
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    W = to_dev(gen.make_favor_directions(128, 128, seed=4), "bf16")
    Qr, Kr, Vr = (t.clone().requires_grad_(True) for t in (Q, K, V))
    O = ssc.performer_coupling(Qr, Kr, Vr, W)
    O.backward(dO.float())
    O2, l2 = ssc.coupling_performer_fwd(Q, K, V, W)
    g2 = ssc.coupling_performer_bwd(Q, K, V, W, O2, dO, l2)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    for a, b in zip((Qr.grad, Kr.grad, Vr.grad), g2):
        assert torch.equal(a.float(), b.to(a.dtype).float())
    O3, _ = ssc.coupling_performer_fwd(Q, K, V, W)
    assert torch.equal(O2, O3)


def test_performer_rejects_unsupported():
    Q = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    V = torch.zeros(4, 256, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(128, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ssc.CouplingError):
        ssc.coupling_performer_fwd(Q, Q, V, W)     # k = 256: no column for the normaliser
    Q96 = torch.zeros(4, 96, dtype=torch.bfloat16, device="cuda")
    W96 = torch.zeros(96, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ssc.CouplingError):
        ssc.coupling_performer_fwd(Q96, Q96, V[:, :8].contiguous(), W96)   # d = 96
    with pytest.raises(ssc.CouplingError):
        ssc.coupling_performer_fwd(Q, Q, V[:, :8].contiguous(), W, scale=-1.0)


def test_performer_without_target_rows():
    """n_N = 0: the backward writes dK = dV = 0, as the linear coupling's."""
    say("performer without target rows")
    c = gen.make_small(1, 300, 128, 200, "bf16", seed=8)
    K, V = to_dev(c["K"], "bf16"), to_dev(c["V"], "bf16")
    W = to_dev(gen.make_favor_directions(128, 128, seed=5), "bf16")
    Q = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    dO = torch.empty(0, 200, dtype=torch.bfloat16, device="cuda")
    O, lnden = ssc.coupling_performer_fwd(Q, K, V, W, 128 ** -0.5)
    assert O.shape == (0, 200)
    dQ, dK, dV = ssc.coupling_performer_bwd(Q, K, V, W, O, dO, lnden, 128 ** -0.5)
    torch.cuda.synchronize()
    assert dQ.shape == (0, 128)
    assert torch.count_nonzero(dK).item() == 0 and torch.count_nonzero(dV).item() == 0
