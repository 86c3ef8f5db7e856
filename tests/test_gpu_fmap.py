"""GPU parity of the functional-map solve C = (Phi^T Phi)^-1 Phi^T O and its
backward dO = Phi (Phi^T Phi)^-1 dC against the fp64 oracle, through the C ABI.

Bars: C is a forward output (max-abs <= 2e-2, rel-Frobenius <= 5e-3), dO a
gradient (rel-Frobenius <= 1e-2).  What the arithmetic gives: Phi enters
exactly (bf16), O as a bf16 high + low pair (relative error about 2^-17), the
Gram sums accumulate in fp32 and the factor and solves run in fp32, so C is
off by roughly kappa(Phi^T Phi) * 1e-5; in the backward the solved X is
rounded to bf16 once before the row product (about 2^-9 / sqrt(3) relative
per element, about 1.1e-3 rel-Frobenius in dO).  Every output is checked in
full, also at 60k rows: the oracle is O(n k^2) here.
"""

import numpy as np
import pytest
import torch

import gen
import spatial_spectral_coupling_amd as ssc
from oracle import dense_fwd, fmap_solve, fmap_solve_bwd
from tests._util import FWD_MAX_ABS, FWD_REL_F, GRAD_REL_F, f64, rel_f, say, to_dev

pytestmark = pytest.mark.gpu


def rhs(Phi64, seed, noise=0.1):
    """O = Phi C0 + noise (fp32), a planted map plus a residual outside the
    basis span, from a seeded stream."""
    n, k = Phi64.shape
    rng = np.random.default_rng([9911, seed, n, k])
    C0 = rng.standard_normal((k, k))
    return (Phi64 @ C0 + noise * rng.standard_normal((n, k))).astype(np.float32)


def check_C(C, ref, what):
    C = np.asarray(C, np.float64)
    err = float(np.max(np.abs(C - ref)))
    rf = rel_f(C, ref)
    say(f"{what} C max-abs {err:.3e} rel-F {rf:.3e}")
    assert np.all(np.isfinite(C)), what
    assert err <= FWD_MAX_ABS, (what, err)
    assert rf <= FWD_REL_F, (what, rf)


def check_dO(dO, ref, what):
    dO = np.asarray(dO, np.float64)
    rf = rel_f(dO, ref)
    say(f"{what} dO rel-F {rf:.3e}")
    assert np.all(np.isfinite(dO)), what
    assert rf <= GRAD_REL_F, (what, rf)


SHAPES = [
    # (n, k, cond): ragged row blocks (2048 rows per Gram block), every padded
    # width (32, 64, 128, 224, 256) with ragged columns, the smallest cases
    (1, 1, 1.0),
    (7, 7, 1.0),
    (300, 7, 1.0),
    (2049, 33, 1.0),
    (4097, 64, 3.0),
    (5000, 200, 1.0),
    (3001, 224, 10.0),
    (3000, 256, 1.0),
    (6000, 129, 10.0),
]


@pytest.mark.parametrize("n,k,cond", SHAPES)
def test_fmap_parity(n, k, cond):
    what = f"fmap n={n} k={k} cond={cond}"
    say(what)
    Pb = gen.make_basis(n, k, seed=n + k, cond=cond)
    Phi = f64(Pb, "bf16")
    O = rhs(Phi, seed=1)
    dC = np.random.default_rng([77, n, k]).standard_normal((k, k)).astype(np.float32)
    Pd = to_dev(Pb, "bf16")
    C = ssc.fmap_solve_fwd(Pd, torch.from_numpy(O).cuda())
    dO = ssc.fmap_solve_bwd(Pd, torch.from_numpy(dC).cuda())
    torch.cuda.synchronize()
    check_C(C.cpu().numpy(), fmap_solve(Phi, O.astype(np.float64)), what)
    check_dO(dO.cpu().numpy(), fmap_solve_bwd(Phi, dC.astype(np.float64)), what)


def test_fmap_full_size_60k():
    """60k rows, k = 200: the basis size of the 60k-vertex coupling."""
    n, k = 60000, 200
    what = f"fmap n={n} k={k}"
    say(what)
    Pb = gen.make_basis(n, k, seed=5)
    Phi = f64(Pb, "bf16")
    O = rhs(Phi, seed=2)
    dC = np.random.default_rng([78, n, k]).standard_normal((k, k)).astype(np.float32)
    Pd = to_dev(Pb, "bf16")
    C = ssc.fmap_solve_fwd(Pd, torch.from_numpy(O).cuda())
    dO = ssc.fmap_solve_bwd(Pd, torch.from_numpy(dC).cuda())
    torch.cuda.synchronize()
    check_C(C.cpu().numpy(), fmap_solve(Phi, O.astype(np.float64)), what)
    check_dO(dO.cpu().numpy(), fmap_solve_bwd(Phi, dC.astype(np.float64)), what)


def test_fmap_after_the_coupling():
    """The pipeline the solve serves: O = coupling forward on the GPU, then C;
    the oracle runs both steps in fp64 on the same inputs."""
    c = gen.make_small(3000, 2500, 128, 200, "bf16", seed=11)
    what = "coupling -> fmap 3000x2500 k=200"
    say(what)
    Pb = gen.make_basis(3000, 200, seed=12)
    Q, K, V = (to_dev(c[x], "bf16") for x in ("Q", "K", "V"))
    O, _ = ssc.coupling_dense_fwd(Q, K, V)
    C = ssc.fmap_solve_fwd(to_dev(Pb, "bf16"), O)
    torch.cuda.synchronize()
    Or, _ = dense_fwd(*(f64(c[x], "bf16") for x in ("Q", "K", "V")), c["scale"])
    check_C(C.cpu().numpy(), fmap_solve(f64(Pb, "bf16"), Or), what)


def test_fmap_autograd():
    n, k = 1500, 64
    say(f"fmap autograd n={n} k={k}")
    Pb = gen.make_basis(n, k, seed=3, cond=2.0)
    Phi = f64(Pb, "bf16")
    O = torch.from_numpy(rhs(Phi, seed=3)).cuda().requires_grad_(True)
    dC = np.random.default_rng(79).standard_normal((k, k))
    C = ssc.fmap_solve(to_dev(Pb, "bf16"), O)
    C.backward(torch.from_numpy(dC.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    check_C(C.detach().cpu().numpy(), fmap_solve(Phi, O.detach().cpu().numpy().astype(np.float64)), "autograd")
    check_dO(O.grad.cpu().numpy(), fmap_solve_bwd(Phi, dC), "autograd")


def test_fmap_rejects_unsupported():
    n, k = 100, 16
    O = torch.zeros(n, k, device="cuda")
    # fp32 basis: unsupported
    with pytest.raises(ssc.CouplingError):
        ssc.fmap_solve_fwd(torch.zeros(n, k, device="cuda"), O)
    # k beyond 256
    with pytest.raises(ssc.CouplingError):
        ssc.fmap_solve_fwd(torch.zeros(400, 257, device="cuda", dtype=torch.bfloat16),
                           torch.zeros(400, 257, device="cuda"))
    # workspace one byte short
    lib = ssc.lib()
    P = torch.zeros(n, k, device="cuda", dtype=torch.bfloat16)
    C = torch.empty(k, k, device="cuda")
    need = lib.ssc_workspace_bytes(ssc.OP_FMAP_FWD, 1, n, 0, 0, k, 0, 0, 0)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = lib.fmap_solve_fwd(1, n, k, P.data_ptr(), O.data_ptr(), C.data_ptr(), ws.data_ptr(), need - 1,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 3  # workspace too small
    torch.cuda.synchronize()
