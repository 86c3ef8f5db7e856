"""GPU parity of the dense coupling (through the C ABI) against the fp64 oracle.

Forward O: max-abs <= 2e-2 and rel-Frobenius <= 5e-3; dQ, dK, dV:
rel-Frobenius <= 1e-2 (bf16 inputs with fp32 accumulation; fp32 inputs use
the same bars).  Sizes span several 128-row blocks and 64-key tiles with
ragged tails; the 60k workload is checked on sampled rows, on a backward whose
upstream gradient is restricted to sampled rows, and on identities that hold
at any size.
"""

import math

import numpy as np
import pytest
import torch

import gen
import spatial_spectral_coupling_amd as ssc
from oracle import dense_bwd, dense_fwd, dense_rows, rowdot
from tests._util import check_fwd, check_grads, f64, rel_f, say, to_dev

pytestmark = pytest.mark.gpu


def run_dense(c):
    dt = c["dtype"]
    Q, K, V, dO = (to_dev(c[x], dt) for x in ("Q", "K", "V", "dO"))
    O, lse = ssc.coupling_dense_fwd(Q, K, V, c["scale"])
    dQ, dK, dV = ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, c["scale"])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (O, lse, dQ, dK, dV)]


def oracle_dense(c):
    dt = c["dtype"]
    Q, K, V, dO = (f64(c[x], dt) for x in ("Q", "K", "V", "dO"))
    O, lse = dense_fwd(Q, K, V, c["scale"])
    return O, lse, dense_bwd(Q, K, V, dO, c["scale"])


SHAPES = [
    ("bf16", 300, 517, 128, 200),
    ("bf16", 129, 1000, 128, 200),
    ("bf16", 1, 1, 128, 200),
    ("bf16", 77, 33, 64, 30),
    ("bf16", 200, 333, 128, 256),
    ("bf16", 200, 150, 128, 100),
    ("bf16", 64, 96, 64, 64),
    ("bf16", 257, 16, 128, 1),
    # padded-width boundaries: forward kp 224 / backward kp 256 (k = 223);
    # forward with its ones column, backward without spare columns (k = 255)
    ("bf16", 150, 170, 128, 223),
    ("bf16", 190, 210, 64, 255),
    ("f32", 300, 517, 64, 30),
    ("f32", 150, 260, 128, 128),
]


@pytest.mark.parametrize("dt,nN,nM,d,k", SHAPES)
def test_dense_parity_small(dt, nN, nM, d, k):
    say("dense small", dt, nN, nM, d, k)
    c = gen.make_small(nN, nM, d, k, dt, seed=nN + nM)
    O, lse, dQ, dK, dV = run_dense(c)
    Or, lser, gr = oracle_dense(c)
    check_fwd(O, Or, lse, lser, what=f"{dt} {nN}x{nM} d{d} k{k}")
    check_grads((dQ, dK, dV), gr, what=f"{dt} {nN}x{nM} d{d} k{k}")


@pytest.mark.parametrize("i", [0, 1])
def test_dense_workload_parity(i):
    say("dense workload", i)
    c = gen.make_config(i)
    O, lse, dQ, dK, dV = run_dense(c)
    Or, lser, gr = oracle_dense(c)
    check_fwd(O, Or, lse, lser, what=c["config"])
    check_grads((dQ, dK, dV), gr, what=c["config"])


def test_dense_one_hot_permutation_returns_permuted_basis():
    say("dense one-hot permutation")
    n = d = 128
    pi = np.random.default_rng(3).permutation(n)
    FN = np.zeros((n, d), np.float32)
    FN[np.arange(n), pi] = 16.0
    FM = np.zeros((n, d), np.float32)
    FM[np.arange(n), np.arange(n)] = 16.0
    Phi = gen.make_small(n, n, d, 200, "bf16", seed=9)["V"]
    Q, K = to_dev(gen.bf16_bits_from_f32(FN), "bf16"), to_dev(gen.bf16_bits_from_f32(FM), "bf16")
    V = to_dev(Phi, "bf16")
    O, _ = ssc.coupling_dense_fwd(Q, K, V, 1 / math.sqrt(d))
    err = np.max(np.abs(O.cpu().numpy() - f64(Phi, "bf16")[pi]))
    say("one-hot max-abs", err)
    assert err < 1e-3


def test_dense_rows_of_map_sum_to_one_and_determinism():
    say("dense ones column + determinism")
    c = gen.make_small(700, 900, 128, 200, "bf16", seed=5)
    V = c["V"].copy()
    V[:, 7] = gen.bf16_bits_from_f32(np.ones(900, np.float32))
    Q, K, Vd, dO = to_dev(c["Q"], "bf16"), to_dev(c["K"], "bf16"), to_dev(V, "bf16"), to_dev(c["dO"], "bf16")
    O1, l1 = ssc.coupling_dense_fwd(Q, K, Vd)
    O2, l2 = ssc.coupling_dense_fwd(Q, K, Vd)
    g1 = ssc.coupling_dense_bwd(Q, K, Vd, O1, dO, l1)
    g2 = ssc.coupling_dense_bwd(Q, K, Vd, O1, dO, l1)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    col = O1[:, 7].cpu().numpy()
    say("ones column max dev", np.max(np.abs(col - 1)))
    assert np.max(np.abs(col - 1)) < 1e-2


def test_dense_reference_fallbacks():
    """The forward's first pass takes each row's reference from the bound
    |q| max|k| on its scores.  Row 5 (query 60 e1) meets a key of norm 60
    orthogonal to it, so the bound sits 459 (log2 units) above its scores and
    its row sum underflows: the workgroup redoes its rows with a running
    reference, and since a later tile's maximum (key 200 = 5 e1, 38 above the
    first tile's) runs more than 32 ahead of it, once more with exact row
    maxima.  Row 129 (query 60 e3, second workgroup) only needs the running
    reference.  Both workgroups must still match the oracle."""
    say("dense reference fallbacks")
    nN, nM, d, k = 130, 300, 128, 200
    c = gen.make_small(nN, nM, d, k, "bf16", seed=21)
    Qf = f64(c["Q"], "bf16").astype(np.float32)
    Kf = f64(c["K"], "bf16").astype(np.float32)
    Qf[5] = 0.0
    Qf[5, 0] = 60.0
    Qf[129] = 0.0
    Qf[129, 2] = 60.0
    Kf[:, 0] = 0.0               # no key but 200 leans along e1
    Kf[200] = 0.0
    Kf[200, 0] = 5.0
    Kf[250] = 0.0
    Kf[250, 1] = 60.0            # the largest key norm, orthogonal to rows 5 and 129
    c["Q"], c["K"] = gen.bf16_bits_from_f32(Qf), gen.bf16_bits_from_f32(Kf)
    scale = 1 / math.sqrt(d)
    Q, K, V = (to_dev(c[x], "bf16") for x in ("Q", "K", "V"))
    O, lse = ssc.coupling_dense_fwd(Q, K, V, scale)
    Or, lser = dense_fwd(f64(c["Q"], "bf16"), f64(c["K"], "bf16"), f64(c["V"], "bf16"), scale)
    check_fwd(O.cpu().numpy(), Or, lse.cpu().numpy(), lser, what="reference fallbacks")
    err5 = np.max(np.abs(O[5].cpu().numpy() - Or[5]))
    say("row 5 max-abs", err5)
    assert err5 <= 2e-2


def test_dense_60k_full_size_sampled():
    """The 60k workload: sampled rows of O, lse and dQ; dK/dV of a backward
    whose upstream gradient lives on sampled rows; identities at full size."""
    say("dense 60k generate")
    c = gen.make_config(2)
    dt, sc = c["dtype"], c["scale"]
    Q, K, V, dO = (to_dev(c[x], dt) for x in ("Q", "K", "V", "dO"))
    say("dense 60k fwd+bwd")
    O, lse = ssc.coupling_dense_fwd(Q, K, V, sc)
    dQ, dK, dV = ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, sc)
    torch.cuda.synchronize()
    n = c["n"]
    rng = np.random.default_rng(0)
    rows = np.unique(np.r_[0, 1, 127, 128, n - 1, rng.choice(n, 250, replace=False)])
    Qf, Kf, Vf, dOf = (f64(c[x], dt) for x in ("Q", "K", "V", "dO"))
    say("dense 60k oracle rows", len(rows))
    Or, lser = dense_rows(Qf, Kf, Vf, sc, rows)
    check_fwd(O.cpu().numpy()[rows], Or, lse.cpu().numpy()[rows], lser, what="60k sampled rows")
    # dQ of a row needs only that row's softmax
    dQr, _, _ = dense_bwd(Qf[rows], Kf, Vf, dOf[rows], sc)
    rf = rel_f(dQ.cpu().numpy()[rows], dQr)
    say("60k sampled dQ rel-F", rf)
    assert rf <= 1e-2
    # identities of the full backward
    dKn, dVn = dK.double().cpu().numpy(), dV.double().cpu().numpy()
    colsum_rel = np.linalg.norm(dKn.sum(0)) / np.linalg.norm(np.abs(dKn).sum(0))
    say("60k sum_j dK_j relative", colsum_rel)
    assert colsum_rel < 1e-3
    dOsum = dOf.sum(0)
    e = np.linalg.norm(dVn.sum(0) - dOsum) / np.linalg.norm(dOsum)
    say("60k sum_j dV_j vs sum_i dO_i", e)
    assert e < 1e-3
    # dK, dV exactly for an upstream gradient restricted to sampled rows
    mask = torch.zeros(n, 1, dtype=dO.dtype, device=dO.device)
    mask[torch.from_numpy(rows).cuda()] = 1
    dOm = (dO * mask).contiguous()
    _, dKm, dVm = ssc.coupling_dense_bwd(Q, K, V, O, dOm, lse, sc)
    torch.cuda.synchronize()
    say("60k row-restricted oracle")
    _, dKr, dVr = dense_bwd(Qf, Kf, Vf, dOf, sc, rows=rows)
    for name, g, r in (("dK", dKm, dKr), ("dV", dVm, dVr)):
        rf = rel_f(g.cpu().numpy(), r)
        say(f"60k restricted {name} rel-F", rf)
        assert rf <= 1e-2


def test_autograd_wrapper_matches_entry_points():
    say("autograd wrapper")
    c = gen.make_small(100, 140, 64, 30, "bf16", seed=1)
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    Qr, Kr, Vr = (t.clone().requires_grad_(True) for t in (Q, K, V))
    O = ssc.dense_coupling(Qr, Kr, Vr)
    O.backward(dO.float())
    O2, lse = ssc.coupling_dense_fwd(Q, K, V)
    dQ, dK, dV = ssc.coupling_dense_bwd(Q, K, V, O2, dO, lse)
    assert torch.equal(O, O2)
    assert torch.equal(Qr.grad, dQ.to(torch.bfloat16))
    assert torch.equal(Vr.grad, dV.to(torch.bfloat16))
