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
    # the remaining padded widths of the paired forward: kp 64 at d = 128,
    # kp 224 at d = 64
    ("bf16", 150, 170, 128, 40),
    ("bf16", 140, 230, 64, 200),
    ("f32", 300, 517, 64, 30),
    ("f32", 150, 260, 128, 128),
]


# bf16 calls this small run as a one-patch geo coupling by default ("split");
# "dense" forces the dense kernels, so both routes are checked
ROUTED = [(r,) + sh for sh in SHAPES for r in (("dense", "split") if sh[0] == "bf16" else ("dense",))]


@pytest.mark.parametrize("route,dt,nN,nM,d,k", ROUTED)
def test_dense_parity_small(route, dt, nN, nM, d, k):
    say("dense small", route, dt, nN, nM, d, k)
    c = gen.make_small(nN, nM, d, k, dt, seed=nN + nM)
    with ssc.dense_route(route):
        O, lse, dQ, dK, dV = run_dense(c)
    Or, lser, gr = oracle_dense(c)
    check_fwd(O, Or, lse, lser, what=f"{dt} {nN}x{nM} d{d} k{k}")
    check_grads((dQ, dK, dV), gr, what=f"{dt} {nN}x{nM} d{d} k{k}")


@pytest.mark.parametrize("i,route", [(0, "auto"), (1, "auto"), (1, "dense")])
def test_dense_workload_parity(i, route):
    say("dense workload", i, route)
    c = gen.cached_config(i)
    with ssc.dense_route(route):
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


@pytest.mark.parametrize("route", ["dense", "split"])
def test_dense_rows_of_map_sum_to_one_and_determinism(route):
    say("dense ones column + determinism", route)
    c = gen.make_small(700, 900, 128, 200, "bf16", seed=5)
    V = c["V"].copy()
    V[:, 7] = gen.bf16_bits_from_f32(np.ones(900, np.float32))
    Q, K, Vd, dO = to_dev(c["Q"], "bf16"), to_dev(c["K"], "bf16"), to_dev(V, "bf16"), to_dev(c["dO"], "bf16")
    with ssc.dense_route(route):
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


@pytest.mark.parametrize("route", ["dense", "split"])
def test_dense_reference_fallbacks(route):
    """The forward's first pass takes each row's reference from the bound
    |q| max|k| on its scores.  Row 5 (query 60 e1) meets a key of norm 60
    orthogonal to it, so the bound sits 459 (log2 units) above its scores and
    its row sum underflows: the workgroup redoes its rows with a running
    reference, and since a later tile's maximum (key 200 = 5 e1, 38 above the
    first tile's) runs more than 32 ahead of it, once more with exact row
    maxima.  Row 129 (query 60 e3, second workgroup) only needs the running
    reference.  Both workgroups must still match the oracle (on the dense
    kernels, and on the one-patch geo route with its split items)."""
    say("dense reference fallbacks", route)
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
    with ssc.dense_route(route):
        O, lse = ssc.coupling_dense_fwd(Q, K, V, scale)
    Or, lser = dense_fwd(f64(c["Q"], "bf16"), f64(c["K"], "bf16"), f64(c["V"], "bf16"), scale)
    check_fwd(O.cpu().numpy(), Or, lse.cpu().numpy(), lser, what=f"reference fallbacks {route}")
    err5 = np.max(np.abs(O[5].cpu().numpy() - Or[5]))
    say("row 5 max-abs", err5)
    assert err5 <= 2e-2


@pytest.mark.timeout(900)
def test_dense_60k_full_size_sampled():
    """The 60k workload: sampled rows of O, lse and dQ; dK/dV of a backward
    whose upstream gradient lives on sampled rows; identities at full size."""
    say("dense 60k generate")
    c = gen.cached_config(2)
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


def test_dense_60k_full_size():
    """The 60k workload against the oracle on every element: O and lse, and
    dQ, dK, dV of the workload's own upstream gradient (the oracle runs in
    full-row blocks on the host cores, about half a minute)."""
    say("dense 60k full generate")
    c = gen.cached_config(2)
    say("dense 60k full gpu")
    O, lse, dQ, dK, dV = run_dense(c)
    say("dense 60k full oracle")
    Or, lser, gr = oracle_dense(c)
    check_fwd(O, Or, lse, lser, what="60k full")
    check_grads((dQ, dK, dV), gr, what="60k full")


@pytest.mark.parametrize("route,dt,nN,nM,d,k", [(r, "bf16", 300, 517, 128, 200) for r in ("dense", "split")] +
                         [(r, "bf16", 200, 333, 128, 256) for r in ("dense", "split")] +
                         [(r, "bf16", 77, 33, 64, 30) for r in ("dense", "split")] +
                         [("dense", "f32", 150, 260, 128, 128)])
def test_dense_backward_without_dv(route, dt, nN, nM, d, k):
    """dV = NULL: the dV products are skipped; dQ and dK are the bits of the
    full call and match the oracle."""
    say("dense bwd without dV", route, dt, nN, nM, d, k)
    c = gen.make_small(nN, nM, d, k, dt, seed=nN + 2 * nM)
    Q, K, V, dO = (to_dev(c[x], dt) for x in ("Q", "K", "V", "dO"))
    with ssc.dense_route(route):
        O, lse = ssc.coupling_dense_fwd(Q, K, V, c["scale"])
        dQ, dK, dV = ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, c["scale"])
        dQ2, dK2, dV2 = ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, c["scale"], need_dV=False)
    torch.cuda.synchronize()
    assert dV2 is None
    assert torch.equal(dQ2, dQ) and torch.equal(dK2, dK)
    _, _, gr = oracle_dense(c)
    check_grads((dQ2.cpu().numpy(), dK2.cpu().numpy(), dV.cpu().numpy()), gr, what=f"no-dV {dt} k{k}")


def test_autograd_skips_dv_for_a_fixed_basis():
    say("autograd fixed basis")
    c = gen.make_small(100, 140, 64, 30, "bf16", seed=2)
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    Qr, Kr = Q.clone().requires_grad_(True), K.clone().requires_grad_(True)
    O = ssc.dense_coupling(Qr, Kr, V)
    O.backward(dO.float())
    O2, lse = ssc.coupling_dense_fwd(Q, K, V)
    dQ, dK, _ = ssc.coupling_dense_bwd(Q, K, V, O2, dO, lse, need_dV=False)
    assert torch.equal(Qr.grad, dQ.to(torch.bfloat16)) and torch.equal(Kr.grad, dK.to(torch.bfloat16))


@pytest.mark.parametrize("route,nN,nM,d,k", [(r,) + sh for sh in ((300, 40000, 128, 200), (70, 33000, 64, 30),
                                                                  (1, 32897, 128, 200))
                                             for r in ("dense", "auto")])
def test_dense_backward_many_key_blocks(route, nN, nM, d, k):
    """More key blocks of 128 rows than one round of 256 workgroups (the
    dK / dV pass runs in two rounds) with few query rows: one to five query
    tiles, ragged in both directions (on the dense kernels, and by default on
    the one-patch route: split dQ items, whole dK/dV items)."""
    say("dense bwd many key blocks", route, nN, nM, d, k)
    c = gen.make_small(nN, nM, d, k, "bf16", seed=nN + nM)
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    with ssc.dense_route(route):
        O, lse = ssc.coupling_dense_fwd(Q, K, V, c["scale"])
        dQ, dK, dV = ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, c["scale"])
        _, dK2, dV2 = ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, c["scale"], need_dV=False)
    torch.cuda.synchronize()
    assert dV2 is None and torch.equal(dK2, dK)
    O_r, lse_r, gr = oracle_dense(c)
    check_fwd(O.cpu().numpy(), O_r, lse.cpu().numpy(), lse_r, what=f"many blocks {nM}")
    check_grads((dQ.cpu().numpy(), dK.cpu().numpy(), dV.cpu().numpy()), gr, what=f"many blocks {nM}")


@pytest.mark.parametrize("nN,nM,d,k", [(32800, 517, 128, 200), (33000, 130, 128, 100), (32900, 70, 128, 40),
                                       (32800, 65, 128, 1), (32850, 300, 64, 200), (32800, 96, 64, 30),
                                       (32800, 200, 64, 100), (32800, 100, 64, 64)])
def test_dense_wide_forward(nN, nM, d, k):
    """From 128 workgroups of 256 rows on (n_N >= 32513) the forward runs the
    wide-wave kernel (a wave owns 64 rows): every padded width it has, ragged
    row and key tails, against the oracle."""
    say("dense wide fwd", nN, nM, d, k)
    c = gen.make_small(nN, nM, d, k, "bf16", seed=nN + nM + k)
    Q, K, V = (to_dev(c[x], "bf16") for x in ("Q", "K", "V"))
    O, lse = ssc.coupling_dense_fwd(Q, K, V, c["scale"])
    torch.cuda.synchronize()
    Or, lser = dense_fwd(f64(c["Q"], "bf16"), f64(c["K"], "bf16"), f64(c["V"], "bf16"), c["scale"])
    check_fwd(O.cpu().numpy(), Or, lse.cpu().numpy(), lser, what=f"wide {nN}x{nM} d{d} k{k}")


def test_dense_wide_forward_fallback():
    """The wide kernel's underflow marks: row 5 (query 60 e1 against a key of
    norm 60 orthogonal to it) and row 32700 (in the last workgroup) send
    their 128-row blocks to the one-wave kernel; all rows match the oracle."""
    say("dense wide fwd fallback")
    nN, nM, d, k = 32800, 300, 128, 200
    c = gen.make_small(nN, nM, d, k, "bf16", seed=23)
    Qf = f64(c["Q"], "bf16").astype(np.float32)
    Kf = f64(c["K"], "bf16").astype(np.float32)
    for r, axis in ((5, 0), (32700, 2)):
        Qf[r] = 0.0
        Qf[r, axis] = 60.0
    Kf[:, 0] = 0.0
    Kf[:, 2] = 0.0
    Kf[250] = 0.0
    Kf[250, 1] = 60.0
    c["Q"], c["K"] = gen.bf16_bits_from_f32(Qf), gen.bf16_bits_from_f32(Kf)
    Q, K, V = (to_dev(c[x], "bf16") for x in ("Q", "K", "V"))
    O, lse = ssc.coupling_dense_fwd(Q, K, V, c["scale"])
    torch.cuda.synchronize()
    Or, lser = dense_fwd(f64(c["Q"], "bf16"), f64(c["K"], "bf16"), f64(c["V"], "bf16"), c["scale"])
    check_fwd(O.cpu().numpy(), Or, lse.cpu().numpy(), lser, what="wide fallback")
    for r in (5, 32700):
        assert np.max(np.abs(O[r].cpu().numpy() - Or[r])) <= 2e-2


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_dense_without_target_rows(dt):
    """n_N = 0: the forward returns empty outputs and the backward writes
    dK = dV = 0 (nothing reads the empty Q, O, dO, lse)."""
    say("dense without target rows", dt)
    c = gen.make_small(1, 300, 64, 30, dtype=dt, seed=6)
    K, V = to_dev(c["K"], dt), to_dev(c["V"], dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    Q = torch.empty(0, 64, dtype=tdt, device="cuda")
    dO = torch.empty(0, 30, dtype=tdt, device="cuda")
    O, lse = ssc.coupling_dense_fwd(Q, K, V, 0.125)
    assert O.shape == (0, 30) and lse.shape == (0,)
    dQ, dK, dV = ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, 0.125)
    torch.cuda.synchronize()
    assert dQ.shape == (0, 64)
    assert torch.count_nonzero(dK).item() == 0 and torch.count_nonzero(dV).item() == 0


def test_dense_route_by_size():
    """By default a bf16 call with at most 128 row blocks a side takes the
    one-patch geo route (its kernels are timed as the geo families); the 60k
    workload and a "dense" route take the dense kernels."""
    say("dense route by size")
    c = gen.make_small(5000, 5000, 128, 200, "bf16", seed=31)
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))

    def launches(family, route, Q, K, V, dO):
        with ssc.dense_route(route), ssc.KernelTimer(family, 8) as t:
            O, lse = ssc.coupling_dense_fwd(Q, K, V)
            ssc.coupling_dense_bwd(Q, K, V, O, dO, lse)
            return t.read()[1]

    assert launches("geo_fwd", "auto", Q, K, V, dO) == 1 and launches("geo_dkv", "auto", Q, K, V, dO) == 1
    assert launches("fwd", "auto", Q, K, V, dO) == 0
    assert launches("geo_fwd", "dense", Q, K, V, dO) == 0 and launches("dkv", "dense", Q, K, V, dO) == 1
    n = 16512  # 129 row blocks of 128: past the split route
    c = gen.make_small(n, 300, 64, 30, "bf16", seed=32)
    Q, K, V, dO = (to_dev(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    assert launches("geo_fwd", "auto", Q, K, V, dO) == 0 and launches("fwd", "auto", Q, K, V, dO) == 1
    # 129 query blocks but 3 key blocks: the backward's short side routes it
    assert launches("geo_dkv", "auto", Q, K, V, dO) == 1 and launches("dkv", "auto", Q, K, V, dO) == 0


@pytest.mark.parametrize("route", ["dense", "auto"])
def test_dense_lopsided_backward(route):
    """20000 target rows (157 blocks: whole dQ items) against 3000 source rows
    (24 blocks: split dK/dV items on the default route), every element
    against the oracle."""
    say("dense lopsided", route)
    c = gen.make_small(20000, 3000, 128, 200, "bf16", seed=43)
    with ssc.dense_route(route):
        O, lse, dQ, dK, dV = run_dense(c)
    Or, lser, gr = oracle_dense(c)
    check_fwd(O, Or, lse, lser, what=f"lopsided {route}")
    check_grads((dQ, dK, dV), gr, what=f"lopsided {route}")


@pytest.mark.timeout(600)
def test_dense_12k_split_route_full():
    """12000 x 12000 (the pages' smaller workloads are about this size): the
    default route splits each of the 94 row blocks' key streams in two;
    every element of O, lse, dQ, dK, dV against the oracle."""
    say("dense 12k split route")
    c = gen.make_small(12000, 12000, 128, 200, "bf16", seed=41)
    O, lse, dQ, dK, dV = run_dense(c)
    say("dense 12k oracle")
    Or, lser, gr = oracle_dense(c)
    check_fwd(O, Or, lse, lser, what="12k split route")
    check_grads((dQ, dK, dV), gr, what="12k split route")


def test_dense_split_route_past_half_a_round():
    """20000 x 2000 forced onto the one-patch route: 157 query blocks leave
    more than half a round over, so they stay whole items (splitting the
    cheapest in two was measured slower); 16 key blocks split in eight."""
    say("dense split route, 157 query blocks")
    c = gen.make_small(20000, 2000, 128, 200, "bf16", seed=44)
    with ssc.dense_route("split"):
        O, lse, dQ, dK, dV = run_dense(c)
    Or, lser, gr = oracle_dense(c)
    check_fwd(O, Or, lse, lser, what="split 157 blocks")
    check_grads((dQ, dK, dV), gr, what="split 157 blocks")
