"""GPU parity of the Geo-FlashAttention path (through the C ABI) against the
fp64 oracle, which works in the original vertex order from patch labels.

Top-s indices: bit-exact (rows whose s-th and (s+1)-th oracle scores tie to
rounding must still be a valid top-s).  O: max-abs <= 2e-2, rel-Frobenius <=
5e-3; dQ, dK, dV: rel-Frobenius <= 1e-2.
"""

import numpy as np
import pytest
import torch

import gen
import spatial_spectral_coupling_amd as ssc
from oracle import (dense_bwd, dense_fwd, geo_bwd, geo_fwd, patch_means, patch_scores, topk)
from tests._util import check_fwd, check_grads, check_idx, f64, say, sorted_problem, to_dev, unsort

pytestmark = pytest.mark.gpu


def gpu_geo(dev, s, scale, idx=None, dO=None):
    if idx is None:
        idx, C = ssc.patch_score_topk(dev["Q"], dev["offN"], dev["K"], dev["offM"], s, return_scores=True)
    else:
        C = None
    O, lse = ssc.coupling_geo_fwd(dev["Q"], dev["K"], dev["V"], dev["offN"], dev["offM"], idx, scale)
    g = ssc.coupling_geo_bwd(dev["Q"], dev["K"], dev["V"], dev["offN"], dev["offM"], idx, O,
                             dev["dO"] if dO is None else dO, lse, scale)
    torch.cuda.synchronize()
    return idx, C, O, lse, g


def oracle_geo(c, s, rows_only=None):
    dt = c["dtype"]
    Q, K, V, dO = (f64(c[x], dt) for x in ("Q", "K", "V", "dO"))
    P_N = c.get("P_N", c.get("P"))
    P_M = c.get("P_M", c.get("P"))
    C = patch_scores(patch_means(Q, c["labN"], P_N), patch_means(K, c["labM"], P_M))
    idx = topk(C, s)
    return Q, K, V, dO, C, idx


def compare_geo(c, s, what):
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    sc = c["scale"]
    say(what, "gpu")
    idx, C, O, lse, (dQ, dK, dV) = gpu_geo(dev, s, sc)
    say(what, "oracle")
    Q, K, V, dO, Cr, idxr = oracle_geo(c, s)
    np.testing.assert_allclose(C.cpu().numpy(), Cr, rtol=1e-12, atol=1e-12 * np.abs(Cr).max())
    check_idx(idx.cpu().numpy(), idxr, Cr, s, what)
    idx_np = idx.cpu().numpy()  # equal to idxr except on audited near-tie rows
    Or, lser = geo_fwd(Q, K, V, c["labN"], c["labM"], idx_np, sc)
    check_fwd(unsort(O.cpu().numpy(), permN), Or, unsort(lse.cpu().numpy(), permN), lser, what)
    gr = geo_bwd(Q, K, V, dO, c["labN"], c["labM"], idx_np, sc)
    got = (unsort(dQ.cpu().numpy(), permN), unsort(dK.cpu().numpy(), permM), unsort(dV.cpu().numpy(), permM))
    check_grads(got, gr, what)
    return dev, idx


GEO_SHAPES = [
    # dtype, n_N, n_M, d, k, P_N, P_M, s
    ("bf16", 600, 700, 128, 200, 9, 11, 3),
    ("bf16", 1500, 1300, 128, 200, 12, 10, 4),
    ("bf16", 400, 450, 64, 30, 7, 6, 2),
    ("bf16", 300, 260, 128, 200, 5, 5, 5),   # s = P_M
    ("bf16", 90, 300, 128, 100, 4, 25, 1),
    ("f32", 500, 520, 64, 30, 6, 8, 3),
    ("bf16", 400, 420, 64, 255, 5, 6, 2),   # forward with a ones column, backward without spare columns
    # 70 target patches: three chunks of the planner's selection passes, the
    # last one partial; s = 66 puts more entries in a chunk than its threads
    # keep in registers
    ("bf16", 700, 720, 64, 30, 70, 72, 66),
]


def test_geo_reference_fallbacks():
    """A key of norm 60 makes the forward's bounded reference (|q| max|k|)
    sit far above the scores of the query of norm 60 (original row 5), so the
    parts of its split work item redo their rows with a running reference
    while the other parts keep the bound: the merge then combines partial sums
    taken at different references."""
    c = gen.make_small(600, 700, 128, 200, "bf16", seed=31, P_N=9, P_M=11, s=3)
    Qf = f64(c["Q"], "bf16").astype(np.float32)
    Kf = f64(c["K"], "bf16").astype(np.float32)
    Qf[5] = 0.0
    Qf[5, 0] = 60.0
    Kf[:, 0] = 0.0
    Kf[200] = 0.0
    Kf[200, 0] = 5.0
    Kf[250] = 0.0
    Kf[250, 1] = 60.0
    c["Q"], c["K"] = gen.bf16_bits_from_f32(Qf), gen.bf16_bits_from_f32(Kf)
    compare_geo(c, 3, "geo reference fallbacks")


@pytest.mark.parametrize("dt,nN,nM,d,k,PN,PM,s", GEO_SHAPES)
def test_geo_parity_small(dt, nN, nM, d, k, PN, PM, s):
    c = gen.make_small(nN, nM, d, k, dt, seed=nN + 3 * nM, P_N=PN, P_M=PM, s=s)
    compare_geo(c, s, f"geo {dt} {nN}x{nM} d{d} k{k} P{PN}/{PM} s{s}")


def test_geo_full_selection_equals_dense_on_gpu():
    say("geo s=P_M vs dense")
    c = gen.make_small(700, 650, 128, 200, "bf16", seed=2, P_N=6, P_M=7, s=7)
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    _, _, O, lse, g = gpu_geo(dev, 7, c["scale"])
    Od, lsed = ssc.coupling_dense_fwd(dev["Q"], dev["K"], dev["V"], c["scale"])
    gd = ssc.coupling_dense_bwd(dev["Q"], dev["K"], dev["V"], Od, dev["dO"], lsed, c["scale"])
    # Same support; the keys arrive in another order, so the reference max at
    # which each probability is rounded to bf16 differs: the two agree to the
    # parity bars (each is separately within them of the oracle).  The row
    # sums are sums of those bf16 probabilities (relative rounding <= 2^-9
    # each), so each lse is within ln(1 + 2^-9) < 1.96e-3 of the exact one and
    # the two within twice that.
    say("geo(s=P_M) vs dense O max-abs", (O - Od).abs().max().item())
    assert (O - Od).abs().max().item() < 2e-2
    assert ((O - Od).norm() / Od.norm()).item() < 5e-3
    assert (lse - lsed).abs().max().item() < 3.92e-3
    for a, b in zip(g, gd):
        assert ((a - b).norm() / b.norm()).item() < 1e-2
    # and each of the two against the dense oracle (full selection = dense
    # support): geo and dense are pinned to the same exact result, not only
    # to each other
    Q, K, V, dO = (f64(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    Or, lser = dense_fwd(Q, K, V, c["scale"])
    gr = dense_bwd(Q, K, V, dO, c["scale"])
    for tag, Ox, lx, gx in (("geo", O, lse, g), ("dense", Od, lsed, gd)):
        check_fwd(unsort(Ox.cpu().numpy(), permN), Or, unsort(lx.cpu().numpy(), permN), lser, f"s=P_M {tag}")
        got = (unsort(gx[0].cpu().numpy(), permN), unsort(gx[1].cpu().numpy(), permM),
               unsort(gx[2].cpu().numpy(), permM))
        check_grads(got, gr, f"s=P_M {tag}")


def test_geo_empty_and_unselected_patches():
    """Empty source patches, a target patch whose support is empty, and a
    non-empty source patch that nobody selects (zero dK, dV)."""
    say("geo empty patches")
    c = gen.make_small(300, 320, 128, 200, "bf16", seed=4, P_N=5, P_M=6, s=2)
    labM = c["labM"].copy()
    labM[labM == 2] = 3          # source patch 2 is now empty
    labM[labM == 5] = 4          # source patch 5 is now empty
    c["labM"] = labM
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    # target 0 selects only empty patches; source patch 3 is never selected
    idx_np = np.array([[2, 5], [2, 1], [0, 1], [4, 2], [1, 0]], dtype=np.int32)
    idx = torch.from_numpy(idx_np).cuda()
    _, _, O, lse, (dQ, dK, dV) = gpu_geo(dev, 2, c["scale"], idx=idx)
    Q, K, V, dO = (f64(c[x], "bf16") for x in ("Q", "K", "V", "dO"))
    Or, lser = geo_fwd(Q, K, V, c["labN"], labM, idx_np, c["scale"])
    On, lsen = unsort(O.cpu().numpy(), permN), unsort(lse.cpu().numpy(), permN)
    rows0 = c["labN"] == 0
    assert np.all(On[rows0] == 0) and np.all(np.isneginf(lsen[rows0]))
    check_fwd(On, Or, lsen, lser, "geo empty")
    gr = geo_bwd(Q, K, V, dO, c["labN"], labM, idx_np, c["scale"])
    got = (unsort(dQ.cpu().numpy(), permN), unsort(dK.cpu().numpy(), permM), unsort(dV.cpu().numpy(), permM))
    assert np.all(got[0][rows0] == 0)
    check_grads(got, gr, "geo empty")
    unsel = labM == 3
    assert unsel.any()
    assert np.all(got[1][unsel] == 0) and np.all(got[2][unsel] == 0)


def test_geo_invalid_selection_fills_nan():
    """A repeated source patch in a row: the planner rejects the selection,
    nothing is computed and the outputs come back as NaN (a result of an
    invalid call cannot pass for a valid one); the call itself returns OK."""
    say("geo invalid idx")
    c = gen.make_small(200, 210, 128, 200, "bf16", seed=6, P_N=4, P_M=4, s=2)
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    bad = torch.tensor([[0, 0], [1, 2], [3, 1], [2, 0]], dtype=torch.int32, device="cuda")  # repeated entry
    O = torch.full((200, 200), 7.0, device="cuda")
    lse = torch.full((200,), 7.0, device="cuda")
    # a workspace holding leftovers (every byte 1): nothing may read a count
    # the planner did not write for this call
    ws = torch.full((ssc.workspace_bytes(ssc.OP_GEO_FWD, torch.bfloat16, 200, 210, 128, 200, 4, 4, 2),),
                    1, dtype=torch.uint8, device="cuda")
    import ctypes
    st = ssc.lib().coupling_geo_fwd(1, 128, 200, 200, 4, ctypes.c_void_p(dev["offN"].data_ptr()), 210, 4,
                                    ctypes.c_void_p(dev["offM"].data_ptr()), 2, ctypes.c_void_p(bad.data_ptr()),
                                    ctypes.c_void_p(dev["Q"].data_ptr()), ctypes.c_void_p(dev["K"].data_ptr()),
                                    ctypes.c_void_p(dev["V"].data_ptr()), 0.1, ctypes.c_void_p(O.data_ptr()),
                                    ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.all(torch.isnan(O)) and torch.all(torch.isnan(lse))


@pytest.mark.parametrize("i", [3])
def test_geo_workload_60k_full(i):
    say("geo workload generate", i)
    c = gen.cached_config(i)
    compare_geo(c, c["s"], c["config"])


def test_geo_workload_160k_sampled():
    """160k, P = 640, s = 16: bit-exact top-s everywhere; O, lse, dQ on every
    row of 48 sampled target patches; dK, dV of a backward whose upstream
    gradient lives on those patches only."""
    say("geo 160k generate")
    c = gen.cached_config(4)
    s, sc = c["s"], c["scale"]
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    say("geo 160k gpu")
    idx, C, O, lse, (dQ, dK, dV) = gpu_geo(dev, s, sc)
    Q, K, V, dO, Cr, idxr = oracle_geo(c, s)
    check_idx(idx.cpu().numpy(), idxr, Cr, s, "160k")
    idx_np = idx.cpu().numpy()
    pats = np.sort(np.random.default_rng(1).choice(P_N, 48, replace=False))
    rows = np.nonzero(np.isin(c["labN"], pats))[0]
    say("geo 160k oracle on", len(rows), "rows")
    # restrict the oracle to the sampled target patches: other labels -> none
    labN_s = np.where(np.isin(c["labN"], pats), c["labN"], -1)
    Or, lser = geo_fwd(Q, K, V, labN_s, c["labM"], idx_np, sc)
    check_fwd(unsort(O.cpu().numpy(), permN)[rows], Or[rows], unsort(lse.cpu().numpy(), permN)[rows],
              lser[rows], "160k sampled")
    dOm_np = np.zeros_like(dO)
    dOm_np[rows] = dO[rows]
    gr = geo_bwd(Q, K, V, dOm_np, labN_s, c["labM"], idx_np, sc)
    rf = np.linalg.norm(unsort(dQ.cpu().numpy(), permN)[rows] - gr[0][rows]) / np.linalg.norm(gr[0][rows])
    say("160k sampled dQ rel-F", rf)
    assert rf <= 1e-2
    maskN = torch.from_numpy(np.isin(c["labN"][permN], pats)).cuda()
    dOm = (dev["dO"] * maskN[:, None].to(dev["dO"].dtype)).contiguous()
    _, _, _, _, (_, dKm, dVm) = gpu_geo(dev, s, sc, idx=idx, dO=dOm)
    check_grads((unsort(dQ.cpu().numpy(), permN)[rows], unsort(dKm.cpu().numpy(), permM),
                 unsort(dVm.cpu().numpy(), permM)), (gr[0][rows], gr[1], gr[2]), "160k restricted")


def test_geo_repeat_in_later_chunk_fills_nan():
    """A repeated entry in row 40 (the planner's second chunk of 32 target
    patches): forward and backward compute nothing and fill every output
    with NaN; the valid selection still works afterwards, bit for bit."""
    import ctypes
    say("geo repeat in a later chunk")
    c = gen.make_small(700, 720, 64, 30, "bf16", seed=8, P_N=70, P_M=72, s=4)
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    sc = c["scale"]
    idx, _, O, lse, g = gpu_geo(dev, 4, sc)
    bad = idx.clone()
    bad[40, 3] = bad[40, 0]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    L = ssc.lib()
    O7 = torch.full_like(O, 7.0)
    lse7 = torch.full_like(lse, 7.0)
    ws = torch.empty((ssc.workspace_bytes(ssc.OP_GEO_FWD, torch.bfloat16, 700, 720, 64, 30, P_N, P_M, 4),),
                     dtype=torch.uint8, device="cuda")
    r = L.coupling_geo_fwd(1, 64, 30, 700, P_N, p(dev["offN"]), 720, P_M, p(dev["offM"]), 4, p(bad),
                           p(dev["Q"]), p(dev["K"]), p(dev["V"]), ctypes.c_float(sc), p(O7), p(lse7), p(ws),
                           ctypes.c_size_t(ws.numel()), st)
    outs = [torch.full_like(x, 7.0) for x in g]
    wsb = torch.empty((ssc.workspace_bytes(ssc.OP_GEO_BWD, torch.bfloat16, 700, 720, 64, 30, P_N, P_M, 4),),
                      dtype=torch.uint8, device="cuda")
    rb = L.coupling_geo_bwd(1, 64, 30, 700, P_N, p(dev["offN"]), 720, P_M, p(dev["offM"]), 4, p(bad),
                            p(dev["Q"]), p(dev["K"]), p(dev["V"]), ctypes.c_float(sc), p(O), p(dev["dO"]), p(lse),
                            p(outs[0]), p(outs[1]), p(outs[2]), p(wsb), ctypes.c_size_t(wsb.numel()), st)
    torch.cuda.synchronize()
    assert r == 0 and rb == 0
    assert torch.all(torch.isnan(O7)) and torch.all(torch.isnan(lse7))
    for x in outs:
        assert torch.all(torch.isnan(x))
    _, _, O2, lse2, g2 = gpu_geo(dev, 4, sc, idx=idx)
    assert torch.equal(O2, O) and torch.equal(lse2, lse)
    for a, b in zip(g2, g):
        assert torch.equal(a, b)


# 1301 / 16, 512 / 8 and 2501 / 32 rank through the candidate groups (the last in the
# kernel sized for the most patches); 2501 / 33, 255 / 255 and 3 / 1 count directly
@pytest.mark.parametrize("P_N,P_M,s", [(9, 1301, 16), (5, 512, 8), (4, 2501, 32), (5, 2501, 33), (7, 255, 255),
                                       (6, 3, 1)])
def test_topk_exact_ties_break_to_lower_index(P_N, P_M, s):
    """Every score exact and many tied: small-integer descriptors, target
    patches of exactly 4 rows (means are exact quarters), source patches of
    one row drawn from 40 distinct vectors.  All products and sums are exact
    in fp64, so the order of (score desc, index asc) is the same on both
    sides and the top-s must agree bit for bit, ties included.  P_M covers an
    odd count, several candidates per thread, and the large-P_M kernel."""
    d = 64
    rng = np.random.default_rng(P_M + 7 * s)
    Qf = rng.integers(-4, 5, size=(4 * P_N, d)).astype(np.float32)
    pool = rng.integers(-4, 5, size=(40, d)).astype(np.float32)
    Kf = pool[rng.integers(0, 40, size=P_M)]
    offN = np.arange(0, 4 * P_N + 1, 4, dtype=np.int32)
    offM = np.arange(P_M + 1, dtype=np.int32)
    labN = np.repeat(np.arange(P_N), 4)
    labM = np.arange(P_M)
    Cr = patch_scores(patch_means(Qf, labN, P_N), patch_means(Kf, labM, P_M))
    assert np.array_equal(Cr * 4, np.round(Cr * 4))  # exact quarters
    idxr = topk(Cr, s)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    idx, C = ssc.patch_score_topk(dev(Qf), torch.from_numpy(offN).cuda(), dev(Kf), torch.from_numpy(offM).cuda(), s,
                                  return_scores=True)
    torch.cuda.synchronize()
    n_ties = int(sum(len(np.unique(r)) < P_M for r in Cr))
    say(f"top-s exact ties P_N={P_N} P_M={P_M} s={s}: rows with tied scores {n_ties}")
    np.testing.assert_array_equal(C.cpu().numpy(), Cr)
    np.testing.assert_array_equal(idx.cpu().numpy(), idxr)


@pytest.mark.timeout(900)
def test_geo_workload_160k_full():
    """160k, P = 640, s = 16 against the oracle on every target patch: O,
    lse, dQ, dK and dV of the workload's own upstream gradient, all rows."""
    say("geo 160k full generate")
    c = gen.cached_config(4)
    compare_geo(c, c["s"], "160k full")


def _raw(t):
    import ctypes
    return ctypes.c_void_p(t.data_ptr())


def test_debug_library_reports_invalid_inputs():
    """libssc_debug.so: the device-side verdicts (repeated selection entry,
    offsets out of order) come back as SSC_ERR_INVALID_ARG after kernels that
    all ran to their end; the release library returns OK (NaN outputs for
    the geo call).  Valid inputs give OK and the release library's bits."""
    import ctypes
    from spatial_spectral_coupling_amd import build as ssc_build
    say("debug library verdicts")
    D = ctypes.CDLL(ssc_build.LIB_DEBUG)
    assert D.ssc_debug_build() == 1
    c = gen.make_small(300, 320, 128, 200, "bf16", seed=31, P_N=6, P_M=7, s=3)
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    idx = ssc.patch_score_topk(dev["Q"], dev["offN"], dev["K"], dev["offM"], 3)
    O_ref, lse_ref = ssc.coupling_geo_fwd(dev["Q"], dev["K"], dev["V"], dev["offN"], dev["offM"], idx, 0.1)
    nws = ssc.workspace_bytes(ssc.OP_GEO_FWD, torch.bfloat16, 300, 320, 128, 200, P_N, P_M, 3)

    def geo_fwd_call(L, sel):
        O = torch.empty(300, 200, device="cuda")
        lse = torch.empty(300, device="cuda")
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        r = L.coupling_geo_fwd(1, 128, 200, 300, P_N, _raw(dev["offN"]), 320, P_M, _raw(dev["offM"]), 3, _raw(sel),
                               _raw(dev["Q"]), _raw(dev["K"]), _raw(dev["V"]), ctypes.c_float(0.1), _raw(O),
                               _raw(lse), _raw(ws), ctypes.c_size_t(nws), st)
        torch.cuda.synchronize()
        return r, O, lse

    r, O, lse = geo_fwd_call(D, idx)
    assert r == 0 and torch.equal(O, O_ref) and torch.equal(lse, lse_ref)
    bad = idx.clone()
    bad[2, 1] = bad[2, 0]
    r, O, _ = geo_fwd_call(D, bad)
    assert r == 1 and torch.all(torch.isnan(O))
    r, O, _ = geo_fwd_call(ssc.lib(), bad)
    assert r == 0 and torch.all(torch.isnan(O))
    out_of_range = idx.clone()
    out_of_range[0, 0] = P_M
    assert geo_fwd_call(D, out_of_range)[0] == 1

    # patch scoring with offsets out of order
    offN_bad = dev["offN"].clone()
    offN_bad[2], offN_bad[3] = dev["offN"][3], dev["offN"][2]
    nwt = ssc.workspace_bytes(ssc.OP_PATCH_TOPK, torch.bfloat16, 300, 320, 128, 1, P_N, P_M, 3)
    for L, want in ((D, 1), (ssc.lib(), 0)):
        for offN, w in ((dev["offN"], 0), (offN_bad, want)):
            out = torch.empty(P_N, 3, dtype=torch.int32, device="cuda")
            ws = torch.empty(nwt, dtype=torch.uint8, device="cuda")
            r = L.patch_score_topk(1, 128, 300, P_N, _raw(offN), _raw(dev["Q"]), 320, P_M, _raw(dev["offM"]),
                                   _raw(dev["K"]), 3, _raw(out), None, _raw(ws), ctypes.c_size_t(nwt), st)
            torch.cuda.synchronize()
            assert r == w, (L, r, w)


@pytest.mark.parametrize("dt,k", [("bf16", 200), ("bf16", 256), ("f32", 30)])
def test_geo_backward_without_dv(dt, k):
    """dV = NULL: dQ and dK are the bits of the full call, and match the oracle."""
    say("geo bwd without dV", dt, k)
    c = gen.make_small(700, 650, 64 if dt == "f32" else 128, k, dt, seed=41, P_N=8, P_M=9, s=3)
    dev, permN, permM, P_N, P_M = sorted_problem(c)
    sc = c["scale"]
    idx, _, O, lse, (dQ, dK, dV) = gpu_geo(dev, 3, sc)
    dQ2, dK2, dV2 = ssc.coupling_geo_bwd(dev["Q"], dev["K"], dev["V"], dev["offN"], dev["offM"], idx, O, dev["dO"],
                                         lse, sc, need_dV=False)
    torch.cuda.synchronize()
    assert dV2 is None
    assert torch.equal(dQ2, dQ) and torch.equal(dK2, dK)
    Q, K, V, dO, Cr, idxr = oracle_geo(c, 3)
    gr = geo_bwd(Q, K, V, dO, c["labN"], c["labM"], idx.cpu().numpy(), sc)
    check_grads((unsort(dQ2.cpu().numpy(), permN), unsort(dK2.cpu().numpy(), permM), unsort(dV.cpu().numpy(), permM)),
                gr, "geo no-dV")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_geo_without_target_rows(dt):
    """No target rows (every target patch empty): the forward returns empty
    outputs, and the backward's dK and dV are zero (no source row is in any
    support); the padding jobs of the backward's plan launch shrink to V."""
    say("geo without target rows", dt)
    c = gen.make_small(1, 300, 64, 30, dtype=dt, seed=5)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    K, V = to_dev(c["K"], dt), to_dev(c["V"], dt)
    Q = torch.empty(0, 64, dtype=tdt, device="cuda")
    dO = torch.empty(0, 30, dtype=tdt, device="cuda")
    offN = torch.zeros(3, dtype=torch.int32, device="cuda")          # two empty target patches
    offM = torch.tensor([0, 100, 220, 300], dtype=torch.int32, device="cuda")
    idx = torch.tensor([[0, 2], [1, 0]], dtype=torch.int32, device="cuda")
    O, lse = ssc.coupling_geo_fwd(Q, K, V, offN, offM, idx, 0.125)
    assert O.shape == (0, 30) and lse.shape == (0,)
    dQ, dK, dV = ssc.coupling_geo_bwd(Q, K, V, offN, offM, idx, O, dO, lse, 0.125)
    torch.cuda.synchronize()
    assert dQ.shape == (0, 64)
    assert torch.count_nonzero(dK).item() == 0 and torch.count_nonzero(dV).item() == 0
