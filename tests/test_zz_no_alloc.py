"""The allocation-free patch scoring (patch_score_topk_noalloc, for callers
that cannot allocate) against the workspace entry point patch_score_topk:
top-s indices and fp64 scores bit-equal, on two calls in a row, the second
with smaller inputs (the shared scratch keeps the first call's contents)."""

import ctypes

import pytest
import torch

import gen
import spatial_spectral_coupling_amd as ssc
from tests._util import say, sorted_problem

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(dev, P_N, P_M, s):
    n_N, d = dev["Q"].shape
    n_M = dev["K"].shape[0]
    idx = torch.full((P_N, s), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((P_N, P_M), float("nan"), dtype=torch.float64, device="cuda")
    st = ssc.lib().patch_score_topk_noalloc(1, d, n_N, P_N, _p(dev["offN"]), _p(dev["Q"]), n_M, P_M,
                                            _p(dev["offM"]), _p(dev["K"]), s, _p(idx), _p(sc),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, st
    return idx, sc


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    # second call smaller in rows, patch counts and s
    for nN, nM, PN, PM, s, seed in ((6000, 6400, 300, 310, 16, 1), (900, 1000, 40, 37, 5, 2)):
        say("no-alloc patch scoring", nN, nM, PN, PM, s)
        c = gen.make_small(nN, nM, 128, 200, "bf16", seed=seed, P_N=PN, P_M=PM, s=s)
        dev = sorted_problem(c)[0]
        idx_ref, sc_ref = ssc.patch_score_topk(dev["Q"], dev["offN"], dev["K"], dev["offM"], s,
                                               return_scores=True)
        idx, sc = _noalloc(dev, PN, PM, s)
        assert torch.equal(idx, idx_ref)
        assert torch.equal(sc, sc_ref)


def test_noalloc_without_scores_at_the_patch_limit():
    # 2048 source patches (the scratch limit), most of them empty
    import numpy as np
    rng = np.random.default_rng(3)
    c = gen.make_small(500, 520, 64, 30, "bf16", seed=3)
    Q = torch.from_numpy(c["Q"].view(np.int16)).view(torch.bfloat16).cuda()
    K = torch.from_numpy(c["K"].view(np.int16)).view(torch.bfloat16).cuda()
    offN = torch.tensor(np.r_[0, np.sort(rng.integers(0, 500, 19)), 500], dtype=torch.int32, device="cuda")
    offM = torch.tensor(np.r_[0, np.sort(rng.integers(0, 520, 2047)), 520], dtype=torch.int32, device="cuda")
    idx_ref = ssc.patch_score_topk(Q, offN, K, offM, 4)
    idx = torch.full((20, 4), -1, dtype=torch.int32, device="cuda")
    st = ssc.lib().patch_score_topk_noalloc(1, 64, 500, 20, _p(offN), _p(Q), 520, 2048, _p(offM), _p(K), 4,
                                            _p(idx), None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(idx, idx_ref)
