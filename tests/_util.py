"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import gen
from oracle import upcast

# Parity bars: forward max-abs <= 2e-2 and rel-Frobenius <= 5e-3, gradients
# rel-Frobenius <= 1e-2, top-s indices bit-exact (ties to the lower index).
FWD_MAX_ABS = 2e-2
FWD_REL_F = 5e-3
GRAD_REL_F = 1e-2
LSE_MAX_ABS = 1e-2


def say(*args):
    """Progress line, flushed, so a GPU run that dies still names its case."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored array (bf16 bits as uint16, or fp32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to(device).contiguous()


def f64(a, dtype):
    return upcast(a, dtype)


def rel_f(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def check_fwd(O, O_ref, lse=None, lse_ref=None, what=""):
    O = np.asarray(O, np.float64)
    err = float(np.max(np.abs(O - O_ref))) if O.size else 0.0
    rf = rel_f(O, O_ref)
    say(f"{what} O max-abs {err:.3e} rel-F {rf:.3e}")
    assert np.all(np.isfinite(O)), what
    assert err <= FWD_MAX_ABS, (what, err)
    assert rf <= FWD_REL_F, (what, rf)
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin), what
        if fin.any():
            e = float(np.max(np.abs(lse[fin] - lse_ref[fin])))
            say(f"{what} lse max-abs {e:.3e}")
            assert e <= LSE_MAX_ABS, (what, e)


def check_grads(got, ref, what=""):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = np.asarray(g, np.float64)
        assert np.all(np.isfinite(g)), (what, name)
        rf = rel_f(g, r)
        say(f"{what} {name} rel-F {rf:.3e}")
        assert rf <= GRAD_REL_F, (what, name, rf)


def sorted_problem(c: dict):
    """Patch-sorted device copies of a geo instance plus the permutations."""
    dtype = c["dtype"]
    P_N = c.get("P_N", c.get("P"))
    P_M = c.get("P_M", c.get("P"))
    permN, offN = gen.patch_sort(c["labN"], P_N)
    permM, offM = gen.patch_sort(c["labM"], P_M)
    dev = dict(
        Q=to_dev(c["Q"][permN], dtype), K=to_dev(c["K"][permM], dtype),
        V=to_dev(c["V"][permM], dtype), dO=to_dev(c["dO"][permN], dtype),
        offN=torch.from_numpy(offN).to("cuda"), offM=torch.from_numpy(offM).to("cuda"))
    return dev, permN, permM, P_N, P_M


def unsort(x_sorted: np.ndarray, perm: np.ndarray) -> np.ndarray:
    out = np.empty_like(x_sorted)
    out[perm] = x_sorted
    return out


def check_idx(idx_gpu: np.ndarray, idx_ref: np.ndarray, C_ref: np.ndarray, s: int, what=""):
    """Bit-exact top-s; rows whose s-th / (s+1)-th scores are within rounding
    of each other (near-ties) must still be a valid top-s set."""
    P_N, P_M = C_ref.shape
    srt = -np.sort(-C_ref, axis=1)
    scale = np.max(np.abs(C_ref)) if C_ref.size else 1.0
    tol = 1e-12 * max(scale, 1e-300)
    near = np.zeros(P_N, bool)
    if s < P_M:
        near = (srt[:, s - 1] - srt[:, s]) <= tol
    mism = np.nonzero(np.any(idx_gpu != idx_ref, axis=1))[0]
    say(f"{what} idx rows differing {len(mism)} (near-tie rows {int(near.sum())})")
    for p in mism:
        assert near[p], (what, "top-s mismatch on a row without a near-tie", p)
        sel = C_ref[p, idx_gpu[p]]
        assert len(set(idx_gpu[p].tolist())) == s
        assert np.all(sel >= srt[p, s - 1] - tol)
