"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/ssc.h declares, and
reject bad arguments with the documented status before any HIP call.  Every
call below fails validation, so nothing reaches the device.
"""

import ctypes
import os
import re

import pytest

import spatial_spectral_coupling_amd as ssc
from spatial_spectral_coupling_amd import build as ssc_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssc.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ssc.library_path):
        ssc_build.build()
    return ssc.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("coupling_dense_fwd", "coupling_dense_bwd", "patch_score_topk", "coupling_geo_fwd",
              "coupling_geo_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_queries(L):
    for code, text in ((OK, b"ok"), (INVALID, b"invalid argument"), (UNSUPPORTED, b"unsupported shape"),
                       (WORKSPACE, b"workspace too small"), (HIPERR, b"HIP launch failed")):
        assert L.ssc_status_string(code) == text
    assert [L.ssc_query(0, k) for k in (1, 30, 32, 33, 100, 200, 224, 225, 256, 257, 0)] == \
        [32, 32, 32, 64, 128, 224, 224, 256, 256, 0, 0]
    assert L.ssc_query(1, 0) == 16
    assert L.ssc_last_hip_error() == 0


def test_workspace_sizes(L):
    w = L.ssc_workspace_bytes
    assert w(ssc.OP_DENSE_FWD, BF16, 60000, 60000, 128, 200, 0, 0, 0) >= 60000 * 224 * 2
    assert w(ssc.OP_DENSE_BWD, BF16, 60000, 60000, 128, 200, 0, 0, 0) > w(ssc.OP_DENSE_FWD, BF16, 60000, 60000,
                                                                          128, 200, 0, 0, 0)
    assert w(ssc.OP_GEO_BWD, BF16, 60000, 60000, 128, 200, 256, 256, 16) > 0
    assert w(ssc.OP_PATCH_TOPK, BF16, 60000, 60000, 128, 0, 256, 256, 16) >= 2 * 256 * 128 * 8
    assert w(ssc.OP_DENSE_FWD, BF16, 10, 10, 96, 200, 0, 0, 0) == 0      # d unsupported
    assert w(ssc.OP_DENSE_FWD, BF16, 10, 10, 128, 300, 0, 0, 0) == 0     # k unsupported
    assert w(ssc.OP_GEO_FWD, BF16, 10, 10, 128, 200, 4, 4, 5) == 0       # s > P_M
    assert w(ssc.OP_DENSE_FWD, F32, 10, 10, 128, 256, 0, 0, 0) == 0      # fp32 compiled up to k = 128


def P(x):
    return ctypes.c_void_p(x)


# distinct, 16-byte aligned fake device addresses far apart (never dereferenced)
A = [P(0x100000 * (i + 1)) for i in range(12)]


def dense_fwd(L, dtype=BF16, nN=64, nM=64, d=128, k=200, Q=None, K=None, V=None, O=None, lse=None,
              ws=None, wsb=1 << 30):
    pick = lambda x, default: default if x is None else x
    return L.coupling_dense_fwd(dtype, nN, nM, d, k, pick(Q, A[0]), pick(K, A[1]), pick(V, A[2]), 0.1,
                                pick(O, A[3]), pick(lse, A[4]), ws, wsb, None)


def test_dense_fwd_validation(L):
    assert dense_fwd(L, d=96) == UNSUPPORTED
    assert dense_fwd(L, k=257) == UNSUPPORTED
    assert dense_fwd(L, nM=0) == INVALID
    assert dense_fwd(L, nN=-1) == INVALID
    assert dense_fwd(L, dtype=7) == INVALID
    assert dense_fwd(L, nN=0) == OK                         # nothing to do, nothing launched
    assert dense_fwd(L, Q=P(0)) == INVALID                  # null pointer
    assert dense_fwd(L, K=P(0x100008)) == INVALID           # misaligned
    assert dense_fwd(L, ws=None) == WORKSPACE               # no workspace
    assert dense_fwd(L, ws=A[5], wsb=16) == WORKSPACE       # too small
    assert dense_fwd(L, O=A[0], ws=A[5]) == INVALID         # output aliases an input
    assert dense_fwd(L, lse=A[3], ws=A[5]) == INVALID       # two outputs overlap


def test_dense_route_mode_and_workspace(L):
    """The thread's dense route (by size / dense kernels / one-patch geo):
    the setter returns the previous mode and ignores other values; the dense
    workspace covers the one-patch route (its offsets plus a one-patch geo
    workspace); a routed call checks every argument before any launch."""
    assert L.ssc_dense_split(0) == -1
    assert L.ssc_dense_split(7) == 0
    assert L.ssc_dense_split(1) == 0
    assert L.ssc_dense_split(-1) == 1
    w = L.ssc_workspace_bytes
    for op, gop in ((ssc.OP_DENSE_FWD, ssc.OP_GEO_FWD), (ssc.OP_DENSE_BWD, ssc.OP_GEO_BWD)):
        for n in (5000, 60000):
            assert w(op, BF16, n, n, 128, 200, 0, 0, 0) >= 256 + w(gop, BF16, n, n, 128, 200, 1, 1, 1)
    assert dense_fwd(L, ws=A[5], wsb=300) == WORKSPACE
    assert dense_fwd(L, K=A[3], ws=A[5]) == INVALID             # output O aliases K: nothing launched


def test_dense_bwd_validation(L):
    f = L.coupling_dense_bwd
    args = lambda **kw: [kw.get("dt", BF16), kw.get("nN", 64), kw.get("nM", 64), kw.get("d", 128), kw.get("k", 200),
                         A[0], A[1], A[2], 0.1, A[3], A[4], A[5], kw.get("dQ", A[6]), A[7], A[8],
                         kw.get("ws", None), kw.get("wsb", 0), None]
    assert f(*args(d=100)) == UNSUPPORTED
    assert f(*args(nM=0)) == INVALID
    assert f(*args()) == WORKSPACE
    assert f(*args(dQ=A[0], ws=A[9], wsb=1 << 40)) == INVALID   # dQ aliases Q
    # no target rows: Q, O, dO, lse and dQ may be NULL (only the workspace check remains)
    assert f(BF16, 0, 64, 128, 200, None, A[1], A[2], 0.1, None, None, None, None, A[7], A[8], None, 0,
             None) == WORKSPACE
    assert f(BF16, 64, 64, 128, 200, None, A[1], A[2], 0.1, A[3], A[4], A[5], A[6], A[7], A[8], None, 0,
             None) == INVALID                                   # with rows, Q is required


def test_patch_topk_validation(L):
    f = L.patch_score_topk
    base = dict(dt=BF16, d=128, nN=100, PN=4, nM=100, PM=4, s=2, ws=A[9], wsb=1 << 30)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["dt"], a["d"], a["nN"], a["PN"], A[0], A[1], a["nM"], a["PM"], A[2], A[3], a["s"], A[4],
                 None, a["ws"], a["wsb"], None)

    assert call(s=5) == INVALID
    assert call(s=0) == INVALID
    assert call(PN=0) == INVALID
    assert call(PM=9000, s=2) == UNSUPPORTED
    assert call(d=96) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE


def test_geo_validation(L):
    f = L.coupling_geo_fwd

    def call(s=2, PM=4, d=128, ws=None, wsb=0):
        return f(BF16, d, 200, 100, 4, A[0], 100, PM, A[1], s, A[2], A[3], A[4], A[5], 0.1, A[6], A[7], ws, wsb,
                 None)

    assert call(s=0) == INVALID
    assert call(s=5) == INVALID
    assert call(d=32) == UNSUPPORTED
    assert call() == WORKSPACE
    g = L.coupling_geo_bwd
    assert g(BF16, 128, 200, 100, 4, A[0], 100, 4, A[1], 2, A[2], A[3], A[4], A[5], 0.1, A[6], A[7], A[8],
             A[9], A[10], A[11], None, 0, None) == WORKSPACE
    # no target rows: Q, O, dO, lse and dQ may be NULL
    assert g(BF16, 128, 200, 0, 4, A[0], 100, 4, A[1], 2, A[2], None, A[4], A[5], 0.1, None, None, None,
             None, A[10], A[11], None, 0, None) == WORKSPACE
    assert g(BF16, 128, 200, 100, 4, A[0], 100, 4, A[1], 2, A[2], None, A[4], A[5], 0.1, A[6], A[7], A[8],
             A[9], A[10], A[11], None, 0, None) == INVALID


def test_linear_validation_and_workspace(L):
    w = L.ssc_workspace_bytes
    assert w(ssc.OP_LINEAR_FWD, BF16, 60000, 60000, 128, 200, 0, 0, 0) >= 128 * 224 * 2 * 2
    assert w(ssc.OP_LINEAR_BWD, BF16, 60000, 60000, 128, 200, 0, 0, 0) > w(ssc.OP_LINEAR_FWD, BF16, 60000,
                                                                           60000, 128, 200, 0, 0, 0)
    assert w(ssc.OP_LINEAR_FWD, BF16, 10, 10, 128, 256, 0, 0, 0) == 0   # no column left for the normaliser
    assert w(ssc.OP_LINEAR_FWD, F32, 10, 10, 128, 64, 0, 0, 0) == 0     # bf16 only
    f = L.coupling_linear_fwd
    args = lambda **kw: [kw.get("dt", BF16), kw.get("nN", 64), kw.get("nM", 64), kw.get("d", 128), kw.get("k", 200),
                         kw.get("Q", A[0]), A[1], A[2], kw.get("O", A[3]), A[4], kw.get("ws", None),
                         kw.get("wsb", 0), None]
    assert f(*args(k=256)) == UNSUPPORTED
    assert f(*args(dt=F32)) == UNSUPPORTED
    assert f(*args(d=96)) == UNSUPPORTED
    assert f(*args(nM=0)) == INVALID
    assert f(*args(nN=0)) == OK
    assert f(*args(Q=P(0))) == INVALID
    assert f(*args()) == WORKSPACE
    assert f(*args(O=A[1], ws=A[9], wsb=1 << 40)) == INVALID     # O aliases K
    g = L.coupling_linear_bwd
    bargs = lambda **kw: [BF16, 64, 64, 128, 200, A[0], A[1], A[2], A[3], A[4], A[5], kw.get("dQ", A[6]), A[7],
                          A[8], kw.get("ws", None), kw.get("wsb", 0), None]
    # no target rows: Q, O, dO, den and dQ may be NULL (dK = dV = 0 are still written)
    assert g(BF16, 0, 64, 128, 200, None, A[1], A[2], None, None, None, None, A[7], A[8], None, 0, None) == WORKSPACE
    assert g(BF16, 64, 64, 128, 200, None, A[1], A[2], A[3], A[4], A[5], A[6], A[7], A[8], None, 0,
             None) == INVALID
    assert g(*bargs()) == WORKSPACE
    assert g(*bargs(dQ=A[4], ws=A[9], wsb=1 << 40)) == INVALID   # dQ aliases dO


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ssc, "_lib", None)
    monkeypatch.setattr(ssc, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ssc.lib()


def test_fmap_and_fps_workspace_sizes(L):
    w = L.ssc_workspace_bytes
    f = w(ssc.OP_FMAP_FWD, BF16, 60000, 0, 0, 200, 0, 0, 0)
    b = w(ssc.OP_FMAP_BWD, BF16, 60000, 0, 0, 200, 0, 0, 0)
    assert f >= 2 * 224 * 224 * 4 and b >= 224 * 224 * 2
    assert w(ssc.OP_FMAP_FWD, F32, 60000, 0, 0, 200, 0, 0, 0) == 0       # bf16 basis only
    assert w(ssc.OP_FMAP_FWD, BF16, 60000, 0, 0, 257, 0, 0, 0) == 0      # k > 256
    assert w(ssc.OP_FMAP_BWD, BF16, 0, 0, 0, 16, 0, 0, 0) == 0           # n < 1
    n, nnz = 160000, 960000
    assert w(ssc.OP_FPS, 0, n, nnz, 0, 0, 640, 0, 0) >= nnz * 8 + n * 12
    assert w(ssc.OP_FPS, 0, n, nnz, 0, 0, n + 1, 0, 0) == 0              # P > n
    assert w(ssc.OP_FPS, 0, n, nnz, 0, 0, 0, 0, 0) == 0                  # P < 1
    assert w(ssc.OP_FPS, 0, 0, 0, 0, 0, 1, 0, 0) == 0                    # no vertex


def test_fmap_validation(L):
    ws = A[5]
    call = lambda dt=BF16, n=100, k=16, Phi=A[0], O=A[1], C=A[2], wsb=1 << 30: \
        L.fmap_solve_fwd(dt, n, k, Phi, O, C, ws, wsb, None)
    assert call(dt=F32) == UNSUPPORTED
    assert call(k=257) == UNSUPPORTED
    assert call(k=0) == INVALID
    assert call(n=0) == INVALID
    assert call(Phi=None) == INVALID
    assert call(C=P(0x100000 + 8)) == INVALID                        # misaligned
    assert call(wsb=16) == WORKSPACE
    assert call(C=A[0]) == INVALID                                   # output aliases the basis
    bwd = lambda dt=BF16, n=100, k=16, dO=A[2], wsb=1 << 30: L.fmap_solve_bwd(dt, n, k, A[0], A[1], dO, ws, wsb,
                                                                              None)
    assert bwd(dt=F32) == UNSUPPORTED
    assert bwd(wsb=16) == WORKSPACE
    assert bwd(dO=A[1]) == INVALID                                   # output aliases dC


def test_fps_validation(L):
    def call(n=100, nnz=600, x=A[0], off=A[1], adj=A[2], Pn=10, seeds=A[3], labels=A[4], dist=A[5], ws=A[6],
             wsb=1 << 30):
        return L.fps_partition(n, nnz, x, off, adj, Pn, seeds, labels, dist, ws, wsb, None)
    assert call(Pn=0) == INVALID
    assert call(Pn=101) == INVALID
    assert call(n=0) == INVALID
    assert call(nnz=-1) == INVALID
    assert call(adj=None) == INVALID                                 # nnz > 0 needs neighbours
    assert call(x=None) == INVALID
    assert call(wsb=64) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(dist=A[0]) == INVALID                                # output aliases the positions
    assert call(labels=A[3]) == INVALID                              # two outputs alias


def test_performer_validation(L):
    w = L.ssc_workspace_bytes
    assert w(ssc.OP_PERFORMER_BWD, BF16, 60000, 60000, 128, 200, 0, 0, 0) > \
        w(ssc.OP_PERFORMER_FWD, BF16, 60000, 60000, 128, 200, 0, 0, 0) > 60000 * 128 * 4
    assert w(ssc.OP_PERFORMER_FWD, BF16, 10, 10, 96, 200, 0, 0, 0) == 0     # d unsupported
    assert w(ssc.OP_PERFORMER_FWD, BF16, 10, 10, 128, 256, 0, 0, 0) == 0    # no normaliser column
    # the feature count m rides in P_N (0 = d): fewer features, less workspace
    assert w(ssc.OP_PERFORMER_FWD, BF16, 1000, 1000, 128, 200, 128, 0, 0) == \
        w(ssc.OP_PERFORMER_FWD, BF16, 1000, 1000, 128, 200, 0, 0, 0)
    assert 0 < w(ssc.OP_PERFORMER_BWD, BF16, 1000, 1000, 128, 200, 64, 0, 0) < \
        w(ssc.OP_PERFORMER_BWD, BF16, 1000, 1000, 128, 200, 128, 0, 0)
    assert w(ssc.OP_PERFORMER_FWD, BF16, 1000, 1000, 64, 200, 128, 0, 0) > 0  # m > d
    assert w(ssc.OP_PERFORMER_FWD, BF16, 10, 10, 128, 200, 96, 0, 0) == 0     # m unsupported
    ws = A[8]

    def fwd(dt=BF16, nN=64, nM=64, d=128, k=200, m=128, scale=0.1, O=A[4], lnden=A[5], wsb=1 << 30):
        return L.coupling_performer_fwd(dt, nN, nM, d, k, m, A[0], A[1], A[2], A[3], scale, O, lnden, ws, wsb, None)
    assert fwd(dt=F32) == UNSUPPORTED
    assert fwd(d=96) == UNSUPPORTED
    assert fwd(m=96) == UNSUPPORTED
    assert fwd(m=256) == UNSUPPORTED
    assert fwd(m=0) == INVALID
    assert fwd(nM=0) == INVALID
    assert fwd(scale=0.0) == INVALID
    assert fwd(scale=-1.0) == INVALID
    assert fwd(wsb=64) == WORKSPACE
    assert fwd(O=A[3]) == INVALID                                   # output aliases W
    assert fwd(nN=0) == OK                                          # nothing to do

    def bwd(dQ=A[6], wsb=1 << 30):
        return L.coupling_performer_bwd(BF16, 64, 64, 128, 200, 128, A[0], A[1], A[2], A[3], 0.1, A[4], A[9], A[5],
                                        dQ, A[7], A[10], ws, wsb, None)
    assert bwd(wsb=64) == WORKSPACE
    assert bwd(dQ=A[0]) == INVALID                                  # gradient aliases Q


def test_row_count_limit(L):
    # the couplings address rows with 32-bit byte offsets: at most 2^22 rows a side
    big = (1 << 22) + 1
    assert dense_fwd(L, nN=big) == UNSUPPORTED
    assert dense_fwd(L, nM=big) == UNSUPPORTED
    assert L.ssc_workspace_bytes(ssc.OP_DENSE_BWD, BF16, big, 64, 128, 200, 0, 0, 0) == 0
    assert L.ssc_workspace_bytes(ssc.OP_LINEAR_FWD, BF16, 64, big, 128, 200, 0, 0, 0) == 0
    assert L.ssc_workspace_bytes(ssc.OP_DENSE_FWD, BF16, 1 << 22, 1 << 22, 128, 200, 0, 0, 0) > 0


def test_debug_library_exports_every_declared_symbol(L):
    # the debug build (SSC_DEBUG) is the same ABI with host-side verdict reads
    if not os.path.exists(ssc_build.LIB_DEBUG):
        ssc_build.build()
    D = ctypes.CDLL(ssc_build.LIB_DEBUG)
    for name in declared_functions():
        assert hasattr(D, name), name
    assert D.ssc_debug_build() == 1
    assert L.ssc_debug_build() == 0


def test_noalloc_patch_scoring_rejects_patch_counts_past_its_scratch(L):
    # the allocation-free patch scoring holds the patch means in a fixed
    # device array: more than 2048 patches a side is refused before any HIP call
    assert L.patch_score_topk_noalloc(BF16, 128, 10, 2049, None, None, 10, 3, None, None, 1, None, None,
                                      None) == WORKSPACE
    assert L.patch_score_topk_noalloc(BF16, 128, 10, 3, None, None, 10, 2049, None, None, 1, None, None,
                                      None) == WORKSPACE
    assert L.patch_score_topk_noalloc(BF16, 96, 10, 3, None, None, 10, 3, None, None, 1, None, None,
                                      None) == UNSUPPORTED
