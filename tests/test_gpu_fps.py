"""GPU parity of the geodesic farthest-point-sampling partition against the
fp64 oracle, through the C ABI.

Bar: bit-exact.  Seeds and labels are integers decided by exact comparisons
of fp64 path sums; both sides form the same sums (edge lengths rounded the
same way, paths summed from the seed outward), so the distances must agree
bit for bit too.  At 160k vertices (640 seeds) the oracle's per-seed runs
take minutes; there the checks are properties that hold at any size: the
distances equal one multi-source shortest-path run from the GPU's seeds, a
seed sits at distance 0 in its own cell, and every other reachable vertex has
a neighbour in its cell through which its distance is formed.
"""

import numpy as np
import pytest
import torch
from scipy.sparse.csgraph import dijkstra

import gen
import spatial_spectral_coupling_amd as ssc
from oracle import edge_lengths, geodesic_fps
from oracle.fps import edge_graph
from tests._util import say

pytestmark = pytest.mark.gpu


def run_gpu(x, off, adj, P):
    seeds, labels, dist = ssc.fps_partition(torch.from_numpy(np.ascontiguousarray(x, np.float64)).cuda(),
                                            torch.from_numpy(off).cuda(), torch.from_numpy(adj).cuda(), P)
    torch.cuda.synchronize()
    return seeds.cpu().numpy(), labels.cpu().numpy(), dist.cpu().numpy()


def check_exact(x, edges, P, what):
    n = len(x)
    off, adj = gen.mesh_csr(edges, n)
    s, l, d = run_gpu(x, off, adj, P)
    s0, l0, d0 = geodesic_fps(x, edges, P)
    say(f"{what}: seeds equal {np.array_equal(s, s0)}, labels equal {np.array_equal(l, l0)}, "
        f"dist equal {np.array_equal(d, d0)}")
    np.testing.assert_array_equal(s, s0)
    np.testing.assert_array_equal(l, l0)
    np.testing.assert_array_equal(d, d0)


def sphere_mesh(n, seed, amp=0.2):
    rng = np.random.default_rng(seed)
    u = gen.fibonacci_sphere(n)
    return u * (1.0 + amp * rng.random((n, 1))), gen.mesh_edges(gen.hull_mesh(u))


@pytest.mark.parametrize("n,P", [(4, 1), (50, 7), (300, 30), (1000, 257), (5000, 64), (2000, 2000)])
def test_fps_sphere_meshes(n, P):
    x, e = sphere_mesh(n, n + P)
    check_exact(x, e, P, f"sphere n={n} P={P}")


def test_fps_grid_ties():
    # a unit grid: integer distances, many exact ties for the argmax and the
    # nearest seed
    m = 33
    ii, jj = np.meshgrid(np.arange(m), np.arange(m), indexing="ij")
    x = np.stack([ii.ravel(), jj.ravel(), np.zeros(m * m)], axis=1).astype(float)
    idx = lambda i, j: i * m + j
    e = [(idx(i, j), idx(i + 1, j)) for i in range(m - 1) for j in range(m)]
    e += [(idx(i, j), idx(i, j + 1)) for i in range(m) for j in range(m - 1)]
    check_exact(x, np.array(e), 40, "grid 33x33 P=40")


def test_fps_wide_vertices_and_long_queues():
    # A hub joined to 10000 rim vertices (a ring): the hub has more
    # neighbours than the padded adjacency holds, so the CSR rows are used,
    # and the first round queues more vertices than the LDS part of the
    # queue takes.
    m = 10000
    t = np.linspace(0.0, 2.0 * np.pi, m, endpoint=False)
    rng = np.random.default_rng(11)
    rim = np.c_[np.cos(t), np.sin(t), 0.1 * rng.random(m)] * (1.0 + 0.05 * rng.random((m, 1)))
    x = np.vstack([np.zeros((1, 3)), rim])
    e = [(0, i) for i in range(1, m + 1)] + [(i, i % m + 1) for i in range(1, m + 1)]
    check_exact(x, np.array(e), 6, f"hub + ring of {m}, P=6")
    # a grid with diagonals: interior vertices have exactly 8 neighbours
    k = 40
    ii, jj = np.meshgrid(np.arange(k), np.arange(k), indexing="ij")
    xg = np.stack([ii.ravel(), jj.ravel(), 0.01 * (ii * jj).ravel() % 1.0], axis=1).astype(float)
    idx = lambda i, j: i * k + j
    eg = [(idx(i, j), idx(i + 1, j)) for i in range(k - 1) for j in range(k)]
    eg += [(idx(i, j), idx(i, j + 1)) for i in range(k) for j in range(k - 1)]
    eg += [(idx(i, j), idx(i + 1, j + 1)) for i in range(k - 1) for j in range(k - 1)]
    eg += [(idx(i, j + 1), idx(i + 1, j)) for i in range(k - 1) for j in range(k - 1)]
    check_exact(xg, np.array(eg), 50, f"grid {k}x{k} with diagonals, P=50")


def test_fps_large_mesh_global_stamps():
    # more vertices than the LDS bitmaps of queued vertices cover (2^18):
    # the per-vertex round stamps in the workspace take over
    x, e = sphere_mesh(270000, 5)
    check_exact(x, e, 3, "sphere n=270000 P=3")


@pytest.mark.parametrize("env", [{"SSC_FPS_WIDE_STEPS": "0"}, {}, {"SSC_FPS_WIDE_STEPS": "1"},
                                 {"SSC_FPS_WIDE_FRONTIER": "0"}, {"SSC_FPS_SPIN_LIMIT": "0"},
                                 {"SSC_FPS_WIDE_BLOCKS": "1", "SSC_FPS_WIDE_FRONTIER": "0"}],
                         ids=["off", "default", "one-step", "every-step", "barrier-gives-up", "one-block"])
def test_fps_multi_workgroup_steps(monkeypatch, env):
    # Meshes from 32768 vertices run their first steps on many workgroups
    # (until a step's largest round queue stays small).  With those steps
    # off, on (the default), limited to step 0, on for every step, with every
    # grid-barrier wait giving up at once (the one-workgroup kernel then
    # redoes every step from the initial state), and on a grid of one
    # workgroup, the results must equal the oracle's bit for bit.
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    x, e = sphere_mesh(40000, 9)
    check_exact(x, e, 12, f"sphere n=40000 P=12 {env}")


def test_fps_multi_workgroup_small_and_irregular(monkeypatch):
    # every step on many workgroups for small meshes, a mesh of several
    # components (unreached vertices stay at +inf until a seed lands there)
    # and a mesh whose hub exceeds the padded adjacency (the one-workgroup
    # kernel then takes every step)
    monkeypatch.setenv("SSC_FPS_WIDE_STEPS", "1000")
    monkeypatch.setenv("SSC_FPS_WIDE_FRONTIER", "0")
    x, e = sphere_mesh(300, 4)
    check_exact(x, e, 30, "sphere n=300 P=30, all steps wide")
    x1 = np.c_[np.arange(5.0), np.zeros(5), np.zeros(5)]
    x2 = np.c_[np.arange(4.0), np.full(4, 10.0), np.zeros(4)]
    x3 = np.c_[np.arange(3.0), np.full(3, 20.0), np.zeros(3)]
    e3 = np.array([[0, 1], [1, 2], [2, 3], [3, 4], [5, 6], [6, 7], [7, 8], [9, 10], [10, 11]])
    for P in (1, 2, 3, 5):
        check_exact(np.vstack([x1, x2, x3]), e3, P, f"three components P={P}, all steps wide")
    m = 2000
    t = np.linspace(0.0, 2.0 * np.pi, m, endpoint=False)
    rim = np.c_[np.cos(t), np.sin(t), np.zeros(m)]
    xh = np.vstack([np.zeros((1, 3)), rim])
    eh = [(0, i) for i in range(1, m + 1)] + [(i, i % m + 1) for i in range(1, m + 1)]
    check_exact(xh, np.array(eh), 5, f"hub + ring of {m}, P=5, wide steps requested")


def test_fps_disconnected_and_single_vertex():
    # three components; with 2 seeds the third stays at +inf with label 0
    x1 = np.c_[np.arange(5.0), np.zeros(5), np.zeros(5)]
    x2 = np.c_[np.arange(4.0), np.full(4, 10.0), np.zeros(4)]
    x3 = np.c_[np.arange(3.0), np.full(3, 20.0), np.zeros(3)]
    x = np.vstack([x1, x2, x3])
    e = np.array([[0, 1], [1, 2], [2, 3], [3, 4], [5, 6], [6, 7], [7, 8], [9, 10], [10, 11]])
    for P in (1, 2, 3, 5):
        check_exact(x, e, P, f"three components P={P}")
    # one vertex, no edges
    s, l, d = run_gpu(np.zeros((1, 3)), np.zeros(2, np.int32), np.zeros(0, np.int32), 1)
    assert s.tolist() == [0] and l.tolist() == [0] and d.tolist() == [0.0]


def test_fps_60k_full_oracle():
    c = gen.make_config(3, with_partition=False)
    x, e = c["xM"], c["edges"]
    say(f"60k mesh: n={len(x)} edges={len(e)}")
    check_exact(x, e, 256, "60k P=256")


def test_fps_160k_properties(monkeypatch):
    c = gen.make_config(4, with_partition=False)
    x, e, n = c["xM"], c["edges"], len(c["xM"])
    say(f"160k mesh: n={n} edges={len(e)}")
    off, adj = gen.mesh_csr(e, n)
    s, l, d = run_gpu(x, off, adj, 640)
    assert len(np.unique(s)) == 640 and s.min() >= 0
    g = edge_graph(x, e)
    dm = dijkstra(g, directed=True, indices=s, min_only=True)
    say(f"160k: dist equal to the multi-source run {np.array_equal(d, dm)}")
    np.testing.assert_array_equal(d, dm)
    np.testing.assert_array_equal(l[s], np.arange(640))
    assert (d[s] == 0).all()
    # every non-seed vertex: a neighbour u in the same cell with d[v] = d[u] + w
    src = np.r_[e[:, 0], e[:, 1]]
    dst = np.r_[e[:, 1], e[:, 0]]
    w = np.r_[edge_lengths(x, e), edge_lengths(x, e)]
    ok = (l[src] == l[dst]) & (d[src] + w == d[dst])
    has = np.zeros(n, bool)
    has[dst[ok]] = True
    has[s] = True
    assert has.all(), int((~has).sum())
    # the sampling order at a few steps: seed t is the vertex farthest from
    # seeds 0 .. t-1 (multi-source runs form the same bits, as above), ties
    # to the lower index
    for t in (1, 2, 5, 17, 100, 639):
        dt = dijkstra(g, directed=True, indices=s[:t], min_only=True)
        assert s[t] == int(np.argmax(dt)), t
    # the first steps run on many workgroups by default: the one-workgroup
    # path gives the same bits
    monkeypatch.setenv("SSC_FPS_WIDE_STEPS", "0")
    s1, l1, d1 = run_gpu(x, off, adj, 640)
    say(f"160k: one-workgroup path equal {np.array_equal(s1, s) and np.array_equal(l1, l) and np.array_equal(d1, d)}")
    np.testing.assert_array_equal(s1, s)
    np.testing.assert_array_equal(l1, l)
    np.testing.assert_array_equal(d1, d)


def test_fps_invalid_inputs():
    x, e = sphere_mesh(100, 1)
    off, adj = gen.mesh_csr(e, 100)
    with pytest.raises(ssc.CouplingError):  # P > n
        run_gpu(x, off, adj, 101)
    bad = adj.copy()
    bad[17] = 100  # neighbour out of range: nothing computed
    s, l, d = run_gpu(x, off, bad, 10)
    assert (s == -1).all() and (l == -1).all() and np.isnan(d).all()
    bad_off = off.copy()
    bad_off[50] = bad_off[51] + 1  # offsets out of order
    s, l, d = run_gpu(x, bad_off, adj, 10)
    assert (s == -1).all() and (l == -1).all() and np.isnan(d).all()
    # a valid call afterwards on the same process still works
    check_exact(x, e, 10, "after invalid inputs")
