"""Pins of the fp64 geodesic FPS partition (oracle.fps) against facts fixed by
the mathematics and by brute force: a straight path (distances are coordinate
differences, exact for integer coordinates), a unit grid (Manhattan
distances), Floyd-Warshall plus the sampling rule written as a plain loop on
tiny meshes, disconnected components, and the tie rules."""

import itertools

import numpy as np
import pytest

import gen
from oracle import edge_lengths, geodesic_fps


def path_graph(n):
    x = np.zeros((n, 3))
    x[:, 0] = np.arange(n)
    e = np.stack([np.arange(n - 1), np.arange(1, n)], axis=1)
    return x, e


def test_path_graph_closed_form():
    n = 11
    x, e = path_graph(n)
    seeds, labels, dist = geodesic_fps(x, e, 3)
    # from vertex 0 the farthest is the other end; then the midpoint 5 (4 and
    # 6 are not tied with it: both ends are seeds, 5 is at distance 5)
    assert seeds.tolist() == [0, 10, 5]
    # nearest seed, ties to the earlier seed: vertex 2.5 does not exist, but
    # 7 and 8 are 2 and 3 from seed 5 / 10: labels by plain comparison
    want_d = np.array([min(abs(i - 0), abs(i - 10), abs(i - 5)) for i in range(n)], float)
    np.testing.assert_array_equal(dist, want_d)
    lab = [int(np.argmin([abs(i - s) for s in (0, 10, 5)])) for i in range(n)]
    assert labels.tolist() == lab


def test_path_graph_tie_to_lower_index():
    # even length: from seeds {0, 9} the vertices 4 and 5 are both at 4 ->
    # the next seed is 4 (lower index)
    x, e = path_graph(10)
    seeds, labels, _ = geodesic_fps(x, e, 3)
    assert seeds.tolist() == [0, 9, 4]
    # vertex 2 is 2 from seed 0 and 2 from seed 4: keeps the earlier seed 0
    assert labels[2] == 0
    # vertex 7: 2 from seed 9, 3 from seed 4 -> seed 1 (vertex 9)
    assert labels[7] == 1


def test_unit_grid_manhattan():
    m = 7
    ii, jj = np.meshgrid(np.arange(m), np.arange(m), indexing="ij")
    x = np.stack([ii.ravel(), jj.ravel(), np.zeros(m * m)], axis=1).astype(float)
    idx = lambda i, j: i * m + j
    e = [(idx(i, j), idx(i + 1, j)) for i in range(m - 1) for j in range(m)]
    e += [(idx(i, j), idx(i, j + 1)) for i in range(m) for j in range(m - 1)]
    e = np.array(e)
    seeds, labels, dist = geodesic_fps(x, e, 4)
    # corner (0,0) -> opposite corner (6,6) at 12 -> the anti-diagonal i + j
    # = 6 is all at 6, lowest index (0,6) -> then the points at 6 from all
    # three seeds are (3,3), (4,2), (5,1), (6,0): the lowest index is (3,3)
    assert seeds.tolist() == [0, idx(6, 6), idx(0, 6), idx(3, 3)]
    S = [(0, 0), (6, 6), (0, 6), (3, 3)]
    for i in range(m):
        for j in range(m):
            dd = [abs(i - a) + abs(j - b) for a, b in S]
            assert dist[idx(i, j)] == min(dd)
            assert labels[idx(i, j)] == int(np.argmin(dd))


def floyd_warshall(n, e, w):
    D = np.full((n, n), np.inf)
    np.fill_diagonal(D, 0.0)
    for (a, b), c in zip(e, w):
        D[a, b] = min(D[a, b], c)
        D[b, a] = min(D[b, a], c)
    for k in range(n):
        D = np.minimum(D, D[:, k:k + 1] + D[k:k + 1, :])
    return D


@pytest.mark.parametrize("n,P,seed", [(40, 5, 0), (60, 12, 1), (25, 25, 2)])
def test_tiny_meshes_brute_force(n, P, seed):
    rng = np.random.default_rng(seed)
    u = gen.fibonacci_sphere(n)
    x = u * (1.0 + 0.2 * rng.random((n, 1)))
    e = gen.mesh_edges(gen.hull_mesh(u))
    D = floyd_warshall(n, e, edge_lengths(x, e))
    seeds, labels, dist = geodesic_fps(x, e, P)
    # the sampling rule as a plain loop over the all-pairs table
    chosen = [0]
    for _ in range(P - 1):
        m = D[chosen].min(axis=0)
        chosen.append(int(np.argmax(m)))
    assert seeds.tolist() == chosen
    Dm = D[chosen]
    np.testing.assert_allclose(dist, Dm.min(axis=0), rtol=1e-14, atol=0)
    # label = first seed attaining the minimum (exact comparisons against the
    # oracle's own distances decide ties; a Floyd-Warshall tie within
    # rounding is accepted if the labelled seed is within 1e-14 of the min)
    for v in range(n):
        assert Dm[labels[v], v] <= Dm[:, v].min() * (1 + 1e-14)


def test_disconnected_components():
    # two separate paths: the second component is unreachable from vertex 0,
    # so its lowest vertex (at +inf) is the next seed
    x1, e1 = path_graph(5)
    x2, e2 = path_graph(4)
    x2[:, 1] = 10.0
    x = np.vstack([x1, x2])
    e = np.vstack([e1, e2 + 5])
    seeds, labels, dist = geodesic_fps(x, e, 2)
    assert seeds.tolist() == [0, 5]
    np.testing.assert_array_equal(dist, [0, 1, 2, 3, 4, 0, 1, 2, 3])
    assert labels.tolist() == [0] * 5 + [1] * 4
    # one seed only: the other component stays at +inf with label 0
    _, labels1, dist1 = geodesic_fps(x, e, 1)
    assert np.isinf(dist1[5:]).all() and (labels1 == 0).all()


def test_edge_length_summation_order():
    x = np.array([[0.1, 0.2, 0.3], [1.7, -2.9, 0.05]])
    d = x[0] - x[1]
    want = np.sqrt((d[0] * d[0] + d[1] * d[1]) + d[2] * d[2])
    assert edge_lengths(x, np.array([[0, 1]]))[0] == want
    assert edge_lengths(x, np.array([[1, 0]]))[0] == want


def test_edge_lengths_pythagorean_and_library():
    # (3, 4, 12) has length 13 exactly; a dropped coordinate or square fails
    x = np.array([[0.0, 0.0, 0.0], [3.0, 4.0, 12.0], [-1.0, 2.0, 2.0]])
    e = np.array([[0, 1], [0, 2]])
    np.testing.assert_array_equal(edge_lengths(x, e), [13.0, 3.0])
    rng = np.random.default_rng(5)
    y = rng.standard_normal((50, 3))
    pairs = np.array(list(itertools.combinations(range(50), 2)))
    np.testing.assert_allclose(edge_lengths(y, pairs),
                               np.linalg.norm(y[pairs[:, 0]] - y[pairs[:, 1]], axis=1), rtol=3e-16)
