"""Seeded input generator: determinism, storage rounding, mesh validity and the
geodesic FPS partition checked against scipy's own Dijkstra (textbook routine).
"""

import hashlib

import numpy as np
import pytest
import scipy.sparse as sp
import scipy.sparse.csgraph as csgraph
import torch

import gen


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    ours = gen.bf16_bits_from_f32(x)
    theirs = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    # ties go to even: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6
    assert gen.bf16_bits_to_f32(ours[5000]) == np.float32(1.0)
    assert gen.bf16_bits_to_f32(ours[5001]) == np.float32(1.0 + 2 ** -6)


def test_make_config_deterministic_and_shaped():
    a, b = gen.make_config(0), gen.make_config(0)
    for key in ("Q", "K", "V", "dO"):
        assert sha(a[key]) == sha(b[key])
    assert a["Q"].shape == (1000, 64) and a["V"].shape == (1000, 30)
    assert a["Q"].dtype == np.float32
    # Phi = sqrt(n) * orthonormal columns  =>  Phi^T Phi = n I
    V = a["V"].astype(np.float64)
    np.testing.assert_allclose(V.T @ V, 1000 * np.eye(30), atol=2e-3)
    c = gen.make_config(1)
    assert c["Q"].dtype == np.uint16 and c["V"].shape == (5000, 200)


def test_small_instances_deterministic():
    a = gen.make_small(37, 41, 64, 30, "bf16", seed=3, P_N=5, P_M=6, s=2)
    b = gen.make_small(37, 41, 64, 30, "bf16", seed=3, P_N=5, P_M=6, s=2)
    for key in ("Q", "K", "V", "dO", "labN", "labM"):
        np.testing.assert_array_equal(a[key], b[key])
    assert set(np.unique(a["labN"])) == set(range(5))


def test_mesh_is_closed_manifold_sphere():
    u = gen.fibonacci_sphere(800)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), 1.0, atol=1e-15)
    faces = gen.hull_mesh(u)
    edges = gen.mesh_edges(faces)
    assert len(u) - len(edges) + len(faces) == 2          # Euler characteristic
    e = np.sort(np.concatenate([faces[:, [0, 1]], faces[:, [1, 2]], faces[:, [2, 0]]]), axis=1)
    _, cnt = np.unique(e, axis=0, return_counts=True)
    assert np.all(cnt == 2)                                # every edge has two faces


def test_rotation_is_ten_degrees():
    R = gen.rotation(np.random.default_rng(5), 10.0)
    np.testing.assert_allclose(R @ R.T, np.eye(3), atol=1e-15)
    assert np.degrees(np.arccos((np.trace(R) - 1) / 2)) == pytest.approx(10.0, abs=1e-9)


def test_fps_partition_against_scipy_dijkstra():
    n, P = 600, 12
    u = gen.fibonacci_sphere(n)
    faces = gen.hull_mesh(u)
    edges = gen.mesh_edges(faces)
    x = u * (1 + 0.1 * np.random.default_rng(1).standard_normal((n, 1)))
    labels, seeds, dist = gen.fps_partition(x, edges, P)
    w = np.linalg.norm(x[edges[:, 0]] - x[edges[:, 1]], axis=1)
    g = sp.coo_matrix((w, (edges[:, 0], edges[:, 1])), shape=(n, n)).tocsr()
    full = csgraph.dijkstra(g, directed=False, indices=seeds)      # [P, n], no limit
    assert seeds[0] == 0
    for t in range(1, P):
        mind = full[:t].min(axis=0)
        assert seeds[t] == int(np.argmax(mind))                    # farthest point, low index on ties
    np.testing.assert_array_equal(labels, np.argmin(full, axis=0))  # Voronoi label, earliest seed on ties
    np.testing.assert_allclose(dist, full.min(axis=0), rtol=1e-15, atol=0)
    assert np.all(np.bincount(labels, minlength=P) > 0)


def test_patch_sort():
    lab = np.array([2, 0, 1, 0, 2, 2, 1], dtype=np.int32)
    perm, off = gen.patch_sort(lab, 4)
    np.testing.assert_array_equal(perm, [1, 3, 2, 6, 0, 4, 5])
    np.testing.assert_array_equal(off, [0, 2, 4, 7, 7])
