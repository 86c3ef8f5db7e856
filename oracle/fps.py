"""Geodesic farthest-point-sampling partition of a mesh, in fp64 -- test
infrastructure only.

Geo-FlashAttention partitions each surface into patches by geodesic
farthest-point sampling (project page, "Abstract" and "Geo-FlashAttention";
ai4snews digest, "Synopsis").  The pages give no further rule; the reading
taken here:

* geodesic distance = shortest path on the mesh's edge graph, an edge
  weighing its Euclidean length sqrt((dx^2 + dy^2) + dz^2) in fp64, a path's
  length summed from its start vertex outward;
* seed 0 is vertex 0; seed t is the vertex farthest (in that distance) from
  the seeds chosen before it, ties to the lower vertex index;
* each vertex is labelled with its nearest seed, ties to the earlier seed.

Written out as the definition: one full single-source shortest-path run per
seed (SciPy's Dijkstra as the library step), the running minimum over the
seeds so far, and the strict "closer than before" test that keeps the
earlier seed on ties.
"""

from __future__ import annotations

import numpy as np
from scipy.sparse import coo_matrix
from scipy.sparse.csgraph import dijkstra

__all__ = ["edge_lengths", "edge_graph", "geodesic_fps"]


def edge_lengths(x, edges) -> np.ndarray:
    """Euclidean length of every edge (i, j): sqrt((dx^2 + dy^2) + dz^2)."""
    x = np.asarray(x, np.float64)
    e = np.asarray(edges, np.int64)
    d = x[e[:, 0]] - x[e[:, 1]]
    return np.sqrt((d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2])


def edge_graph(x, edges):
    """Symmetric sparse weight matrix of a list of unique undirected edges."""
    e = np.asarray(edges, np.int64)
    w = edge_lengths(x, e)
    n = len(x)
    return coo_matrix((np.r_[w, w], (np.r_[e[:, 0], e[:, 1]], np.r_[e[:, 1], e[:, 0]])),
                      shape=(n, n)).tocsr()


def geodesic_fps(x, edges, P: int):
    """Farthest-point sampling of P seeds and the geodesic Voronoi labels.

    x: [n x 3] positions; edges: [E x 2] unique undirected vertex pairs (no
    zero-length edges).  Returns (seeds int64 [P] in sampling order,
    labels int32 [n] = index t of the nearest seed, dist float64 [n] =
    distance to the nearest seed; +inf where no seed is reachable, and such
    vertices keep label 0).
    """
    n = len(x)
    if not 1 <= P <= n:
        raise ValueError("need 1 <= P <= n")
    g = edge_graph(x, edges)
    dist = np.full(n, np.inf)
    labels = np.zeros(n, np.int32)
    seeds = np.zeros(P, np.int64)
    s = 0
    for t in range(P):
        seeds[t] = s
        ds = dijkstra(g, directed=True, indices=s)
        closer = ds < dist
        dist[closer] = ds[closer]
        labels[closer] = t
        s = int(np.argmax(dist))  # first index of the largest distance
    return seeds, labels, dist
