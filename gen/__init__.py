"""Seeded synthetic inputs for the spatial-spectral coupling.

This module builds the workloads on which both the HIP library and the fp64
oracle run: meshes, descriptors F_N / F_M, the basis Phi_M, the upstream
gradient dO and the geodesic farthest-point-sampling (FPS) patch labels. It
holds none of the coupling's own arithmetic (no scores, softmax, means or
products of descriptors), so the oracle and the GPU path can share it.

What the pages fix (spatial-spectral-attention.github.io, "How it works"):
Q = F_N are the target descriptors, K = F_M the source descriptors and
V = Phi_M the source Laplace-Beltrami basis with k = 200 columns; the
Geo-FlashAttention section partitions each surface into geodesic patches by
farthest-point sampling.  Everything else below is the stated recipe of the
synthetic stand-ins (random-Fourier-feature descriptors, a QR-orthonormal
Gaussian in place of eigenfunctions, Fibonacci-lattice sphere meshes), with
the readings recorded in the project design notes.
"""

from __future__ import annotations

import dataclasses
import hashlib
import json
import math
import os
import shutil
import tempfile
from typing import Dict, Optional

import numpy as np
import scipy.sparse as sp
import scipy.sparse.csgraph as csgraph
from scipy.spatial import ConvexHull

__all__ = [
    "WORKLOADS",
    "Config",
    "bf16_bits_from_f32",
    "bf16_bits_to_f32",
    "fibonacci_sphere",
    "hull_mesh",
    "mesh_edges",
    "one_ring_smoother",
    "rotation",
    "fps_partition",
    "patch_sort",
    "make_config",
    "cached_config",
    "make_small",
]


# ----------------------------------------------------------------------------
# workload table
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    n: int                 # n_N = n_M
    d: int                 # descriptor width
    k: int                 # basis size
    dtype: str             # "f32" or "bf16" (storage of Q, K, V, dO)
    geometry: str          # "sphere-uniform" | "mesh" | "mesh-two" | "cortical"
    patches: int = 0       # P per shape (0 = dense variant)
    s: int = 0             # top-s source patches per target patch
    seed_index: int = -1   # SeedSequence([1234, seed_index])


WORKLOADS = (
    Config(0, "dense-1k-f32", 1000, 64, 30, "f32", "sphere-uniform", seed_index=0),
    Config(1, "dense-5k-bf16", 5000, 128, 200, "bf16", "mesh", seed_index=1),
    Config(2, "dense-60k-bf16", 60000, 128, 200, "bf16", "mesh-two", seed_index=2),
    Config(3, "geo-60k-bf16-P256-s16", 60000, 128, 200, "bf16", "mesh-two",
           patches=256, s=16, seed_index=2),
    Config(4, "geo-160k-bf16-P640-s16", 160000, 128, 200, "bf16", "cortical",
           patches=640, s=16, seed_index=4),
)

# Named RNG streams, spawned from one SeedSequence in this fixed order.
_STREAMS = ("mesh_src", "mesh_tgt", "rotation", "rff", "jitter", "noise_N",
            "noise_M", "phi", "dO", "points")


def _streams(seed_index: int) -> Dict[str, np.random.Generator]:
    ss = np.random.SeedSequence([1234, seed_index])
    return {name: np.random.default_rng(child)
            for name, child in zip(_STREAMS, ss.spawn(len(_STREAMS)))}


# ----------------------------------------------------------------------------
# bf16 storage (round to nearest even, as the inputs are quantised once)
# ----------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    Inputs are finite by construction.  The bias 0x7FFF plus the lowest kept
    bit implements ties-to-even on the 16 discarded bits.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------
def fibonacci_sphere(n: int) -> np.ndarray:
    """n near-uniform unit directions on a golden-angle spiral (fp64)."""
    i = np.arange(n, dtype=np.float64)
    z = 1.0 - (2.0 * i + 1.0) / n
    r = np.sqrt(np.maximum(0.0, 1.0 - z * z))
    phi = i * (math.pi * (3.0 - math.sqrt(5.0)))
    return np.stack([r * np.cos(phi), r * np.sin(phi), z], axis=1)


def hull_mesh(u: np.ndarray) -> np.ndarray:
    """Triangles of the convex hull of points on the sphere (int64 [F,3])."""
    return np.asarray(ConvexHull(u).simplices, dtype=np.int64)


def mesh_edges(faces: np.ndarray) -> np.ndarray:
    """Unique undirected edges (i < j), sorted, int64 [E,2]."""
    e = np.concatenate([faces[:, [0, 1]], faces[:, [1, 2]], faces[:, [2, 0]]])
    e = np.sort(e, axis=1)
    return np.unique(e, axis=0)


def mesh_csr(edges: np.ndarray, n: int):
    """CSR adjacency of unique undirected edges, both directions of every
    edge, neighbours ascending: (off int32 [n+1], adj int32 [2E])."""
    e = np.asarray(edges, np.int64)
    src = np.r_[e[:, 0], e[:, 1]]
    dst = np.r_[e[:, 1], e[:, 0]]
    order = np.lexsort((dst, src))
    off = np.zeros(n + 1, np.int64)
    np.add.at(off, src + 1, 1)
    return np.cumsum(off).astype(np.int32), dst[order].astype(np.int32)


def one_ring_smoother(n: int, edges: np.ndarray) -> sp.csr_matrix:
    """Closed 1-ring mean operator: (I + A) / (1 + deg)."""
    i, j = edges[:, 0], edges[:, 1]
    a = sp.coo_matrix((np.ones(2 * len(edges)), (np.r_[i, j], np.r_[j, i])),
                      shape=(n, n)).tocsr()
    a = a + sp.identity(n, format="csr")
    deg = np.asarray(a.sum(axis=1)).ravel()
    return sp.diags(1.0 / deg) @ a


def rotation(rng: np.random.Generator, degrees: float = 10.0) -> np.ndarray:
    """Rotation by exactly `degrees` about an axis uniform on S^2 (Rodrigues)."""
    axis = rng.standard_normal(3)
    axis /= np.linalg.norm(axis)
    th = math.radians(degrees)
    kx = np.array([[0.0, -axis[2], axis[1]],
                   [axis[2], 0.0, -axis[0]],
                   [-axis[1], axis[0], 0.0]])
    return np.eye(3) + math.sin(th) * kx + (1.0 - math.cos(th)) * (kx @ kx)


def _edge_graph(x: np.ndarray, edges: np.ndarray) -> sp.csr_matrix:
    w = np.linalg.norm(x[edges[:, 0]] - x[edges[:, 1]], axis=1)
    n = len(x)
    g = sp.coo_matrix((np.r_[w, w], (np.r_[edges[:, 0], edges[:, 1]],
                                      np.r_[edges[:, 1], edges[:, 0]])), shape=(n, n))
    return g.tocsr()


def fps_partition(x: np.ndarray, edges: np.ndarray, P: int):
    """Geodesic farthest-point sampling and Voronoi labels.

    Geodesic distance = shortest path on the edge graph with Euclidean edge
    lengths (fp64).  Seed 0 is vertex 0; each next seed is the vertex whose
    distance to the chosen seeds is largest (ties -> lower vertex index).
    A vertex's label is the FPS order of its nearest seed (ties -> the earlier
    seed, since a label only moves on a strictly smaller distance).

    Returns (labels int32 [n], seeds int64 [P], dist float64 [n]).
    """
    n = len(x)
    if not (1 <= P <= n):
        raise ValueError("need 1 <= P <= n")
    g = _edge_graph(x, edges)
    dist = np.full(n, np.inf)
    labels = np.zeros(n, dtype=np.int32)
    seeds = np.zeros(P, dtype=np.int64)
    cur = 0
    for t in range(P):
        seeds[t] = cur
        limit = np.inf if t == 0 else float(dist.max())
        dn = csgraph.dijkstra(g, directed=False, indices=int(cur), limit=limit)
        better = dn < dist
        dist = np.where(better, dn, dist)
        labels[better] = t
        if t + 1 < P:
            cur = int(np.argmax(dist))
    return labels, seeds, dist


def patch_sort(labels: np.ndarray, P: int):
    """Patch-contiguous order: by label, then by original index.

    Returns (perm int64 [n], off int32 [P+1]); rows of patch p occupy
    [off[p], off[p+1]) of x[perm].
    """
    labels = np.asarray(labels)
    perm = np.lexsort((np.arange(len(labels)), labels))
    cnt = np.bincount(labels, minlength=P)
    off = np.zeros(P + 1, dtype=np.int32)
    off[1:] = np.cumsum(cnt)
    return perm.astype(np.int64), off


# ----------------------------------------------------------------------------
# descriptors, basis, upstream gradient
# ----------------------------------------------------------------------------
def _rff(x, W, b):
    return np.cos(x @ W.T + b)


def _radius_mesh(u, S, rng, amp, steps):
    r = 1.0 + amp * rng.standard_normal(len(u))
    for _ in range(steps):
        r = S @ r
    return r


def _radius_cortical(u, S, rng):
    # r = 1 + 0.3 * sum_t S^t z_t over smoothing scales t in {3, 10, 30}
    acc = np.zeros(len(u))
    for t in (3, 10, 30):
        z = rng.standard_normal(len(u))
        for _ in range(t):
            z = S @ z
        acc += z
    return np.maximum(1.0 + 0.3 * acc, 0.2)


def _geometry(cfg: Config, st):
    """Source / target vertex positions (fp64) and the shared edge list."""
    n = cfg.n
    if cfg.geometry == "sphere-uniform":
        g = st["points"].standard_normal((n, 3))
        xm = g / np.linalg.norm(g, axis=1, keepdims=True)
        return xm, None, None, None
    u = fibonacci_sphere(n)
    faces = hull_mesh(u)
    edges = mesh_edges(faces)
    S = one_ring_smoother(n, edges)
    if cfg.geometry == "mesh":
        xm = _radius_mesh(u, S, st["mesh_src"], 0.1, 3)[:, None] * u
        xn_base = xm
    elif cfg.geometry == "mesh-two":
        xm = _radius_mesh(u, S, st["mesh_src"], 0.1, 3)[:, None] * u
        xn_base = _radius_mesh(u, S, st["mesh_tgt"], 0.1, 3)[:, None] * u
    elif cfg.geometry == "cortical":
        xm = _radius_cortical(u, S, st["mesh_src"])[:, None] * u
        xn_base = _radius_cortical(u, S, st["mesh_tgt"])[:, None] * u
    else:
        raise ValueError(cfg.geometry)
    return xm, xn_base, faces, edges


def _finish(cfg: Config, st, xm, xn_base):
    n, d, k = cfg.n, cfg.d, cfg.k
    R = rotation(st["rotation"], 10.0)
    if xn_base is None:
        xn_base = xm
    # jitter N(0, 0.01): variance 0.01, sigma 0.1 per coordinate
    xn = xn_base @ R.T + 0.1 * st["jitter"].standard_normal((n, 3))
    # W ~ N(0, 4^2) entrywise, b ~ U[0, 2pi); shared by both shapes
    W = 4.0 * st["rff"].standard_normal((d, 3))
    b = st["rff"].uniform(0.0, 2.0 * math.pi, d)
    sig = math.sqrt(0.1)  # N(0, 0.1) descriptor noise
    FN = _rff(xn, W, b) + sig * st["noise_N"].standard_normal((n, d))
    FM = _rff(xm, W, b) + sig * st["noise_M"].standard_normal((n, d))
    G = st["phi"].standard_normal((n, k))
    Qr, _ = np.linalg.qr(G, mode="reduced")
    Phi = math.sqrt(n) * Qr
    dO = st["dO"].standard_normal((n, k))
    return xn, FN, FM, Phi, dO


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    f32 = np.ascontiguousarray(a64, dtype=np.float32)
    return bf16_bits_from_f32(f32) if dtype == "bf16" else f32


def make_config(i: int, with_partition: Optional[bool] = None) -> dict:
    """Inputs of workload i as stored arrays.

    Returned keys: Q, K, V, dO (uint16 bf16 bits or float32; row-major),
    dtype, n, d, k, scale, and for geo workloads labN, labM (int32 per-vertex
    patch labels in original order), P, s.  Positions xN, xM (fp64) and the
    edge list are included for the mesh workloads.
    """
    cfg = WORKLOADS[i]
    st = _streams(cfg.seed_index)
    xm, xn_base, faces, edges = _geometry(cfg, st)
    xn, FN, FM, Phi, dO = _finish(cfg, st, xm, xn_base)
    out = dict(config=cfg.name, index=i, dtype=cfg.dtype, n=cfg.n, d=cfg.d, k=cfg.k,
               scale=1.0 / math.sqrt(cfg.d),
               Q=_store(FN, cfg.dtype), K=_store(FM, cfg.dtype),
               V=_store(Phi, cfg.dtype), dO=_store(dO, cfg.dtype),
               xN=xn, xM=xm, edges=edges)
    if with_partition is None:
        with_partition = cfg.patches > 0
    if with_partition and cfg.patches > 0:
        labN, _, _ = fps_partition(xn, edges, cfg.patches)
        labM, _, _ = fps_partition(xm, edges, cfg.patches)
        out.update(labN=labN, labM=labM, P=cfg.patches, s=cfg.s)
    return out


# ----------------------------------------------------------------------------
# cached workloads
# ----------------------------------------------------------------------------
def _generator_version() -> str:
    """sha256 of this module's source: any change to the recipe invalidates
    every cached workload."""
    with open(os.path.abspath(__file__), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def _sha256_file(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as fh:
        for chunk in iter(lambda: fh.read(1 << 22), b""):
            h.update(chunk)
    return h.hexdigest()


def cached_config(i: int, root: Optional[str] = None) -> dict:
    """make_config(i), kept on disk: root/cfg{i}/ holds one .npy per array
    and manifest.json (workload name, seed index, generator version = sha256
    of this module, and per array its file, shape, dtype and sha256).  A
    cache whose manifest or any file does not match is regenerated.  root
    defaults to $SSC_DATA_DIR, else data/ next to this package."""
    cfg = WORKLOADS[i]
    root = root or os.environ.get("SSC_DATA_DIR") or os.path.join(
        os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "data")
    d = os.path.join(root, f"cfg{i}")
    version = _generator_version()
    man_path = os.path.join(d, "manifest.json")
    try:
        with open(man_path) as fh:
            man = json.load(fh)
        if (man.get("generator_version") == version and man.get("config") == cfg.name
                and man.get("seed_index") == cfg.seed_index):
            out = dict(man["scalars"])
            for name, meta in man["arrays"].items():
                path = os.path.join(d, meta["file"])
                if _sha256_file(path) != meta["sha256"]:
                    raise ValueError(f"{path}: checksum mismatch")
                a = np.load(path, allow_pickle=False)
                if list(a.shape) != meta["shape"] or str(a.dtype) != meta["dtype"]:
                    raise ValueError(f"{path}: shape or dtype mismatch")
                out[name] = a
            return out
    except (OSError, ValueError, KeyError, json.JSONDecodeError):
        pass
    out = make_config(i)
    os.makedirs(root, exist_ok=True)
    tmp = tempfile.mkdtemp(prefix=f"cfg{i}.", dir=root)
    arrays = {}
    for name, v in out.items():
        if isinstance(v, np.ndarray):
            f = name + ".npy"
            np.save(os.path.join(tmp, f), v, allow_pickle=False)
            arrays[name] = {"file": f, "shape": list(v.shape), "dtype": str(v.dtype),
                            "sha256": _sha256_file(os.path.join(tmp, f))}
    scalars = {k: (v.item() if isinstance(v, np.generic) else v) for k, v in out.items()
               if not isinstance(v, np.ndarray)}
    with open(os.path.join(tmp, "manifest.json"), "w") as fh:
        json.dump({"config": cfg.name, "index": i, "seed_index": cfg.seed_index,
                   "generator_version": version, "scalars": scalars, "arrays": arrays}, fh, indent=1)
    shutil.rmtree(d, ignore_errors=True)
    try:
        os.replace(tmp, d)
    except OSError:  # another process placed its copy first
        shutil.rmtree(tmp, ignore_errors=True)
    return out


def make_small(n_N: int, n_M: int, d: int, k: int, dtype: str = "bf16",
               seed: int = 0, P_N: int = 0, P_M: int = 0, s: int = 0,
               spread: float = 1.0) -> dict:
    """Small seeded instances for parity tests (any sizes, ragged tails).

    Descriptors follow the same random-Fourier-feature recipe on random
    points of the unit sphere; when P_N / P_M are given, patch labels come
    from geodesic FPS on a Fibonacci hull mesh of each shape (needs
    n >= 4 and P <= n).  `spread` scales the descriptors (sharper or flatter
    softmax rows).
    """
    ss = np.random.SeedSequence([4321, seed, n_N, n_M, d, k])
    r = [np.random.default_rng(c) for c in ss.spawn(8)]
    W = 4.0 * r[0].standard_normal((d, 3))
    b = r[0].uniform(0.0, 2.0 * math.pi, d)

    def shape(m, rng):
        if m >= 4 and (P_N or P_M):
            u = fibonacci_sphere(m)
            faces = hull_mesh(u)
            edges = mesh_edges(faces)
            R = rotation(rng, float(rng.uniform(0, 360)))
            x = u @ R.T
            return x, edges
        g = rng.standard_normal((m, 3))
        return g / np.linalg.norm(g, axis=1, keepdims=True), None

    xn, eN = shape(n_N, r[1])
    xm, eM = shape(n_M, r[2])
    sig = math.sqrt(0.1)
    FN = spread * (_rff(xn, W, b) + sig * r[3].standard_normal((n_N, d)))
    FM = spread * (_rff(xm, W, b) + sig * r[4].standard_normal((n_M, d)))
    G = r[5].standard_normal((n_M, k))
    if n_M >= k:
        Qr, _ = np.linalg.qr(G, mode="reduced")
        Phi = math.sqrt(n_M) * Qr
    else:
        Phi = G
    dO = r[6].standard_normal((n_N, k))
    out = dict(config=f"small-{n_N}x{n_M}-d{d}-k{k}-{dtype}", dtype=dtype,
               n_N=n_N, n_M=n_M, d=d, k=k, scale=1.0 / math.sqrt(d),
               Q=_store(FN, dtype), K=_store(FM, dtype), V=_store(Phi, dtype),
               dO=_store(dO, dtype))
    if P_N and P_M:
        out["labN"] = fps_partition(xn, eN, P_N)[0] if eN is not None else \
            (np.arange(n_N) % P_N).astype(np.int32)
        out["labM"] = fps_partition(xm, eM, P_M)[0] if eM is not None else \
            (np.arange(n_M) % P_M).astype(np.int32)
        out.update(P_N=P_N, P_M=P_M, s=s)
    return out


def make_basis(n: int, k: int, seed: int = 0, cond: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """A seeded spectral-basis stand-in [n x k] (stored bf16 bits or fp32):
    sqrt(n) times orthonormal columns, mixed by a random rotation after
    scaling the columns geometrically from 1 down to 1/cond, so the basis has
    condition number about `cond` (cond = 1: orthogonal columns of norm
    sqrt(n), like an eigenbasis orthonormal in the vertex inner product)."""
    ss = np.random.SeedSequence([8765, seed, n, k])
    r = [np.random.default_rng(c) for c in ss.spawn(2)]
    G = r[0].standard_normal((n, k))
    Qr, _ = np.linalg.qr(G, mode="reduced") if n >= k else (G / math.sqrt(max(n, 1)), None)
    scales = np.geomspace(1.0, 1.0 / cond, k)
    W, _ = np.linalg.qr(r[1].standard_normal((k, k)))
    return _store(math.sqrt(n) * (Qr * scales) @ W.T, dtype)


def make_favor_directions(m: int, d: int, seed: int = 0, orthogonal: bool = True,
                          dtype: str = "bf16") -> np.ndarray:
    """Random feature directions W [m x d] for the Performer coupling, drawn
    from a seeded stream: Gaussian rows, or (orthogonal=True) blocks of d
    orthonormal rows scaled by the norms of independent Gaussian vectors, so
    that every row keeps the N(0, I) length distribution."""
    rng = np.random.default_rng(np.random.SeedSequence([2468, seed, m, d]))
    if not orthogonal:
        return _store(rng.standard_normal((m, d)), dtype)
    blocks = []
    for _ in range((m + d - 1) // d):
        Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        blocks.append(Qm.T)
    W = np.vstack(blocks)[:m]
    norms = np.linalg.norm(rng.standard_normal((m, d)), axis=1)
    return _store(W * norms[:, None], dtype)
