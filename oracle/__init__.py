"""fp64 CPU oracle of the spatial-spectral coupling -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it and shares no code,
header, table or helper with it; the two meet only in the seeded input
generator (`gen`), which holds none of the method's arithmetic.

What it computes (spatial-spectral-attention.github.io, "How it works" and
"Geo-FlashAttention"; ai4snews digest, "Interpretation"):

* dense coupling   Pi_NM Phi_M = softmax(F_N F_M^T * scale) Phi_M with
  Q = F_N (target descriptors), K = F_M (source descriptors), V = Phi_M,
  softmax over source vertices for each target vertex, scale = 1/sqrt(d);
  its backward (dQ, dK, dV for an upstream gradient dO of the product);
* Geo-FlashAttention: per-shape patches -> patch-mean descriptors ->
  patch scores -> top-s source patches per target patch -> the exact softmax
  of each target row restricted to the union of its selected source patches;
  forward and backward for the fixed selection;
* the linear-attention (ELU feature map) coupling, the pages' linearized
  baseline (`oracle.linear`), forward and backward;
* the least-squares functional map C = Phi_N^+ (Pi Phi_M) that the coupled
  pipelines compute from the product (`oracle.fmap`), forward and backward;
* the geodesic farthest-point-sampling patch partition (`oracle.fps`);
* the Performer (FAVOR+ positive random features) coupling, the pages'
  second linearized baseline (`oracle.performer`), forward and backward.

Every function is the plain definition, written out in fp64 with NumPy; a
pure-Python brute force (`oracle.brute`) covers tiny inputs.  Parity status:
every function here is pinned by the CPU tests (closed forms, invariants,
library routines, finite differences) -- none is "parity unpinned".
"""

from .dense import upcast, dense_fwd, dense_bwd, dense_rows, rowdot
from .geo import (patch_means, patch_scores, topk, cut_gaps, geo_support,
                  geo_fwd, geo_bwd, executed_pairs)
from .linear import elu1, elu1_grad, linear_fwd, linear_bwd, linear_weights
from .fmap import fmap_solve, fmap_solve_bwd
from .fps import edge_lengths, geodesic_fps
from .performer import favor_features, performer_fwd, performer_bwd

__all__ = ["upcast", "dense_fwd", "dense_bwd", "dense_rows", "rowdot",
           "patch_means", "patch_scores", "topk", "cut_gaps", "geo_support",
           "geo_fwd", "geo_bwd", "executed_pairs",
           "elu1", "elu1_grad", "linear_fwd", "linear_bwd", "linear_weights",
           "fmap_solve", "fmap_solve_bwd", "edge_lengths", "geodesic_fps",
           "favor_features", "performer_fwd", "performer_bwd"]
