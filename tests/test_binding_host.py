"""Host-side checks of the Python binding's argument validation (no GPU).

The binding hands raw device pointers to the C ABI, so a tensor of the wrong
shape or dtype would make a kernel read or write past its buffer.  Every
entry point must reject such tensors with TypeError / ValueError naming the
argument before any pointer is taken; well-formed CPU tensors get past those
checks and stop at the device check.
"""

import pytest
import torch

import spatial_spectral_coupling_amd as ssc

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def z(*shape, dtype=BF):
    return torch.zeros(*shape, dtype=dtype)


def test_dense_fwd_checks():
    Q, K, V = z(5, 128), z(7, 128), z(7, 200)
    with pytest.raises(ValueError, match="K must"):
        ssc.coupling_dense_fwd(Q, z(6, 128), V)
    with pytest.raises(TypeError):
        ssc.coupling_dense_fwd(Q, K.float(), V)
    with pytest.raises(TypeError, match="O must"):
        ssc.coupling_dense_fwd(Q, K, V, O=z(5, 200))
    with pytest.raises(ValueError, match="O must"):
        ssc.coupling_dense_fwd(Q, K, V, O=z(5, 100, dtype=F32))
    with pytest.raises(ValueError, match="lse must"):
        ssc.coupling_dense_fwd(Q, K, V, lse=z(4, dtype=F32))
    with pytest.raises(ValueError, match="matrix"):
        ssc.coupling_dense_fwd(z(5, 128, 1), K, V)
    with pytest.raises(ValueError, match="GPU"):
        ssc.coupling_dense_fwd(Q, K, V)


def test_dense_bwd_checks():
    Q, K, V = z(5, 128), z(7, 128), z(7, 200)
    O, dO, lse = z(5, 200, dtype=F32), z(5, 200), z(5, dtype=F32)
    with pytest.raises(ValueError, match="O must"):
        ssc.coupling_dense_bwd(Q, K, V, z(5, 199, dtype=F32), dO, lse)
    with pytest.raises(TypeError, match="O must"):
        ssc.coupling_dense_bwd(Q, K, V, z(5, 200), dO, lse)
    with pytest.raises(ValueError, match="dO must"):
        ssc.coupling_dense_bwd(Q, K, V, O, z(6, 200), lse)
    with pytest.raises(ValueError, match="lse must"):
        ssc.coupling_dense_bwd(Q, K, V, O, dO, z(7, dtype=F32))
    with pytest.raises(TypeError, match="lse must"):
        ssc.coupling_dense_bwd(Q, K, V, O, dO, z(5, dtype=torch.float64))
    with pytest.raises(ValueError, match="K must"):
        ssc.coupling_dense_bwd(Q, z(7, 64), V, O, dO, lse)
    with pytest.raises(ValueError, match="GPU"):
        ssc.coupling_dense_bwd(Q, K, V, O, dO, lse, need_dV=False)


def test_patch_topk_checks():
    Q, K = z(10, 128), z(12, 128)
    offN, offM = torch.tensor([0, 4, 10], dtype=I32), torch.tensor([0, 12], dtype=I32)
    with pytest.raises(TypeError, match="offN"):
        ssc.patch_score_topk(Q, offN.long(), K, offM, 1)
    with pytest.raises(ValueError, match="offM"):
        ssc.patch_score_topk(Q, offN, K, torch.tensor([0], dtype=I32), 1)
    with pytest.raises(ValueError, match="width"):
        ssc.patch_score_topk(Q, offN, z(12, 64), offM, 1)
    with pytest.raises(ValueError, match="GPU"):
        ssc.patch_score_topk(Q, offN, K, offM, 1)


def test_geo_checks():
    Q, K, V = z(10, 128), z(12, 128), z(12, 200)
    offN, offM = torch.tensor([0, 4, 10], dtype=I32), torch.tensor([0, 5, 12], dtype=I32)
    idx = torch.tensor([[1], [0]], dtype=I32)
    O, dO, lse = z(10, 200, dtype=F32), z(10, 200), z(10, dtype=F32)
    with pytest.raises(TypeError, match="idx"):
        ssc.coupling_geo_fwd(Q, K, V, offN, offM, idx.long())
    with pytest.raises(ValueError, match="idx"):
        ssc.coupling_geo_fwd(Q, K, V, offN, offM, torch.tensor([[1]], dtype=I32))
    with pytest.raises(ValueError, match="idx"):
        ssc.coupling_geo_fwd(Q, K, V, offN, offM, torch.tensor([1, 0], dtype=I32))
    with pytest.raises(TypeError, match="idx"):
        ssc.coupling_geo_bwd(Q, K, V, offN, offM, idx.long(), O, dO, lse)
    with pytest.raises(ValueError, match="idx"):
        ssc.coupling_geo_bwd(Q, K, V, offN, offM, torch.tensor([[1]], dtype=I32), O, dO, lse)
    with pytest.raises(ValueError, match="dO must"):
        ssc.coupling_geo_bwd(Q, K, V, offN, offM, idx, O, z(10, 100), lse)
    with pytest.raises(TypeError, match="offM"):
        ssc.coupling_geo_bwd(Q, K, V, offN, offM.float(), idx, O, dO, lse)
    with pytest.raises(ValueError, match="GPU"):
        ssc.coupling_geo_fwd(Q, K, V, offN, offM, idx)
    with pytest.raises(ValueError, match="GPU"):
        ssc.coupling_geo_bwd(Q, K, V, offN, offM, idx, O, dO, lse, need_dV=False)


def test_linear_performer_fmap_checks():
    Q, K, V = z(5, 128), z(7, 128), z(7, 200)
    O, dO, den = z(5, 200, dtype=F32), z(5, 200), z(5, dtype=F32)
    with pytest.raises(ValueError, match="K must"):
        ssc.coupling_linear_fwd(Q, z(7, 64), V)
    with pytest.raises(ValueError, match="O must"):
        ssc.coupling_linear_bwd(Q, K, V, z(4, 200, dtype=F32), dO, den)
    with pytest.raises(ValueError, match="W must"):
        ssc.coupling_performer_fwd(Q, K, V, z(128, 64))
    with pytest.raises(ValueError, match="W must"):
        ssc.coupling_performer_bwd(Q, K, V, z(64, 96), O, dO, den)
    with pytest.raises(ValueError, match="O must"):
        ssc.fmap_solve_fwd(z(50, 200), z(50, 199, dtype=F32))
    with pytest.raises(TypeError, match="dC must"):
        ssc.fmap_solve_bwd(z(50, 200), z(200, 200))
