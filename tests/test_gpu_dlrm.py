"""GPU parity of the DLRM dot-product interaction (rec_dlrm_interact; DLRM
essay §2.3, §4.2) against the CPU oracle: every entry of every sample's
upper triangle (diagonal included, row by row).  fp32 products with fp32
accumulation in a different order than the oracle's fp64 loop: each entry's
error is measured against the size of its terms, sum_k |z_ik z_jk| (from the
oracle), at the fp32 tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, FP32_TOL, say
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu


def _run(z, guard=3):
    B, F, d = z.shape
    P = F * (F + 1) // 2
    zt = torch.from_numpy(np.ascontiguousarray(z, np.float32)).to(DEV)
    out = torch.full((B * P + guard,), 7.0, dtype=torch.float32, device=DEV)
    R.rec_dlrm_interact(zt, B, F, d, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[B * P:] == 7.0), "written past the output"
    return o[: B * P].reshape(B, P)


@pytest.mark.parametrize("B,F,d", [(1, 1, 16), (3, 5, 16), (7, 17, 32), (64, 27, 96), (300, 217, 96),
                                   (5, 256, 16), (4, 33, 160), (2, 217, 160), (1000, 16, 16)])
def test_dlrm_interact_parity(B, F, d):
    say(f"dlrm B={B} F={F} d={d}")
    rng = np.random.default_rng(B * 1000 + F + d)
    z = rng.standard_normal((B, F, d)).astype(np.float32)
    z[0, 0] = 0.0                                   # a zero vector: its row is exact zeros
    got = _run(z)
    ref, scale = oracle.get().dlrm_interact(z, want_scale=True)
    err = np.abs(got.astype(np.float64) - ref) / np.maximum(scale, 1e-30)
    say(f"  max error / term size {err.max():.3e}")
    assert err.max() <= FP32_TOL
    assert np.all(got[0, :F] == 0.0)


def test_dlrm_interact_independent_and_deterministic():
    """A sample's output depends on its own vectors only: a permuted batch
    gives the permuted outputs, bit for bit; the same batch twice gives the
    same bits."""
    rng = np.random.default_rng(3)
    z = rng.standard_normal((700, 27, 96)).astype(np.float32)
    perm = rng.permutation(700)
    a, a2 = _run(z), _run(z)
    b = _run(np.ascontiguousarray(z[perm]))
    assert np.array_equal(a, a2) and np.array_equal(a[perm], b)


def test_dlrm_interact_zero_batch():
    out = torch.full((8,), 7.0, device=DEV)
    z = torch.zeros(16, device=DEV)
    R.rec_dlrm_interact(z, 0, 5, 16, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
