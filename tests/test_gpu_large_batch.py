"""The whole forward at a million samples (2^20, 16 x 2^20 bags and about
4.2 M packed positions: many KJT blocks and segments, and attention groups
of about 16 K positions each) against the oracle on 512 sampled rows (the
first two and last two samples among them); every attention output finite."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import BF16_TOL, DEV, oracle_forward, row_rel_err, say
from sparse_embedding_din_amd import pipeline as PL

pytestmark = pytest.mark.gpu


def test_whole_forward_million_samples():
    m = synth.make_model(synth.WORKLOADS[2], bias=True)
    B = 1 << 20
    b = synth.make_batch(m, B=B, batch_index=3)
    say(f"whole forward B={B} nnz={b.values.size} P={b.seq_stride}")
    tabs, mlp = PL.DeviceTables(m.tables, DEV), PL.DeviceMLP(m, DEV)
    db = PL.DeviceBatch(b, DEV)
    f = PL.SparseDinForward(tabs, mlp, B, m.cfg.max_len, DEV)
    f.run_whole(db)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([[0, 1, B - 2, B - 1],
                                    rng.choice(B, 508, replace=False)]))
    it = torch.from_numpy(idx).to(DEV)
    pooled = f.pooled[:B].index_select(0, it).cpu().numpy()
    att = f.att[:B].index_select(0, it).cpu().numpy()
    o = oracle_forward(m, b, samples=idx, want_scores=False)
    assert row_rel_err(pooled, o["pooled"]) <= 1e-6
    assert row_rel_err(att, o["att"]) <= BF16_TOL
    assert np.all(np.isfinite(f.att[:B].cpu().numpy()))
