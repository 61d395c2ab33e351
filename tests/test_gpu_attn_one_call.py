"""GPU parity of the one-call DIN attention, rec_din_attn_fwd ("当前现状分析"
§4.2, §4.4; the plan is built inside the caller's workspace), against the
CPU oracle: outputs per row within the MLP precision's tolerance, scores and
softmax weights per packed position, resolved sequence rows bit-exact, and
bit-identical to the plan-based call (rec_din_plan + rec_din_attn_fwd_plan)
on the same inputs.  Also max_len at its largest, 1024, with sequences of
several hundred positions and some past the cap."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import BF16_TOL, DEV, FP32_TOL, Run, oracle_forward, oracle_rows, row_rel_err, say
from sparse_embedding_din_amd import pipeline as PL

pytestmark = pytest.mark.gpu


def _one_call(r, B, max_len, seq_tables=None):
    """rec_din_attn_fwd on a finished Run (its pooled output is the query)."""
    f, db = r.fwd, r.db
    P = int(np.minimum(r.batch.seq_lengths, max_len).sum())
    att = torch.full((B, 48), np.nan, dtype=torch.float32, device=DEV)
    sc = torch.full((max(P, 1),), np.nan, dtype=torch.float32, device=DEV)
    wt = torch.full((max(P, 1),), np.nan, dtype=torch.float32, device=DEV)
    rows = torch.full((3 * max(db.seq_stride, 1),), -7, dtype=torch.int64, device=DEV)
    saved = f.att
    f.att = att
    f.din_one_call(db, scores=sc, weights=wt, rows_out=rows)
    f.att = saved
    torch.cuda.synchronize()
    return (att.cpu().numpy(), sc.cpu().numpy()[:P], wt.cpu().numpy()[:P],
            rows.cpu().numpy().reshape(3, -1))


@pytest.mark.parametrize("cfg,B", [(1, 256), (1, 37), (2, 8192)])
def test_attn_one_call_parity(cfg, B):
    m = synth.make_model(synth.WORKLOADS[cfg], bias=True)
    b = synth.make_batch(m, B=B)
    r = Run(m, b)
    say(f"one-call attention cfg={cfg} B={B}")
    att, sc, wt, rows = _one_call(r, B, m.cfg.max_len)
    # same plan, same split: bit-identical to the plan-based call
    assert np.array_equal(att.view(np.uint32), r.att.view(np.uint32))
    P = sc.size
    assert np.array_equal(sc.view(np.uint32), r.scores[:P].view(np.uint32))
    assert np.array_equal(wt.view(np.uint32), r.weights[:P].view(np.uint32))
    o = oracle_forward(m, b, want_scores=True)
    tol = FP32_TOL if m.mlp_dtype == "f32" else BF16_TOL
    assert row_rel_err(att, o["att"]) <= tol
    starts = r.packed_start
    L = np.minimum(b.seq_lengths, m.cfg.max_len)
    escale = max(np.max(np.abs(o["scores"][np.arange(m.cfg.max_len)[None, :] < L[:, None]])), 1e-30)
    for s in range(0, B, max(1, B // 512)):
        n = int(L[s])
        assert np.max(np.abs(sc[starts[s]: starts[s] + n] - o["scores"][s, :n]), initial=0) <= tol * escale
        assert np.max(np.abs(wt[starts[s]: starts[s] + n] - o["weights"][s, :n]), initial=0) <= tol
    _, seq = oracle_rows(m, b)
    assert np.array_equal(rows[:, : b.seq_stride], seq)


def test_attn_one_call_max_len_1024():
    """Sequences of up to 1100 positions with max_len 1024 (the largest the
    library takes): a sample spans many 16-position tiles and several waves."""
    cfg = dataclasses.replace(synth.WORKLOADS[1], max_len=1024)
    m = synth.make_model(cfg, bias=True)
    b = synth.make_batch(m, B=64)
    rng = np.random.default_rng(1024)
    L = rng.integers(0, 40, size=64).astype(np.int32)
    L[[0, 5, 9, 20, 33, 63]] = [1100, 1024, 1023, 700, 129, 300]
    L[[3, 40]] = 0
    P = int(L.sum())
    seq = np.empty((3, P), dtype=np.int64)
    for i in range(3):
        seq[i] = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=P, dtype=np.int64)
    b = dataclasses.replace(b, seq_lengths=L, seq_values=seq, seq_stride=P)
    say(f"one-call attention max_len 1024, B=64, P={P}")
    r = Run(m, b)
    att, sc, wt, rows = _one_call(r, 64, 1024)
    assert np.array_equal(att.view(np.uint32), r.att.view(np.uint32))
    o = oracle_forward(m, b, want_scores=True)
    assert row_rel_err(att, o["att"]) <= FP32_TOL
    assert row_rel_err(r.att, o["att"]) <= FP32_TOL
    starts = r.packed_start
    Lc = np.minimum(L, 1024)
    for s in range(64):
        n = int(Lc[s])
        if n == 0:
            assert not att[s].any()
            continue
        assert abs(float(wt[starts[s]: starts[s] + n].sum()) - 1.0) <= 1e-5
        assert np.max(np.abs(wt[starts[s]: starts[s] + n] - o["weights"][s, :n])) <= FP32_TOL
    # rows are resolved (and written) only for the positions read
    _, seqr = oracle_rows(m, b)
    offs = np.concatenate([[0], np.cumsum(L.astype(np.int64))[:-1]])
    read = np.zeros(P, dtype=bool)
    for s in range(64):
        read[offs[s]: offs[s] + Lc[s]] = True
    assert np.array_equal(rows[:, :P][:, read], seqr[:, read])
    assert np.all(rows[:, :P][:, ~read] == -7)
