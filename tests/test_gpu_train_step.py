"""One sparse training step through the library, end to end, against the same
chain through the oracle ("当前现状分析": the run-config table's training
step; §4.4's forward): the forward (pooled bags and DIN attention), the
attention's backward from a given dL/d att, the query gradient added into the
pooled gradient at the query columns (adgroup, cate, brand), and the sparse
AdaGrad step over the bags' and the sequence rows' gradients.  The new tables
match the oracle's per row within the fp32 tolerance, and rows the step does
not read keep their bits."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, FP32_TOL, row_rel_err, say, settle_relu_ties
from sparse_embedding_din_amd import pipeline as PL
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B", [256, 2048])
def test_sparse_train_step(B):
    say(f"train step tiny fp32 B={B}")
    m = synth.make_model(synth.WORKLOADS[1], bias=True)
    b = synth.make_batch(m, B=B)
    rng = np.random.default_rng(B)
    T, P = synth.T, int(b.seq_lengths.sum())
    g_att = rng.standard_normal((B, 48)).astype(np.float32)
    g_pool = rng.standard_normal((B, T * 16)).astype(np.float32)   # from the deep tower
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731

    # GPU: forward, attention backward, AdaGrad
    tabs = PL.DeviceTables(m.tables, DEV)
    fwd = PL.SparseDinForward(tabs, PL.DeviceMLP(m, DEV), B, m.cfg.max_len, DEV)
    db = PL.DeviceBatch(b, DEV)
    pooled, att = fwd.run(db)
    seq_off = np.concatenate([[0], np.cumsum(b.seq_lengths.astype(np.int64))[:-1]])
    mlp = PL.DeviceMLP(m, DEV, packed=False)
    gq = torch.empty(B, 48, dtype=torch.float32, device=DEV)
    gs = torch.empty(3, P, 16, dtype=torch.float32, device=DEV)
    wsb = R.rec_din_attn_bwd_workspace_bytes(P, False)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    R.rec_din_attn_bwd(tabs.array(list(synth.SEQ_KEYS)), db.seq_values, P, to(seq_off),
                       db.seq_lengths, m.cfg.max_len, B, pooled, T * 16, synth.QUERY_COL, mlp.desc,
                       to(g_att), gq, gs, workspace=ws, workspace_bytes=wsb)
    gp = to(g_pool)
    for k, c in enumerate(synth.QUERY_COL):
        gp[:, c:c + 16] += gq[:, 16 * k:16 * k + 16]
    w = [torch.from_numpy(np.asarray(t["values"], np.float32)).to(DEV) for t in m.tables]
    acc = [torch.zeros(int(t["rows"]), 16, dtype=torch.float32, device=DEV) for t in m.tables]
    atabs = [R.adagrad_table(w[t], acc[t], int(m.tables[t]["rows"])) for t in range(T)]
    off = np.concatenate([[0], np.cumsum(b.lengths.astype(np.int64))[:-1]])
    wsa = R.rec_embbag_adagrad_workspace_bytes(T, B, b.values.size, P)
    wa = torch.empty(wsa, dtype=torch.uint8, device=DEV)
    R.rec_embbag_adagrad(atabs, T, B, db.values, db.lengths, to(off), b.values.size, gp,
                         synth.SEQ_KEYS, db.seq_values, P, P, gs, 1e-3, 1e-10, wa, wsa)
    torch.cuda.synchronize()
    gs_gpu = gs.cpu().numpy()

    # oracle: the same chain in fp64
    orc = oracle.get()
    o = oracle.forward(m, b)
    q = o["query"]
    ob = orc.din_bwd([m.tables[k] for k in synth.SEQ_KEYS], b.seq_values, P, seq_off,
                     b.seq_lengths, m.cfg.max_len, q, m.w1, m.b1, m.w2, m.b2, m.w3, m.b3, g_att,
                     gates=True)
    # a first-layer ReLU gate within rounding of zero may go either way
    settle_relu_ties({"gs": gs_gpu}, ob, m, b.seq_values, seq_off, b.seq_lengths, m.cfg.max_len,
                     q, P)
    og_pool = g_pool.astype(np.float64)
    for k, c in enumerate(synth.QUERY_COL):
        og_pool[:, c:c + 16] += ob["gq"][:, 16 * k:16 * k + 16]
    ogs = ob["gs"].reshape(P, 3, 16).transpose(1, 0, 2)
    ow, oacc, _, touched = orc.embbag_adagrad(
        m.tables, B, b.values, b.lengths, off, og_pool.astype(np.float32),
        [t["values"] for t in m.tables], [np.zeros((int(t["rows"]), 16)) for t in m.tables],
        seq=(np.array(synth.SEQ_KEYS, np.int32), b.seq_values, ogs.astype(np.float32)))
    worst_w = worst_a = 0.0
    for t in range(T):
        k = touched[t]
        gw = w[t].cpu().numpy()
        ga = acc[t].cpu().numpy()
        w0 = np.asarray(m.tables[t]["values"], np.float32)
        assert np.array_equal(gw[~k].view(np.uint32), w0[~k].view(np.uint32)), t
        assert not ga[~k].any(), t
        if k.any():
            worst_w = max(worst_w, row_rel_err(gw[k], ow[t][k]))
            worst_a = max(worst_a, row_rel_err(ga[k], oacc[t][k]))
    say(f"  weights err {worst_w:.2e}, accumulator err {worst_a:.2e}")
    assert worst_w <= FP32_TOL and worst_a <= FP32_TOL, (worst_w, worst_a)
