"""GPU parity of the DLRM forward (rec_dlrm_fwd; DLRM essay §2.3 four layers,
§3.2 sum and mean bags, §4.2 widths) against the CPU oracle on the same
seeded inputs: the interaction input z per row (fp32 tolerance), every
interaction output and the logit against the size of their terms, the
probability; the essay's example model (13 dense features, 8 tables, d = 96)
at B = 8192 with all-sum and with mixed sum/mean bags; ragged and one-sample
batches, empty bags, other widths and table counts; the same call twice,
bit-identical; wide models (z and the interaction through memory): the
217-feature shape (216 tables of width 96) on a small batch and, at B = 4096,
on sampled rows, and models wide by their table count or their width."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, FP32_TOL, row_rel_err, say
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu


def _to(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a if dtype is None else a.astype(dtype))).to(DEV)


def _gpu(m, b, want_inter=True):
    cfg = m.cfg
    S, d, B = len(m.tables), cfg.dim, b.B
    F = S + 1
    np_ = F * (F + 1) // 2
    keep = dict(tabs=[_to(t) for t in m.tables],
                w=[_to(getattr(m, k)) for k in ("wb1", "bb1", "wb2", "bb2", "wt1", "bt1", "wt2",
                                                  "bt2", "wt3")])
    mlp = R.dlrm_mlp(cfg.n_dense, d, S, *keep["w"], m.bt3)
    tabs = [R.table(R.REC_DIRECT, t.shape[0], keep["tabs"][i], dim=d) for i, t in enumerate(m.tables)]
    off = np.concatenate([[0], np.cumsum(b.lengths.astype(np.int64))[:-1]])
    z = torch.full((B, F, d), np.nan, dtype=torch.float32, device=DEV)
    inter = torch.full((B, np_), np.nan, dtype=torch.float32, device=DEV) if want_inter else None
    logit = torch.full((B,), np.nan, dtype=torch.float32, device=DEV)
    prob = torch.full((B,), np.nan, dtype=torch.float32, device=DEV)
    vals = _to(b.values if b.values.size else np.zeros(1, np.int64))
    R.rec_dlrm_fwd(mlp, tabs, list(m.modes), B, _to(b.dense), vals, _to(b.lengths), _to(off), z, inter,
                   logit, prob)
    torch.cuda.synchronize()
    out = dict(z=z.cpu().numpy(), logit=logit.cpu().numpy(), prob=prob.cpu().numpy())
    if want_inter:
        out["inter"] = inter.cpu().numpy()
    return out


def _check(m, b, tag):
    say(f"dlrm fwd {tag}: B={b.B} S={len(m.tables)} d={m.cfg.dim} modes={m.modes}")
    got = _gpu(m, b)
    ref = oracle.get().dlrm_fwd(m, b.dense, b.values, b.lengths)
    B, F = b.B, len(m.tables) + 1
    ez = row_rel_err(got["z"].reshape(B * F, -1), ref["z"].reshape(B * F, -1))
    ei = float(np.max(np.abs(got["inter"] - ref["inter"]) / np.maximum(ref["iscale"], 1e-30)))
    el = float(np.max(np.abs(got["logit"] - ref["logit"]) / np.maximum(ref["lscale"], 1e-30)))
    ep = float(np.max(np.abs(got["prob"] - ref["prob"]) / np.maximum(0.25 * ref["lscale"], 1e-30)))
    say(f"  z {ez:.1e}, interaction {ei:.1e}, logit {el:.1e}, prob {ep:.1e}")
    assert ez <= FP32_TOL and ei <= FP32_TOL and el <= FP32_TOL and ep <= FP32_TOL
    return got


@pytest.mark.parametrize("w", [1, 2])
def test_dlrm_fwd_essay_model_B8192(w):
    m = synth.make_dlrm(synth.DLRM_WORKLOADS[w], bias=True)
    b = synth.make_dlrm_batch(m)
    _check(m, b, synth.DLRM_WORKLOADS[w].name)


def test_dlrm_fwd_long_bags():
    """Bags of up to 30 ids (eight rounds of four), a fifth of them empty,
    sum and mean pooling side by side."""
    cfg = dataclasses.replace(synth.DLRM_WORKLOADS[2], bag_max=30,
                              modes=tuple(i % 2 for i in range(len(synth.DLRM_WORKLOADS[2].sizes))))
    m = synth.make_dlrm(cfg, bias=True)
    b = synth.make_dlrm_batch(m, B=200, batch_index=3)
    S = len(m.tables)
    rng = np.random.default_rng(30)
    keep = rng.random((S, 200)) >= 0.2
    L = np.where(keep, b.lengths.reshape(S, 200), 0).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(b.lengths.astype(np.int64))])
    vals = [b.values[starts[i]: starts[i] + L.reshape(-1)[i]] for i in range(S * 200)]
    b2 = dataclasses.replace(b, lengths=L.reshape(-1).copy(), values=np.concatenate(vals))
    assert L.max() > 24
    _check(m, b2, "long bags")


def test_dlrm_fwd_ragged_and_empty_bags():
    m = synth.make_dlrm(synth.DLRM_WORKLOADS[2], bias=True)
    for B in (1, 37, 1000):
        b = synth.make_dlrm_batch(m, B=B, batch_index=B)
        S = len(m.tables)
        L = b.lengths.reshape(S, B).copy()
        L[:, ::3] = 0                             # every third sample: all bags empty
        L[S - 1, 1 % B] = 0
        starts = np.concatenate([[0], np.cumsum(b.lengths.astype(np.int64))])
        vals = []
        for t in range(S):
            for bb in range(B):
                i0 = starts[t * B + bb]
                vals.append(b.values[i0: i0 + L[t, bb]])
        b2 = dataclasses.replace(b, lengths=L.reshape(-1).copy(), values=np.concatenate(vals))
        got = _check(m, b2, f"ragged B={B}")
        for t in range(S):
            assert not got["z"][::3, 1 + t].any()


@pytest.mark.parametrize("sizes,dim,nd,modes", [((7,), 32, 1, (1,)), ((300, 20, 5), 256, 3, (0, 1, 1)),
                                                ((1000,) * 15, 64, 40, (1, 0) * 7 + (1,)),
                                                # five, six and seven float4 per lane of a row
                                                ((100, 12), 160, 4, (0, 1)),
                                                ((400, 30, 7, 3), 192, 2, (0, 1, 0, 1)),
                                                ((250, 9, 60), 224, 5, (1, 1, 0))])
def test_dlrm_fwd_shapes(sizes, dim, nd, modes):
    cfg = dataclasses.replace(synth.DLRM_WORKLOADS[1], sizes=sizes, dim=dim, n_dense=nd, modes=modes)
    m = synth.make_dlrm(cfg, bias=True, emb_scale=8.0)
    b = synth.make_dlrm_batch(m, B=333)
    _check(m, b, f"S={len(sizes)} d={dim}")


def test_dlrm_fwd_deterministic():
    m = synth.make_dlrm(synth.DLRM_WORKLOADS[2], bias=True)
    b = synth.make_dlrm_batch(m, B=2048)
    a, c = _gpu(m, b), _gpu(m, b)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), c[k].view(np.uint32)), k


def _sub_batch(m, b, idx):
    """The samples idx of batch b as a batch of their own (key-major)."""
    S, B = len(m.tables), b.B
    L = b.lengths.reshape(S, B)
    starts = np.concatenate([[0], np.cumsum(b.lengths.astype(np.int64))])
    vals = [b.values[starts[t * B + i]: starts[t * B + i] + L[t, i]] for t in range(S) for i in idx]
    return synth.DlrmBatch(len(idx), b.dense[idx], L[:, idx].reshape(-1).copy(),
                           np.concatenate(vals) if vals else np.zeros(0, np.int64))


def test_dlrm_fwd_wide_217_small():
    cfg = dataclasses.replace(synth.DLRM_WORKLOADS[3], sizes=tuple(20 + 7 * t for t in range(216)),
                              modes=(0, 1) * 108)
    m = synth.make_dlrm(cfg, bias=True)
    b = synth.make_dlrm_batch(m, B=40)
    _check(m, b, "F=217 d=96")


@pytest.mark.parametrize("sizes,dim,modes", [((50,) * 40, 32, (1, 0) * 20),     # 40 tables
                                             ((300,) * 12, 96, (0,) * 12),       # (S+1) * d = 1248
                                             # 255 features: 32,640 pairs, a whole number of the
                                             # top layer's 128-input stages
                                             ((40,) * 254, 32, (0, 1) * 127)])
def test_dlrm_fwd_wide_by_tables_or_width(sizes, dim, modes):
    cfg = dataclasses.replace(synth.DLRM_WORKLOADS[1], sizes=sizes, dim=dim, modes=modes)
    m = synth.make_dlrm(cfg, bias=True, emb_scale=4.0)
    b = synth.make_dlrm_batch(m, B=77)
    _check(m, b, f"wide S={len(sizes)} d={dim}")


def test_dlrm_fwd_wide_217_B4096_sampled():
    """The 217-feature model at B = 4096 (the interaction's measured shape):
    the oracle on 12 samples spread over the batch, compared row by row."""
    cfg = dataclasses.replace(synth.DLRM_WORKLOADS[3], sizes=(500,) * 216)
    m = synth.make_dlrm(cfg, bias=True)
    b = synth.make_dlrm_batch(m)
    got = _gpu(m, b)
    idx = np.array([0, 1, 15, 16, 17, 1000, 2047, 2048, 3000, 4078, 4094, 4095])
    sub = _sub_batch(m, b, idx)
    ref = oracle.get().dlrm_fwd(m, sub.dense, sub.values, sub.lengths)
    F = len(m.tables) + 1
    ez = row_rel_err(got["z"][idx].reshape(len(idx) * F, -1), ref["z"].reshape(len(idx) * F, -1))
    ei = float(np.max(np.abs(got["inter"][idx] - ref["inter"]) / np.maximum(ref["iscale"], 1e-30)))
    el = float(np.max(np.abs(got["logit"][idx] - ref["logit"]) / np.maximum(ref["lscale"], 1e-30)))
    say(f"dlrm fwd F=217 B=4096 sampled: z {ez:.1e}, interaction {ei:.1e}, logit {el:.1e}")
    assert ez <= FP32_TOL and ei <= FP32_TOL and el <= FP32_TOL
    assert np.all(np.isfinite(got["logit"])) and np.all((got["prob"] > 0) & (got["prob"] < 1))
