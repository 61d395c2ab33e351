"""GPU parity of the sparse backward with its AdaGrad step (rec_embbag_adagrad;
"当前现状分析": sparse AdaGrad in the run-config table, an accumulator as large
as the table in §3) against the CPU oracle, table by table and row by row:

  * rows the batch reads: the new weights and the accumulator within the fp32
    tolerance per row (max |gpu - oracle| over the row / max |oracle| over the
    row); from a zero accumulator the accumulator is g^2, so that comparison
    checks the summed gradient itself;
  * rows the batch does not read: weights and accumulator bit for bit as they
    were;
  * the same call twice gives bit-identical tables (every sum has one order).

Cases: the tiny tables with and without sequence gradients, a non-zero
starting accumulator, a row read ten thousand times (its run crosses hundreds
of 16-read chunks), empty bags, one sample, sequence-only and bag-only calls,
and the full Taobao-shaped (B = 8192) and skewed (B = 65536, Zipf ids) batches
at their real table sizes."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, FP32_TOL, row_rel_err, say
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu

SEQ_TABLE = np.array(synth.SEQ_KEYS, np.int32)


def _rows(t):
    return int(t) if isinstance(t, (int, np.integer)) else int(t["rows"])


def _gpu_step(tables, B, values, lengths, offsets, dp, weights, accums, lr, eps, seq):
    """Run rec_embbag_adagrad on copies of weights/accums; `tables` holds row
    counts (direct tables) or generator table dicts (direct or hash).  Returns
    the new (weights, accums) as numpy fp32 lists."""
    T = len(tables)
    tw = [torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(DEV) for w in weights]
    ta = [torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV) for a in accums]
    keep, tabs = [], []
    for t in range(T):
        tb = tables[t]
        if isinstance(tb, dict) and tb["kind"] == "hash":
            k = torch.from_numpy(tb["keys"]).to(DEV)
            d = torch.from_numpy(tb["digests"]).to(DEV)
            keep += [k, d]
            tabs.append(R.adagrad_table(tw[t], ta[t], _rows(tb), R.REC_HASH, k, d))
        else:
            tabs.append(R.adagrad_table(tw[t], ta[t], _rows(tb)))
    nnz = int(values.size)
    v = torch.from_numpy(np.ascontiguousarray(values, np.int64)).to(DEV)
    ln = torch.from_numpy(np.ascontiguousarray(lengths, np.int32)).to(DEV)
    of = torch.from_numpy(np.ascontiguousarray(offsets, np.int64)).to(DEV)
    g = torch.from_numpy(np.ascontiguousarray(dp, np.float32)).to(DEV)
    if seq is None:
        st, sv, gs, stride, P = None, None, None, 0, 0
    else:
        st = seq[0]
        sv = torch.from_numpy(np.ascontiguousarray(seq[1], np.int64)).to(DEV)
        gs = torch.from_numpy(np.ascontiguousarray(seq[2], np.float32)).to(DEV)
        stride, P = int(seq[1].shape[1]), int(seq[2].shape[1])
    wsb = R.rec_embbag_adagrad_workspace_bytes(T, B, nnz, P)
    assert wsb > 0 or nnz + P == 0
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    R.rec_embbag_adagrad(tabs, T, B, v, ln, of, nnz, g, st, sv, stride, P, gs, lr, eps, ws, wsb)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in tw], [x.cpu().numpy() for x in ta]


def _check(rows, B, values, lengths, offsets, dp, weights, accums, lr, eps, seq, tag):
    gw, ga = _gpu_step(rows, B, values, lengths, offsets, dp, weights, accums, lr, eps, seq)
    ow, oa, _, touched = oracle.get().embbag_adagrad(rows, B, values, lengths, offsets, dp,
                                                     weights, accums, lr=lr, eps=eps, seq=seq)
    worst_w = worst_a = 0.0
    for t in range(len(rows)):
        m = touched[t]
        w0 = np.asarray(weights[t], np.float32)
        a0 = np.asarray(accums[t], np.float32)
        # bit for bit, so the NaN of an empty hash slot must stay that NaN
        assert np.array_equal(gw[t][~m].view(np.uint32), w0[~m].view(np.uint32)), (tag, t)
        assert np.array_equal(ga[t][~m].view(np.uint32), a0[~m].view(np.uint32)), (tag, t)
        if not m.any():
            continue
        worst_w = max(worst_w, row_rel_err(gw[t][m], ow[t][m]))
        worst_a = max(worst_a, row_rel_err(ga[t][m], oa[t][m]))
    say(f"  {tag}: touched rows {sum(int(x.sum()) for x in touched)}, "
        f"weights err {worst_w:.2e}, accum err {worst_a:.2e}")
    assert worst_w <= FP32_TOL and worst_a <= FP32_TOL, (tag, worst_w, worst_a)
    return gw, ga


def _offsets(lengths):
    return np.concatenate([[0], np.cumsum(lengths.astype(np.int64))]).astype(np.int64)


def _model_case(cfg_i, B, seed, with_seq=True, cfg=None):
    m = synth.make_model(cfg or synth.WORKLOADS[cfg_i])
    b = synth.make_batch(m, B=B)
    rng = np.random.default_rng(seed)
    dp = rng.standard_normal((b.B, 256)).astype(np.float32)
    P = int(b.seq_lengths.sum())
    seq = (SEQ_TABLE, b.seq_values, rng.standard_normal((3, P, 16)).astype(np.float32)) \
        if with_seq else None
    rows = list(m.tables)
    weights = [np.asarray(t["values"], np.float32) for t in m.tables]
    return m, b, dp, seq, rows, weights


@pytest.mark.parametrize("with_seq", [True, False])
def test_adagrad_tiny(with_seq):
    say(f"adagrad tiny B=256 seq={with_seq}")
    m, b, dp, seq, rows, weights = _model_case(1, 256, 5, with_seq)
    zero = [np.zeros((_rows(r), 16), np.float32) for r in rows]
    _check(rows, b.B, b.values, b.lengths, _offsets(b.lengths)[:-1], dp, weights, zero, 1e-3,
           1e-10, seq, "zero accumulator")
    rng = np.random.default_rng(6)
    acc = [rng.uniform(0.0, 2.0, (_rows(r), 16)).astype(np.float32) for r in rows]
    _check(rows, b.B, b.values, b.lengths, _offsets(b.lengths)[:-1], dp, weights, acc, 0.05,
           1e-10, seq, "random accumulator, lr 0.05")


def test_adagrad_deterministic():
    say("adagrad determinism B=1024")
    m, b, dp, seq, rows, weights = _model_case(1, 1024, 8)
    acc = [np.zeros((_rows(r), 16), np.float32) for r in rows]
    args = (rows, b.B, b.values, b.lengths, _offsets(b.lengths)[:-1], dp, weights, acc, 1e-3,
            1e-10, seq)
    w1, a1 = _gpu_step(*args)
    w2, a2 = _gpu_step(*args)
    for t in range(len(rows)):
        assert np.array_equal(w1[t].view(np.uint32), w2[t].view(np.uint32))
        assert np.array_equal(a1[t].view(np.uint32), a2[t].view(np.uint32))


def _custom(rows, B, lens_hi, seed, P=0, empty_every=0):
    rng = np.random.default_rng(seed)
    T = len(rows)
    lengths = rng.integers(1, lens_hi + 1, size=T * B).astype(np.int32)
    if empty_every:
        lengths[::empty_every] = 0
    nnz = int(lengths.sum())
    values = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=nnz, dtype=np.int64)
    dp = rng.standard_normal((B, T * 16)).astype(np.float32)
    weights = [rng.normal(0, 0.05, (r, 16)).astype(np.float32) for r in rows]
    acc = [np.zeros((r, 16), np.float32) for r in rows]
    seq = None
    if P:
        sv = rng.integers(-1000, 10**9, size=(3, P + 5), dtype=np.int64)
        seq = (np.array([0, T - 1, 0], np.int32), sv, rng.standard_normal((3, P, 16)).astype(np.float32))
    return lengths, values, dp, weights, acc, seq


@pytest.mark.parametrize("rows,B,lens_hi,P,empty_every", [
    ((1, 7), 5000, 3, 0, 0),          # row 0 of table 0 read ~10,000 times
    ((1, 3, 2), 3000, 2, 700, 5),     # hot rows from bags and sequences, empty bags
    ((5,), 1, 1, 0, 0),               # one sample, one id
    ((40, 9), 37, 4, 0, 3),           # ragged: contributions not a multiple of 16
    ((100003, 17), 333, 3, 2049, 0),  # a large table and a small one
])
def test_adagrad_edges(rows, B, lens_hi, P, empty_every):
    say(f"adagrad edges rows={rows} B={B} P={P}")
    lengths, values, dp, weights, acc, seq = _custom(list(rows), B, lens_hi, 11 + B, P, empty_every)
    _check(list(rows), B, values, lengths, _offsets(lengths)[:-1], dp, weights, acc, 1e-3, 1e-10,
           seq, f"rows={rows}")


def test_adagrad_sequence_only_and_bags_only():
    say("adagrad sequence only / bags only")
    rows = [11, 29]
    lengths, values, dp, weights, acc, seq = _custom(rows, 64, 2, 3, P=100)
    zero_len = np.zeros_like(lengths)
    _check(rows, 64, values[:0], zero_len, _offsets(zero_len)[:-1], dp, weights, acc, 1e-3, 1e-10,
           seq, "sequence only")
    _check(rows, 64, values, lengths, _offsets(lengths)[:-1], dp, weights, acc, 1e-3, 1e-10, None,
           "bags only")


@pytest.mark.parametrize("cfg_i,B", [(2, 8192), (4, 65536)])
def test_adagrad_full_size(cfg_i, B):
    say(f"adagrad full size cfg={synth.WORKLOADS[cfg_i].name} B={B}")
    m, b, dp, seq, rows, weights = _model_case(cfg_i, B, 20 + cfg_i)
    zero = [np.zeros((_rows(r), 16), np.float32) for r in rows]
    _check(rows, b.B, b.values, b.lengths, _offsets(b.lengths)[:-1], dp, weights, zero, 1e-3,
           1e-10, seq, f"{synth.WORKLOADS[cfg_i].name}")


HASH_TINY = synth.Config(91, "hash_tiny", 64, tuple(synth.TINY_SIZES), "u123", "geom4", "f32",
                         hash_keys=(0, 1, 2, 3, 4), hash_capacity=3000)


@pytest.mark.parametrize("cfg_i,B", [(0, 300), (5, 8192)])
def test_adagrad_hash(cfg_i, B):
    """Hash tables ("集成 DynamicEmb" §3.2): a hit updates its slot, a miss
    (which read the zero vector) updates nothing, and empty slots keep their
    NaN bits."""
    cfg = HASH_TINY if cfg_i == 0 else synth.WORKLOADS[cfg_i]
    say(f"adagrad hash cfg={cfg.name} B={B}")
    m, b, dp, seq, rows, weights = _model_case(cfg_i, B, 40 + cfg_i, cfg=cfg)
    zero = [np.zeros((_rows(r), 16), np.float32) for r in rows]
    _check(rows, b.B, b.values, b.lengths, _offsets(b.lengths)[:-1], dp, weights, zero, 1e-3,
           1e-10, seq, cfg.name)
