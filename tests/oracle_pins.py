"""Pins for the CPU oracle: checks of it against things other than itself.

Each pin takes an `oracle.Oracle` instance and raises AssertionError when the
oracle disagrees with what the pages and the mathematics fix:

  * library routines that compute the same thing another way:
      numpy cumsum (offsets), Python/numpy floor modulo (direct rows), a Python
      dict over the slots (hash hit/miss), torch.nn.functional.embedding_bag
      in fp64 (sum pooling), and the pages' own PADDED formulation of DIN
      attention written with torch fp64 library ops ("MultiTowerDIN：当前现状分析"
      §4.2/§4.4: pad to [B,100,48], cat, MLP on every position, mask, softmax,
      bmm) against the oracle's padding-free loop;
  * closed forms and invariants: one-position sequence -> weight 1 and output
    equal to that position exactly; zero score weights -> the mean of the
    sequence; identical positions -> that position; softmax weights sum to 1;
    a shift of the score bias leaves weights and output unchanged; permuting a
    sample's positions permutes its weights and leaves its output unchanged;
    a single-id bag pools to that row exactly; a hash miss adds exact zeros.

They are plain functions so that tests/test_oracle_mutants.py can run every
pin against deliberately broken copies of the oracle and check that each
planted mistake is caught.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import synth

TINY_HASH = synth.Config(91, "hash_tiny", 64, tuple(synth.TINY_SIZES), "u123", "geom4", "f32",
                         hash_keys=(0, 1, 2, 3, 4), hash_capacity=3000)


# ----------------------------------------------------------------------------
# independent helpers (library routines / language semantics)
def py_rows(tab: dict, raw: np.ndarray) -> np.ndarray:
    raw = np.asarray(raw, dtype=np.int64)
    if tab["kind"] == "direct":
        return np.mod(raw, np.int64(tab["rows"]))           # numpy: sign of divisor (floor)
    d = {int(k): s for s, k in enumerate(tab["keys"].tolist()) if k != synth.EMPTY_KEY}
    return np.array([d.get(int(r), -1) for r in raw.tolist()], dtype=np.int64)


def torch_pooled(model, batch) -> np.ndarray:
    """Per-table torch embedding_bag(mode='sum') in fp64; hash misses index an
    appended all-zero row."""
    B = batch.B
    lengths = batch.lengths.reshape(synth.T, B)
    starts = np.concatenate([[0], np.cumsum(batch.lengths)])
    out = []
    for k in range(synth.T):
        tab = model.tables[k]
        lo, hi = starts[k * B], starts[(k + 1) * B]
        rows = py_rows(tab, batch.values[lo:hi])
        w = np.asarray(tab["values"], dtype=np.float64)
        w = np.concatenate([w, np.zeros((1, 16))], axis=0)
        rows = np.where(rows < 0, w.shape[0] - 1, rows)
        bag_off = np.concatenate([[0], np.cumsum(lengths[k])[:-1]])
        t = F.embedding_bag(torch.from_numpy(rows), torch.from_numpy(np.nan_to_num(w)),
                            torch.from_numpy(bag_off.astype(np.int64)), mode="sum")
        out.append(t.numpy())
    return np.concatenate(out, axis=1)


def torch_padded_din(model, batch, query, seq_offsets, max_len, pad_to=100):
    """The pages' padded DIN: [B,pad,48] zero beyond the real length, cat
    [q, s, q-s, q*s], the MLP on every position, mask to -inf, softmax, bmm."""
    B = batch.B
    S = np.zeros((B, pad_to, 48))
    L = np.minimum(batch.seq_lengths.astype(np.int64), max_len)
    for i, k in enumerate(synth.SEQ_KEYS):
        tab = model.tables[k]
        w = np.asarray(tab["values"], dtype=np.float64)
        for b in range(B):
            n = int(L[b])
            if n == 0:
                continue
            ids = batch.seq_values[i, seq_offsets[b]: seq_offsets[b] + n]
            r = py_rows(tab, ids)
            S[b, :n, 16 * i:16 * i + 16] = np.where(r[:, None] < 0, 0.0, w[np.maximum(r, 0)])
    St = torch.from_numpy(S)
    Q = torch.from_numpy(np.asarray(query, np.float64))[:, None, :].expand(B, pad_to, 48)
    X = torch.cat([Q, St, Q - St, Q * St], dim=-1)
    h1 = torch.relu(F.linear(X, torch.from_numpy(model.w1.astype(np.float64)),
                             torch.from_numpy(model.b1.astype(np.float64))))
    h2 = torch.relu(F.linear(h1, torch.from_numpy(model.w2.astype(np.float64)),
                             torch.from_numpy(model.b2.astype(np.float64))))
    e = F.linear(h2, torch.from_numpy(model.w3.astype(np.float64))[None, :],
                 torch.tensor([float(model.b3)], dtype=torch.float64)).squeeze(-1)
    mask = torch.arange(pad_to)[None, :] < torch.from_numpy(L)[:, None]
    p = torch.softmax(e.masked_fill(~mask, float("-inf")), dim=-1)
    p = torch.where(mask, p, torch.zeros_like(p))          # empty sample: no weights
    att = torch.bmm(p[:, None, :], St).squeeze(1)
    return att.numpy(), e.numpy(), p.numpy(), S


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def _seq_offsets(batch):
    return np.concatenate([[0], np.cumsum(batch.seq_lengths)])[:-1].astype(np.int64)


def _query_from(pooled):
    return np.concatenate([pooled[:, c:c + 16] for c in synth.QUERY_COL], axis=1)


def _tiny(bias=True, B=64, emb_std=0.05, w3_scale=1.0):
    m = synth.make_model(synth.WORKLOADS[1], bias=bias, emb_std=emb_std, w3_scale=w3_scale)
    b = synth.make_batch(m, B=B)
    return m, b


# ----------------------------------------------------------------------------
def pin_offsets(orc):
    rng = np.random.default_rng(1)
    for n in (0, 1, 7, 1000):
        L = rng.integers(0, 5, size=n).astype(np.int32)
        o = orc.lengths_to_offsets(L)
        assert o.shape == (n + 1,)
        assert o[0] == 0
        assert np.array_equal(o[1:], np.cumsum(L.astype(np.int64)))
        assert np.array_equal(np.diff(o), L)


def pin_floor_mod(orc):
    i64 = np.iinfo(np.int64)
    Ns = [1, 2, 3, 5, 98, 101, 1141730, 846812, 2**31 - 1, 2**32 + 15, 2**62 + 3, i64.max]
    raws = [0, 1, -1, 2, -2, 100, -100, 101, -101, 1141729, 1141730, -1141730, -1141731,
            i64.max, i64.min, i64.min + 1, i64.max - 1, 2**32, -(2**32), 2**62, -(2**62)]
    rng = np.random.default_rng(2)
    raws += [int(x) for x in rng.integers(i64.min, i64.max, size=200, dtype=np.int64)]
    for N in Ns:
        for r in raws + [N - 1, N, -N, N + 1, -N - 1] if N < i64.max else raws:
            if not (i64.min <= r <= i64.max):
                continue
            got = orc.floor_mod(r, N)
            assert got == r % N, (r, N, got)            # Python: floor semantics
            assert 0 <= got < N
            assert (r - got) % N == 0                    # r == got (mod N), big ints


def pin_hash(orc):
    m = synth.make_model(TINY_HASH)
    for k in TINY_HASH.hash_keys:
        tab = m.tables[k]
        stored = tab["stored"]
        rng = np.random.default_rng(3 + k)
        misses = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=300,
                              dtype=np.int64)
        q = np.concatenate([stored[:500], misses, [synth.EMPTY_KEY, 0, 1]])
        got = orc.resolve(tab, q)
        ref = py_rows(tab, q)
        assert np.array_equal(got, ref)
        hit = got >= 0
        assert np.array_equal(tab["keys"][got[hit]], q[hit])
        assert np.all(hit[:500])
        assert got[-3] == -1                              # the empty marker is never a key


def pin_embbag_direct(orc):
    m, b = _tiny()
    # put empty bags in (a deep feature with no id for some samples)
    L = b.lengths.reshape(synth.T, b.B).copy()
    L[3, ::5] = 0
    L[0, 1] = 0
    vals = []
    starts = np.concatenate([[0], np.cumsum(b.lengths)])
    for k in range(synth.T):
        for bb in range(b.B):
            i = k * b.B + bb
            vals.append(b.values[starts[i]: starts[i] + L[k, bb]])
    b.lengths = L.reshape(-1).astype(np.int32)
    b.values = np.concatenate(vals).astype(np.int64)
    off = orc.lengths_to_offsets(b.lengths)
    got = orc.embbag(m.tables, b.B, b.values, b.lengths, off)
    ref = torch_pooled(m, b)
    assert got.shape == (b.B, 256)
    assert _rel(got, ref) < 1e-14
    assert np.all(got[::5, 48:64] == 0.0)
    # a single-id bag pools to its row exactly (price bags hold one id)
    price = b.values[off[15 * b.B]: off[16 * b.B]]
    assert np.array_equal(got[:, 240:256], m.tables[15]["values"][np.mod(price, 101)].astype(np.float64))


def pin_embbag_hash(orc):
    m = synth.make_model(TINY_HASH)
    b = synth.make_batch(m, B=TINY_HASH.B)
    off = orc.lengths_to_offsets(b.lengths)
    got = orc.embbag(m.tables, b.B, b.values, b.lengths, off)
    ref = torch_pooled(m, b)
    assert np.all(np.isfinite(got))                       # NaN-poisoned empty slots never read
    assert _rel(got, ref) < 1e-14
    # linearity: dropping the missed ids changes nothing
    lo, hi = off[0], off[b.B]
    rows = py_rows(m.tables[0], b.values[lo:hi])
    assert (rows < 0).any()


def _din_case(orc, m, b, max_len=100, pad_to=100):
    off = orc.lengths_to_offsets(b.lengths)
    pooled = orc.embbag(m.tables, b.B, b.values, b.lengths, off)
    q = _query_from(pooled)
    soff = _seq_offsets(b)
    seq_tabs = [m.tables[k] for k in synth.SEQ_KEYS]
    att, sc, wt = orc.din(seq_tabs, b.seq_values, b.seq_stride, soff, b.seq_lengths, max_len,
                          q, m.w1, m.b1, m.w2, m.b2, m.w3, m.b3, want_scores=True)
    return att, sc, wt, q, soff


def pin_din_vs_padded(orc):
    for emb_std, w3s in ((0.05, 1.0), (1.0, 20.0)):      # near-uniform and peaky softmax
        m, b = _tiny(emb_std=emb_std, w3_scale=w3s)
        b.seq_lengths[3] = 0                               # an empty click sequence
        b.seq_lengths[5] = 1
        att, sc, wt, q, soff = _din_case(orc, m, b)
        ratt, re_, rp, _ = torch_padded_din(m, b, q, soff, 100)
        assert _rel(att, ratt) < 1e-12
        L = np.minimum(b.seq_lengths, 100)
        for bb in range(b.B):
            n = int(L[bb])
            assert _rel(sc[bb, :n], re_[bb, :n]) < 1e-12
            assert _rel(wt[bb, :n], rp[bb, :n]) < 1e-12
            assert np.all(wt[bb, n:] == 0.0)
        assert np.all(att[3] == 0.0)
        if w3s > 1.0:
            assert wt.max() > 0.9                          # the peaky case really is peaky
    # truncation to max_len: the padded form with only the first 3 positions
    m, b = _tiny()
    att, sc, wt, q, soff = _din_case(orc, m, b, max_len=3)
    ratt, _, _, _ = torch_padded_din(m, b, q, soff, 3, pad_to=3)
    assert _rel(att, ratt) < 1e-12


def pin_din_closed_forms(orc):
    m, b = _tiny()
    orig = b.seq_lengths.copy()
    starts = np.concatenate([[0], np.cumsum(orig)])
    L = np.minimum(orig, 6).astype(np.int32)
    L[0] = 1
    b.seq_values = np.ascontiguousarray(np.concatenate(
        [b.seq_values[:, starts[i]: starts[i] + L[i]] for i in range(b.B)], axis=1))
    b.seq_lengths = L
    b.seq_stride = b.seq_values.shape[1]
    att, sc, wt, q, soff = _din_case(orc, m, b)
    _, _, _, S = torch_padded_din(m, b, q, soff, 100)
    # one position: weight exactly 1, output exactly that position
    assert wt[0, 0] == 1.0 and np.array_equal(att[0], S[0, 0])
    # weights sum to one over the valid positions
    L = b.seq_lengths
    for bb in range(b.B):
        assert abs(wt[bb, :L[bb]].sum() - 1.0) < 1e-12
    # score bias shift: weights and output unchanged, scores shift by the same amount
    seq_tabs = [m.tables[k] for k in synth.SEQ_KEYS]
    att2, sc2, wt2 = orc.din(seq_tabs, b.seq_values, b.seq_stride, soff, L, 100, q, m.w1, m.b1,
                             m.w2, m.b2, m.w3, m.b3 + 3.25, want_scores=True)
    assert _rel(att2, att) < 1e-12 and _rel(wt2, wt) < 1e-12
    for bb in range(b.B):
        assert np.allclose(sc2[bb, :L[bb]] - sc[bb, :L[bb]], 3.25, atol=1e-12, rtol=0)
    # zero score weights: uniform weights, output = mean of the positions
    att3 = orc.din(seq_tabs, b.seq_values, b.seq_stride, soff, L, 100, q, m.w1, m.b1, m.w2,
                   m.b2, np.zeros(64), -0.7)
    for bb in range(b.B):
        assert _rel(att3[bb], S[bb, :L[bb]].mean(axis=0)) < 1e-13
    # permuting a sample's positions: output unchanged, weights permuted
    rng = np.random.default_rng(5)
    perm_seq = b.seq_values.copy()
    perms = []
    for bb in range(b.B):
        p = rng.permutation(int(L[bb]))
        perms.append(p)
        perm_seq[:, soff[bb]: soff[bb] + L[bb]] = b.seq_values[:, soff[bb] + p]
    att4, sc4, wt4 = orc.din(seq_tabs, perm_seq, b.seq_stride, soff, L, 100, q, m.w1, m.b1,
                             m.w2, m.b2, m.w3, m.b3, want_scores=True)
    assert _rel(att4, att) < 1e-12
    for bb in range(b.B):
        assert _rel(wt4[bb, :L[bb]], wt[bb, perms[bb]]) < 1e-12
    # identical positions: the output is that position
    same = b.seq_values.copy()
    for bb in range(b.B):
        same[:, soff[bb]: soff[bb] + L[bb]] = b.seq_values[:, soff[bb]: soff[bb] + 1]
    att5 = orc.din(seq_tabs, same, b.seq_stride, soff, L, 100, q, m.w1, m.b1, m.w2, m.b2,
                   m.w3, m.b3)
    for bb in range(b.B):
        assert _rel(att5[bb], S[bb, 0]) < 1e-14
    # sample independence: evaluating a subset gives the same rows
    sub = np.array([7, 2, 40], dtype=np.int64)
    att6 = orc.din(seq_tabs, b.seq_values, b.seq_stride, soff, L, 100, q[sub], m.w1, m.b1,
                   m.w2, m.b2, m.w3, m.b3, samples=sub)
    assert np.array_equal(att6, att[sub])


def pin_din_hash(orc):
    """Sequence rows through hash tables: misses contribute exact zero rows."""
    m = synth.make_model(TINY_HASH, bias=True)
    b = synth.make_batch(m, B=TINY_HASH.B)
    att, sc, wt, q, soff = _din_case(orc, m, b)
    ratt, re_, rp, _ = torch_padded_din(m, b, q, soff, 100)
    assert np.all(np.isfinite(att))
    assert _rel(att, ratt) < 1e-12


# ----------------------------------------------------------------------------
# Deep tower + final MLP ("MultiTowerDIN：当前现状分析" §4.4 compute graph).
def _sparse_towers(rng, ns):
    """A tower whose every layer is a sparse integer-ish map, so each output
    has a closed form in index arithmetic: every row of every matrix has one
    or two non-zeros, biases are chosen so that the ReLUs clip some units."""
    tw = synth.Towers(*(None,) * 10)
    x = rng.uniform(0.0, 1.0, (ns, 300))             # row stride 300 > 256
    x[:, 256:] = -7.0                                # columns past 256 must not be read
    att = rng.uniform(-1.0, 1.0, (ns, 48))
    p1 = rng.permutation(256)
    tw.wd1 = np.zeros((512, 256)); tw.bd1 = np.zeros(512)
    tw.wd1[np.arange(256), p1] = 1.0                 # d1[r] = x[p1[r]]
    tw.wd1[256 + np.arange(256), p1] = -1.0          # d1[256 + r] = relu(0.5 - x[p1[r]])
    tw.bd1[256:] = 0.5
    p2 = rng.permutation(512)
    a2, c2 = p2[:256], p2[256:]
    tw.wd2 = np.zeros((256, 512)); tw.bd2 = np.full(256, 0.3)
    tw.wd2[np.arange(256), a2] = 1.0                 # d2[r] = relu(0.3 + d1[a2] - 2 d1[c2])
    tw.wd2[np.arange(256), c2] = -2.0
    a3 = rng.permutation(256)[:128]
    tw.wd3 = np.zeros((128, 256)); tw.bd3 = np.full(128, -0.1)
    tw.wd3[np.arange(128), a3] = 1.5                 # d3[r] = relu(1.5 d2[a3] - 0.1)
    pf = rng.permutation(176)
    af = np.concatenate([pf[:40], 128 + rng.permutation(48)[:24]])  # 24 rows start in att
    cf = rng.permutation(176)[:64]
    cf = np.where(cf == af, (cf + 1) % 176, cf)
    tw.wf = np.zeros((64, 176)); tw.bf = np.full(64, 0.05)
    tw.wf[np.arange(64), af] = 1.0                   # f[r] = relu(0.05 + z[af] - z[cf])
    tw.wf[np.arange(64), cf] = -1.0
    tw.wo = rng.uniform(-1.0, 1.0, 64); tw.bo = 0.25
    d1 = np.concatenate([x[:, p1], np.maximum(0.5 - x[:, p1], 0.0)], axis=1)
    d2 = np.maximum(0.3 + d1[:, a2] - 2.0 * d1[:, c2], 0.0)
    d3 = np.maximum(1.5 * d2[:, a3] - 0.1, 0.0)
    z = np.concatenate([d3, att], axis=1)
    f = np.maximum(0.05 + z[:, af] - z[:, cf], 0.0)
    logit = (f * tw.wo[None, :]).sum(axis=1) + tw.bo
    tw.expected_scale = np.abs(f * tw.wo[None, :]).sum(axis=1) + abs(tw.bo)
    return tw, x, att, d3, logit


def pin_towers_closed_forms(orc):
    rng = np.random.default_rng(11)
    tw, x, att, d3, logit = _sparse_towers(rng, 40)
    assert np.mean(d3 == 0.0) > 0.05 and np.mean(d3 > 0.0) > 0.3   # the ReLUs clip
    deep, lg, pr, sc = orc.towers(x, att, tw, want_scale=True)
    assert _rel(sc, tw.expected_scale) < 1e-14
    assert _rel(deep, d3) < 1e-14
    assert _rel(lg, logit) < 1e-14
    assert np.max(np.abs(lg - logit)) < 1e-13
    # the logit goes through the logistic function: exact special values
    z = synth.Towers(np.zeros((512, 256)), np.zeros(512), np.zeros((256, 512)), np.zeros(256),
                     np.zeros((128, 256)), np.zeros(128), np.zeros((64, 176)), np.zeros(64),
                     np.ones(64), 0.0)
    for bo, want in ((0.0, 0.5), (np.log(3.0), 0.75), (-np.log(3.0), 0.25), (np.log(9.0), 0.9)):
        z.bo = float(bo)
        _, lg0, pr0 = orc.towers(x[:3], att[:3], z)
        assert np.all(lg0 == bo) and np.all(np.abs(pr0 - want) < 1e-15), (bo, pr0)
    # zero weights: every layer passes only its ReLU'd bias
    z.bd1 = rng.uniform(-1, 1, 512); z.bd3 = rng.uniform(-1, 1, 128)
    z.bf = rng.uniform(-1, 1, 64); z.wo = rng.uniform(-1, 1, 64); z.bo = 0.125
    deep0, lg0, _ = orc.towers(x[:2], att[:2], z)
    assert np.array_equal(deep0, np.broadcast_to(np.maximum(z.bd3, 0.0), (2, 128)))
    assert np.all(np.abs(lg0 - (0.125 + np.dot(z.wo, np.maximum(z.bf, 0.0)))) < 1e-15)


def pin_towers_library(orc):
    """torch fp64 Linear/ReLU/sigmoid on the generator's weights; positive
    homogeneity without biases; rows are independent."""
    m, b = _tiny(bias=True, B=48, emb_std=1.0)
    tw = m.towers
    rng = np.random.default_rng(5)
    x = rng.standard_normal((48, 256)) * 0.5
    att = rng.standard_normal((48, 48)) * 0.5
    deep, lg, pr = orc.towers(x, att, tw)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    h = F.relu(F.linear(t(x), t(tw.wd1), t(tw.bd1)))
    h = F.relu(F.linear(h, t(tw.wd2), t(tw.bd2)))
    d3 = F.relu(F.linear(h, t(tw.wd3), t(tw.bd3)))
    f = F.relu(F.linear(torch.cat([d3, t(att)], dim=1), t(tw.wf), t(tw.bf)))
    rl = F.linear(f, t(tw.wo)[None, :]).squeeze(1) + tw.bo
    assert _rel(deep, d3.numpy()) < 1e-12
    assert _rel(lg, rl.numpy()) < 1e-12
    assert np.max(np.abs(pr - torch.sigmoid(rl).numpy())) < 1e-14
    # no biases: f(2x) = 2 f(x) (ReLU nets are positively homogeneous)
    nb = synth.Towers(tw.wd1, np.zeros(512), tw.wd2, np.zeros(256), tw.wd3, np.zeros(128),
                      tw.wf, np.zeros(64), tw.wo, 0.0)
    d_a, l_a, _ = orc.towers(x, att, nb)
    d_b, l_b, _ = orc.towers(2.0 * x, 2.0 * att, nb)
    assert _rel(d_b, 2.0 * d_a) < 1e-14 and _rel(l_b, 2.0 * l_a) < 1e-14
    assert _rel(d_a, deep) > 1e-3                      # the biases do matter
    sub = np.array([9, 0, 31])
    d_s, l_s, _ = orc.towers(x[sub], att[sub], tw)
    assert np.array_equal(d_s, deep[sub]) and np.array_equal(l_s, lg[sub])


def _distinct_keys(rng, n):
    I64 = np.iinfo(np.int64)
    k = np.unique(rng.integers(I64.min, I64.max, size=2 * n + 8, dtype=np.int64))
    return rng.permutation(k[k != synth.EMPTY_KEY])[:n]


def _stored_map(tab):
    occ = np.nonzero(tab["keys"] != synth.EMPTY_KEY)[0]
    return {int(tab["keys"][s]): tab["values"][s].tobytes() for s in occ}


def pin_hash_insert(orc):
    """The insert side ("集成 DynamicEmb" §6.4 rebuild, §4.2 scores) against the
    generator's own implementation of the table convention and its
    round-based builder, dict semantics for insert-or-assign, and planted
    breaks of the convention."""
    rng = np.random.default_rng(2024)
    vals = lambda n: rng.standard_normal((n, 16)).astype(np.float32)
    # (1) a key into an empty table sits on its home slot with its digest, as
    # the generator computes them; one key has a zero low byte (digest 1)
    zero_low = next(k for k in range(1, 10**6)
                    if int(synth.splitmix64_mix(np.array([k], np.int64))[0]) & 0xFF == 0)
    keys1 = np.append(_distinct_keys(rng, 12), zero_low)
    for cap in (1, 2, 7, 1000, 300000):
        h = synth.splitmix64_mix(keys1)
        for k, home, dig in zip(keys1, synth.home_slot(h, cap), synth.digest_of(h)):
            t = orc.empty_hash_table(cap)
            assert orc.hash_insert(t, np.array([k]), vals(1))[0] == home
            assert t["keys"][home] == k and t["digests"][home] == dig
    # (2) key by key against the generator's builder: the same stored map,
    # every key where its slot says, both tables valid
    cap, n = 3001, 2400
    keys, v = _distinct_keys(rng, n), vals(n)
    t = orc.empty_hash_table(cap)
    slots = orc.hash_insert(t, keys, v)
    g = synth.build_hash_table(keys, v, cap)
    assert np.all(slots >= 0) and np.array_equal(t["keys"][slots], keys)
    assert orc.hash_check(t["keys"], t["digests"]) == 0
    assert orc.hash_check(g["keys"], g["digests"]) == 0
    assert _stored_map(t) == _stored_map(g)
    # (3) insert-or-assign is a dict update: old keys keep their slots and
    # take the new values, new keys are added; LFU counts, STEP overwrites
    expect = {int(k): x.tobytes() for k, x in zip(keys, v)}
    upd, fresh = rng.choice(keys, 500, replace=False), _distinct_keys(rng, 200)
    fresh = fresh[~np.isin(fresh, keys)][:100]
    nu, nf = vals(upd.size), vals(fresh.size)
    s2 = orc.hash_insert(t, np.concatenate([upd, fresh]), np.concatenate([nu, nf]),
                         mode=orc.SCORE_LFU)
    expect.update({int(k): x.tobytes() for k, x in zip(upd, nu)})
    expect.update({int(k): x.tobytes() for k, x in zip(fresh, nf)})
    assert _stored_map(t) == expect
    where = {int(k): int(sl) for k, sl in zip(keys, slots)}
    assert s2[: upd.size].tolist() == [where[int(k)] for k in upd]
    assert orc.hash_check(t["keys"], t["digests"]) == 0
    assert np.all(t["scores"][s2] == 1)
    orc.hash_insert(t, upd[:50], nu[:50], mode=orc.SCORE_LFU)
    assert np.all(t["scores"][s2[:50]] == 2) and np.all(t["scores"][s2[50:]] == 1)
    orc.hash_insert(t, upd[:10], nu[:10], mode=orc.SCORE_STEP, step=77)
    assert np.all(t["scores"][s2[:10]] == 77) and np.all(t["scores"][s2[10:50]] == 2)
    # (4) a full table stores nothing more (NO_EVICTION) but still assigns
    t4 = orc.empty_hash_table(16)
    k4 = _distinct_keys(rng, 20)
    s4 = orc.hash_insert(t4, k4, vals(20))
    assert np.all(s4[:16] >= 0) and np.all(s4[16:] == -1)
    assert set(t4["keys"].tolist()) == set(k4[:16].tolist())
    before = t4["keys"].copy()
    assert orc.hash_insert(t4, k4[3:4], vals(1))[0] == s4[3]
    assert np.array_equal(t4["keys"], before) and orc.hash_check(t4["keys"], t4["digests"]) == 0
    # (5) the probe wraps: two keys homed on the last slot take it and slot 0
    cand = np.arange(1, 5000, dtype=np.int64)
    last = cand[synth.home_slot(synth.splitmix64_mix(cand), 8) == 7][:2]
    t5 = orc.empty_hash_table(8)
    assert list(orc.hash_insert(t5, last, vals(2))) == [7, 0]
    # (6) the empty marker is never stored
    t6 = orc.empty_hash_table(5)
    assert orc.hash_insert(t6, np.array([synth.EMPTY_KEY]), vals(1))[0] == -2
    assert np.all(t6["keys"] == synth.EMPTY_KEY)
    # (7) the check flags each kind of break, one at a time
    occ = np.nonzero(g["keys"] != synth.EMPTY_KEY)[0]
    homes = synth.home_slot(synth.splitmix64_mix(g["keys"][occ]), cap)
    bad = g["digests"].copy()
    bad[occ[0]] ^= 0x80
    assert orc.hash_check(g["keys"], bad) == 1                        # wrong digest
    moved = occ[np.nonzero(homes != occ)[0][0]]                       # a key off its home
    gk, gd = g["keys"].copy(), g["digests"].copy()
    gk[moved - 1], gd[moved - 1] = synth.EMPTY_KEY, 0                 # hole on its path
    assert orc.hash_check(gk, gd) >= 1
    gd2 = g["digests"].copy()
    gd2[np.nonzero(g["keys"] == synth.EMPTY_KEY)[0][0]] = 5
    assert orc.hash_check(g["keys"], gd2) == 1                        # digest on an empty slot
    e = occ[0]                                                        # first empty slot after
    while g["keys"][e] != synth.EMPTY_KEY:                            # key occ[0]'s cluster
        e = (e + 1) % cap
    gk3, gd3 = g["keys"].copy(), g["digests"].copy()
    gk3[e], gd3[e] = g["keys"][occ[0]], g["digests"][occ[0]]          # a reachable second copy
    assert orc.hash_check(gk3, gd3) == 1


def pin_dlrm_interact(orc):
    """DLRM dot-product interaction (DLRM essay §2.3, §4.2) against torch fp64
    bmm with triu_indices (row-major, diagonal included), and closed forms:
    orthonormal rows give the identity's triangle, F copies of one vector give
    |v|^2 everywhere, a power-of-two scale c scales every entry by c^2 exactly,
    and F = 1 gives the squared norm."""
    rng = np.random.default_rng(77)
    for B, F, d in ((3, 1, 4), (2, 5, 8), (4, 27, 96), (1, 217, 96)):
        z = rng.standard_normal((B, F, d)).astype(np.float32)
        got, sc = orc.dlrm_interact(z, want_scale=True)
        assert got.shape == (B, F * (F + 1) // 2)
        zt = torch.from_numpy(z).double()
        gram = torch.bmm(zt, zt.transpose(1, 2).contiguous())
        iu = torch.triu_indices(F, F)
        ref = gram[:, iu[0], iu[1]].numpy()
        assert np.max(np.abs(got - ref) / np.maximum(sc, 1e-300)) < 1e-13
        absg = torch.bmm(zt.abs(), zt.abs().transpose(1, 2).contiguous())[:, iu[0], iu[1]].numpy()
        assert np.allclose(sc, absg, rtol=1e-12, atol=0)
        z4 = (z * 4.0).astype(np.float32)
        assert np.array_equal(orc.dlrm_interact(z4), 16.0 * got)
    F, d = 6, 8
    eye = np.zeros((1, F, d), np.float32)
    eye[0, np.arange(F), np.arange(F)] = 1.0
    iu = np.triu_indices(F)
    assert np.array_equal(orc.dlrm_interact(eye)[0], (iu[0] == iu[1]).astype(np.float64))
    v = rng.standard_normal(d).astype(np.float32)
    same = np.tile(v, (1, F, 1))
    n2 = float(np.dot(v.astype(np.float64), v.astype(np.float64)))
    assert np.allclose(orc.dlrm_interact(same)[0], n2, rtol=1e-15, atol=0)
    assert np.allclose(orc.dlrm_interact(v.reshape(1, 1, d))[0], [n2], rtol=1e-15, atol=0)


def _torch_sparse_step(m, b, dpooled, seq, weights, opt_state, lr, eps):
    """The pages' training step for the tables ("当前现状分析" run-config table:
    sparse AdaGrad) written with torch library routines in fp64: per-table
    embedding_bag(mode='sum') and embedding, autograd for the table gradients,
    and torch.optim.Adagrad for the step.  Every table gets one extra all-zero
    row that hash misses index (the constant zero vector of "集成 DynamicEmb"
    §3.2); that row is not part of the table.  Returns the tensors, the
    optimizer and the gradients of the real rows."""
    B = b.B
    starts = np.concatenate([[0], np.cumsum(b.lengths)])
    L = b.lengths.reshape(synth.T, B)
    if weights is None:
        weights = [torch.tensor(np.concatenate([np.asarray(t["values"], np.float64),
                                                np.zeros((1, 16))]), requires_grad=True)
                   for t in m.tables]
        opt_state = torch.optim.Adagrad(weights, lr=lr, eps=eps, initial_accumulator_value=0.0,
                                        foreach=False)

    def rows_of(k, raw):
        r = py_rows(m.tables[k], raw)
        return torch.from_numpy(np.where(r < 0, int(m.tables[k]["rows"]), r))

    opt_state.zero_grad()
    loss = torch.zeros((), dtype=torch.float64)
    for k in range(synth.T):
        lo, hi = starts[k * B], starts[(k + 1) * B]
        bag_off = torch.from_numpy(np.concatenate([[0], np.cumsum(L[k])[:-1]]).astype(np.int64))
        pooled = F.embedding_bag(rows_of(k, b.values[lo:hi]), weights[k], bag_off, mode="sum")
        g = torch.from_numpy(dpooled[:, 16 * k:16 * k + 16].astype(np.float64))
        loss = loss + (pooled * g).sum()
    if seq is not None:
        st, sv, ds = seq
        P = ds.shape[1]
        for f in range(3):
            loss = loss + (F.embedding(rows_of(st[f], sv[f, :P]), weights[st[f]]) *
                           torch.from_numpy(ds[f].astype(np.float64))).sum()
    loss.backward()
    grads = [w.grad.detach()[:-1].clone().numpy() for w in weights]
    opt_state.step()
    return weights, opt_state, grads


def _adagrad_two_steps(orc, m, b, seed):
    off = orc.lengths_to_offsets(b.lengths)
    rng = np.random.default_rng(seed)
    P = int(b.seq_lengths.sum())
    st = np.array(synth.SEQ_KEYS, np.int32)
    w = [np.asarray(t["values"], np.float32) for t in m.tables]
    G = [np.zeros((int(t["rows"]), 16), np.float32) for t in m.tables]
    tw, topt = None, None
    for step, lr in ((0, 1e-3), (1, 1e-3)):
        dp = rng.standard_normal((b.B, 256)).astype(np.float32)
        ds = rng.standard_normal((3, P, 16)).astype(np.float32)
        seq = (st, b.seq_values, ds)
        nw, nG, grad, touched = orc.embbag_adagrad(m.tables, b.B, b.values, b.lengths, off, dp, w,
                                                   G, lr=lr, eps=1e-10, seq=seq)
        tw, topt, tgrad = _torch_sparse_step(m, b, dp, seq, tw, topt, lr, 1e-10)
        for k in range(synth.T):
            m_ = touched[k]
            tw_k = tw[k].detach()[:-1].numpy()
            assert _rel(grad[k], tgrad[k]) < 1e-13, (step, k)
            assert _rel(nw[k][m_], tw_k[m_]) < 1e-13, (step, k)
            assert _rel(nG[k], topt.state[tw[k]]["sum"][:-1].numpy()) < 1e-13, (step, k)
            # rows nobody read (empty hash slots hold NaN) keep their bits
            w0 = np.asarray(w[k], np.float64)[~m_]
            assert np.array_equal(nw[k][~m_], w0, equal_nan=True)
            assert np.array_equal(tw_k[~m_], w0, equal_nan=True)
            assert np.array_equal(nG[k][~m_], np.asarray(G[k], np.float64)[~m_])
            assert np.all(np.isfinite(nw[k][m_]))
            if step == 0:
                gk = grad[k][touched[k]]
                assert np.array_equal(nG[k][touched[k]], gk * gk)
                want = np.asarray(w[k], np.float64)[touched[k]] - lr * gk / (np.abs(gk) + 1e-10)
                assert _rel(nw[k][touched[k]], want) < 1e-15
        w = [a.astype(np.float64) for a in nw]
        G = [a.astype(np.float64) for a in nG]


def pin_embbag_adagrad(orc):
    """Backward of the sum-pooled bags and of the sequence rows, then sparse
    AdaGrad ("当前现状分析" run-config table and §3), against torch fp64
    autograd through embedding_bag / embedding and torch.optim.Adagrad, for two
    steps in a row (the second from the first's accumulators), with empty bags
    and repeated ids, on direct tables and on hash tables whose misses read
    the zero vector ("集成 DynamicEmb" §3.2) and so take no gradient; closed
    forms: after one step from a zero accumulator G = g^2 exactly and w moves
    by lr * g / (|g| + eps); untouched rows keep their bits; a repeated id
    counts once per repetition."""
    m, b = _tiny(B=48)
    L = b.lengths.reshape(synth.T, b.B).copy()
    L[2, ::4] = 0
    L[7, 3] = 0
    vals, starts = [], np.concatenate([[0], np.cumsum(b.lengths)])
    for k in range(synth.T):
        for bb in range(b.B):
            i = k * b.B + bb
            vals.append(b.values[starts[i]: starts[i] + L[k, bb]])
    b.lengths = L.reshape(-1).astype(np.int32)
    b.values = np.concatenate(vals).astype(np.int64)
    _adagrad_two_steps(orc, m, b, 91)
    mh = synth.make_model(TINY_HASH)
    bh = synth.make_batch(mh, B=40)
    _adagrad_two_steps(orc, mh, bh, 92)
    # a hash miss takes no gradient: a bag of misses touches nothing
    rows = [int(t["rows"]) for t in m.tables]
    lens = np.zeros(synth.T, np.int32)
    lens[0] = 2
    stored = set(mh.tables[0]["keys"].tolist())
    miss = [x for x in range(1, 100) if x not in stored][:2]
    o1 = orc.lengths_to_offsets(lens)
    dp = np.ones((1, 256), np.float32)
    zh = [np.zeros((int(t["rows"]), 16)) for t in mh.tables]
    _, _, grad, touched = orc.embbag_adagrad(mh.tables, 1, np.array(miss, np.int64), lens, o1, dp,
                                             zh, zh)
    assert not any(t.any() for t in touched) and all(not g.any() for g in grad)
    # a repeated id adds its bag's gradient once per repetition: one bag of
    # table 8 (3 rows) holding id 4 three times moves row 1 by 3 * dpooled
    lens = np.zeros(synth.T, np.int32)
    lens[8] = 3
    v = np.array([4, 4, 4], np.int64)
    o1 = orc.lengths_to_offsets(lens)
    dp = np.zeros((1, 256), np.float32)
    dp[0, 128:144] = np.arange(1, 17, dtype=np.float32) / 8
    z = [np.zeros((r, 16)) for r in rows]
    _, nG, grad, touched = orc.embbag_adagrad(rows, 1, v, lens, o1, dp, z, z, lr=1e-3)
    assert [int(t.sum()) for t in touched] == [1 if k == 8 else 0 for k in range(synth.T)]
    assert np.array_equal(grad[8][1], 3.0 * dp[0, 128:144].astype(np.float64))
    assert np.array_equal(nG[8][1], (3.0 * dp[0, 128:144].astype(np.float64)) ** 2)


def _torch_din_grads(model, batch, query, seq_offsets, max_len, gatt, pad_to=100):
    """Autograd of sum(att * gatt) through the pages' padded DIN, in fp64:
    gradients of the query, of every real sequence row, and of the MLP."""
    B = batch.B
    S = np.zeros((B, pad_to, 48))
    L = np.minimum(batch.seq_lengths.astype(np.int64), max_len)
    for i, k in enumerate(synth.SEQ_KEYS):
        tab = model.tables[k]
        w = np.asarray(tab["values"], dtype=np.float64)
        for b in range(B):
            n = int(L[b])
            ids = batch.seq_values[i, seq_offsets[b]: seq_offsets[b] + n]
            r = py_rows(tab, ids)
            S[b, :n, 16 * i:16 * i + 16] = np.where(r[:, None] < 0, 0.0, w[np.maximum(r, 0)])
    leaf = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)  # noqa: E731
    St, Qt = leaf(S), leaf(query)
    W1, B1, W2, B2 = leaf(model.w1), leaf(model.b1), leaf(model.w2), leaf(model.b2)
    W3, B3 = leaf(model.w3), leaf([float(model.b3)])
    Q = Qt[:, None, :].expand(B, pad_to, 48)
    X = torch.cat([Q, St, Q - St, Q * St], dim=-1)
    z1 = F.linear(X, W1, B1)
    h1 = torch.relu(z1)
    h1.retain_grad()
    z2 = F.linear(h1, W2, B2)
    h2 = torch.relu(z2)
    e = F.linear(h2, W3[None, :], B3).squeeze(-1)
    mask = torch.arange(pad_to)[None, :] < torch.from_numpy(L)[:, None]
    pw = torch.softmax(e.masked_fill(~mask, float("-inf")), dim=-1)
    pw = torch.where(mask, pw, torch.zeros_like(pw))
    att = torch.bmm(pw[:, None, :], St).squeeze(1)
    (att * torch.from_numpy(np.asarray(gatt, np.float64))).sum().backward()
    P = int(seq_offsets[-1] + batch.seq_lengths[-1]) if B else 0
    gs = np.zeros((P, 48))
    # per position index: z1 / (the size of its terms), dL/dh1, z2 / size
    with torch.no_grad():
        a1 = X.abs() @ W1.abs().T + B1.abs()
        a2 = h1.abs() @ W2.abs().T + B2.abs()
    r1, v1, r2 = np.zeros((P, 256)), np.zeros((P, 256)), np.zeros((P, 64))
    for b in range(B):
        o, n = int(seq_offsets[b]), int(L[b])
        gs[o: o + n] = St.grad[b, :n].numpy()
        r1[o: o + n] = (z1[b, :n] / a1[b, :n]).detach().numpy()
        v1[o: o + n] = h1.grad[b, :n].numpy()
        r2[o: o + n] = (z2[b, :n] / a2[b, :n]).detach().numpy()
    return dict(gq=Qt.grad.numpy(), gs=gs, dw1=W1.grad.numpy(), db1=B1.grad.numpy(),
                dw2=W2.grad.numpy(), db2=B2.grad.numpy(), dw3=W3.grad.numpy(),
                db3=float(B3.grad[0]), r1=r1, v1=v1, r2=r2)


def pin_din_bwd(orc):
    """DIN attention backward against torch fp64 autograd through the pages'
    padded formulation ("当前现状分析" §4.2, §4.4), every gradient; closed
    forms: one-position sequences take no MLP gradient and pass g straight to
    their row (p = 1 whatever the score), zero score weights give every row
    g / L and no gradient to W1, W2 or the query; and central finite
    differences of the oracle's own forward for entries of W1, b2, w3 and of a
    query."""
    for bias, emb_std, w3s in ((True, 0.05, 1.0), (True, 1.0, 20.0)):
        m, b = _tiny(bias=bias, B=24, emb_std=emb_std, w3_scale=w3s)
        off = _seq_offsets(b)
        pooled = orc.embbag(m.tables, b.B, b.values, b.lengths, orc.lengths_to_offsets(b.lengths))
        q = _query_from(pooled)
        g = np.random.default_rng(5).standard_normal((b.B, 48))
        seq_tabs = [m.tables[k] for k in synth.SEQ_KEYS]
        got = orc.din_bwd(seq_tabs, b.seq_values, b.seq_stride, off, b.seq_lengths, 100, q, m.w1,
                          m.b1, m.w2, m.b2, m.w3, m.b3, g, gates=True)
        ref = _torch_din_grads(m, b, q, off, 100, g)
        for k in ("gq", "gs", "dw1", "db1", "dw2", "db2", "dw3"):
            assert _rel(got[k], ref[k]) < 1e-12, (k, _rel(got[k], ref[k]))
        # the gate outputs: pre-activations over their terms' sizes (within
        # [-1, 1]) and the gradient reaching h1 (autograd's dL/dh1)
        P = ref["r1"].shape[0]
        for k in ("r1", "v1", "r2"):
            assert _rel(got[k][:P], ref[k]) < 1e-12, (k, _rel(got[k][:P], ref[k]))
        assert np.abs(got["r1"]).max() <= 1 and np.abs(got["r2"]).max() <= 1
        assert (got["v1"] != 0).any() and (got["r1"] > 0).any() and (got["r1"] < 0).any()
        assert abs(got["db3"] - ref["db3"]) <= 1e-12 * max(1.0, abs(ref["db3"]))
        assert np.all(got["gq_scale"] >= np.abs(got["gq"]) * (1 - 1e-12))
        # db3 vanishes: the softmax ignores a common shift of the scores
        assert abs(got["db3"]) <= 1e-13 * got["db3_scale"] and got["db3_scale"] > 0
    # finite differences of the oracle's forward (loss = sum(att * g))
    m, b = _tiny(bias=True, B=6)
    off = _seq_offsets(b)
    seq_tabs = [m.tables[k] for k in synth.SEQ_KEYS]
    q = np.random.default_rng(6).normal(0, 0.05, (b.B, 48))
    g = np.random.default_rng(7).standard_normal((b.B, 48))

    def loss(w1, b2, w3, qq):
        att = orc.din(seq_tabs, b.seq_values, b.seq_stride, off, b.seq_lengths, 100, qq, w1, m.b1,
                      m.w2, b2, w3, m.b3)
        return float(np.sum(att * g))

    got = orc.din_bwd(seq_tabs, b.seq_values, b.seq_stride, off, b.seq_lengths, 100, q, m.w1, m.b1,
                      m.w2, m.b2, m.w3, m.b3, g)
    base = [np.array(m.w1, np.float64), np.array(m.b2, np.float64), np.array(m.w3, np.float64), q]
    for which, idx, key in ((0, (7, 100), "dw1"), (0, (200, 5), "dw1"), (1, (3,), "db2"),
                            (2, (11,), "dw3"), (3, (2, 40), "gq")):
        h = 1e-6
        up = [x.copy() for x in base]
        dn = [x.copy() for x in base]
        up[which][idx] += h
        dn[which][idx] -= h
        fd = (loss(*up) - loss(*dn)) / (2 * h)
        an = got[key][idx]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, idx, fd, an)
    # one-position sequences: p = 1, no MLP gradient, ds = g, dq = 0
    m, b = _tiny(bias=True, B=16)
    b.seq_lengths = np.ones(b.B, np.int32)
    b.seq_values = np.ascontiguousarray(b.seq_values[:, :b.B])
    b.seq_stride = b.B
    off = _seq_offsets(b)
    q = np.random.default_rng(8).normal(0, 0.05, (b.B, 48))
    g = np.random.default_rng(9).standard_normal((b.B, 48))
    got = orc.din_bwd([m.tables[k] for k in synth.SEQ_KEYS], b.seq_values, b.seq_stride, off,
                      b.seq_lengths, 100, q, m.w1, m.b1, m.w2, m.b2, m.w3, m.b3, g)
    assert np.array_equal(got["gs"], g) and not got["gq"].any()
    for k in ("dw1", "db1", "dw2", "db2", "dw3"):
        assert not got[k].any(), k
    assert got["db3"] == 0.0
    # zero score weights: uniform weights, ds = g / L, nothing reaches W1, W2 or q
    m, b = _tiny(bias=True, B=16, w3_scale=0.0)
    off = _seq_offsets(b)
    got = orc.din_bwd([m.tables[k] for k in synth.SEQ_KEYS], b.seq_values, b.seq_stride, off,
                      b.seq_lengths, 100, q, m.w1, m.b1, m.w2, m.b2, m.w3, m.b3, g)
    Ls = np.minimum(b.seq_lengths, 100)
    for bb in range(b.B):
        rows = got["gs"][off[bb]: off[bb] + Ls[bb]]
        assert np.allclose(rows, g[bb] / Ls[bb], rtol=1e-14, atol=1e-16)
    for k in ("gq", "dw1", "db1", "dw2", "db2"):
        assert not got[k].any(), k


def _torch_dlrm(m, dense, values, lengths):
    """The DLRM essay's forward (§2.3, §4.2) written with torch library
    routines in fp64: F.embedding_bag per table (mode 'sum' or 'mean', offsets
    from a cumulative sum of the lengths), F.linear + relu for the bottom and
    top MLPs, bmm with triu_indices for the interaction, sigmoid."""
    import torch.nn.functional as Fn
    S = len(m.tables)
    B = dense.shape[0]
    D = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    x = D(dense)
    h = torch.relu(Fn.linear(torch.relu(Fn.linear(x, D(m.wb1), D(m.bb1))), D(m.wb2), D(m.bb2)))
    L = np.asarray(lengths, np.int64).reshape(S, B)
    starts = np.concatenate([[0], np.cumsum(L.reshape(-1))])
    vecs = [h]
    for t in range(S):
        ids = torch.from_numpy(np.asarray(values[starts[t * B]: starts[(t + 1) * B]], np.int64))
        off = torch.from_numpy(starts[t * B: (t + 1) * B] - starts[t * B])
        mode = "mean" if m.modes[t] == 1 else "sum"
        vecs.append(Fn.embedding_bag(ids, D(m.tables[t]), off, mode=mode))
    z = torch.stack(vecs, dim=1)                                   # [B][S+1][d]
    gram = torch.bmm(z, z.transpose(1, 2).contiguous())
    iu = torch.triu_indices(S + 1, S + 1)
    inter = gram[:, iu[0], iu[1]]
    t2 = torch.relu(Fn.linear(torch.relu(Fn.linear(inter, D(m.wt1), D(m.bt1))), D(m.wt2), D(m.bt2)))
    logit = t2 @ D(m.wt3) + m.bt3
    return z.numpy(), inter.numpy(), logit.numpy(), torch.sigmoid(logit).numpy()


def pin_dlrm_fwd(orc):
    """The DLRM forward (DLRM essay §2.3 four layers, §3.2 sum / mean bags,
    §4.2 widths) against torch fp64 library routines (F.embedding_bag in sum
    and mean mode, F.linear, bmm + triu_indices, sigmoid), on a small model
    with mixed modes and empty bags; and closed forms: a one-id bag equals its
    row in both modes, a bag of one id repeated k times equals the row in mean
    mode and k times it in sum mode, an empty bag is 0 in both modes, zero
    top weights give logit = bt3, and a zero bottom MLP zeroes every pair with
    the dense vector."""
    import dataclasses
    cfg = dataclasses.replace(synth.DLRM_WORKLOADS[2], sizes=(50, 40, 30, 20, 9), n_dense=5,
                              dim=32, modes=(0, 1, 1, 0, 1), bag_max=4)
    m = synth.make_dlrm(cfg, bias=True, emb_scale=4.0)
    b = synth.make_dlrm_batch(m, B=24)
    L = b.lengths.reshape(5, 24).copy()
    L[1, 3] = 0
    L[0, 7] = 0
    vals = []
    starts = np.concatenate([[0], np.cumsum(b.lengths)])
    rng = np.random.default_rng(5)
    for t in range(5):
        for bb in range(24):
            vals.append(rng.integers(0, cfg.sizes[t], size=int(L[t, bb])))
    values = np.concatenate(vals).astype(np.int64)
    got = orc.dlrm_fwd(m, b.dense, values, L.reshape(-1))
    z, inter, logit, prob = _torch_dlrm(m, b.dense, values, L.reshape(-1))
    assert _rel(got["z"], z) < 1e-13
    assert np.max(np.abs(got["inter"] - inter) / np.maximum(got["iscale"], 1e-300)) < 1e-13
    assert np.max(np.abs(got["logit"] - logit) / np.maximum(got["lscale"], 1e-300)) < 1e-13
    assert np.max(np.abs(got["prob"] - prob)) < 1e-13
    assert not got["z"][3, 2].any() and not got["z"][7, 1].any()        # empty bags
    # closed forms on hand-made bags: table t, sample 0
    B = 4
    dense = np.zeros((B, 5), np.float32)
    Lc = np.ones((5, B), np.int32)
    row = 7
    Lc[1, 0], Lc[0, 0], Lc[3, 1] = 3, 3, 0
    vals = []
    for t in range(5):
        for bb in range(B):
            vals.append(np.full(int(Lc[t, bb]), row + 0 * bb, np.int64))
    values = np.concatenate(vals)
    mz = dataclasses.replace(m, bb1=np.zeros_like(m.bb1), bb2=np.zeros_like(m.bb2))
    g = orc.dlrm_fwd(mz, dense, values, Lc.reshape(-1))
    for t in range(5):
        r = m.tables[t][row].astype(np.float64)
        k = int(Lc[t, 0])
        want = r if (m.modes[t] == 1 or k == 1) else k * r
        assert np.array_equal(g["z"][0, 1 + t], want), t
    assert not g["z"][1, 4].any()                                   # empty bag, table 3
    assert not g["z"][:, 0].any()                                   # zero dense, zero biases
    F = 6
    iu = np.triu_indices(F)
    assert not g["inter"][:, iu[0] == 0].any()                      # pairs with the dense vector
    m0 = dataclasses.replace(m, wt3=np.zeros_like(m.wt3))
    g0 = orc.dlrm_fwd(m0, b.dense, b.values, b.lengths)
    assert np.all(g0["logit"] == m.bt3) and np.allclose(g0["prob"], 1 / (1 + np.exp(-m.bt3)),
                                                        rtol=1e-15, atol=0)


def pin_hash_admit(orc):
    """Frequency admission and score-driven eviction ("集成 DynamicEmb" §4.1
    threshold, §4.2 STEP / LFU / NO_EVICTION) against the pinned insert, the
    generator's convention and closed forms: with threshold 1 and room it is
    the insert of the distinct ids; ids are admitted exactly at the call
    where their running count reaches the threshold (LFU starting from that
    count); a full table evicts the oldest (STEP) or least used (LFU) entries
    stored before the call, the smaller id first on equal scores, scores
    saturating at 2^32 - 2; a used id is not the oldest any more; a new id
    takes the first free slot (empty or tombstone) from its home; NO_EVICTION
    admits nothing into a full table and keeps the counts; reserved ids are
    neither stored nor counted; a full counter table counts no new id."""
    NONE, STEP, LFU = orc.SCORE_NONE, orc.SCORE_STEP, orc.SCORE_LFU
    rng = np.random.default_rng(4141)
    vals = lambda n: rng.standard_normal((n, 16)).astype(np.float32)  # noqa: E731
    # (1) threshold 1, room, NO_EVICTION: the insert of the distinct ids in
    # first-occurrence order, with the values of their first occurrence
    cap = 997
    base = _distinct_keys(rng, 300)
    keys = np.concatenate([base, base[::3], base[::7]])
    v = vals(keys.size)
    t, c = orc.empty_hash_table(cap), orc.empty_counter_table(2048)
    slots, cnt = orc.hash_admit(t, c, keys, v, 1, NONE)
    t2 = orc.empty_hash_table(cap)
    s2 = orc.hash_insert(t2, base, v[:300])
    for f in ("keys", "digests"):
        assert np.array_equal(t[f], t2[f]), f
    occ = t["keys"] != -1
    assert np.array_equal(t["values"][occ], t2["values"][occ])
    assert np.array_equal(slots[:300], s2) and list(cnt) == [300, 0, 0]
    assert orc.hash_check(t["keys"], t["digests"]) == 0
    # (2) running counts: admitted at the first call where the count reaches 3
    t, c = orc.empty_hash_table(101), orc.empty_counter_table(101)
    k = np.array([11, 22, 33], np.int64)
    calls = [np.array([11, 22]), np.array([11, 33, 33]), np.array([22, 11, 33]), np.array([22, 22])]
    admitted_at = {}
    for step, kk in enumerate(calls):
        sl, _ = orc.hash_admit(t, c, kk.astype(np.int64), vals(kk.size), 3, LFU, step)
        for key in k:
            s_ = orc.hash_find_slow(t, int(key))
            if s_ >= 0 and int(key) not in admitted_at:
                admitted_at[int(key)] = step
                # LFU starts from the running count that reached the threshold
                assert t["scores"][s_] == {11: 3, 33: 3, 22: 4}[int(key)], (key, t["scores"][s_])
        for key, s_ in zip(kk, sl):
            assert (s_ >= 0) == (int(key) in admitted_at)
    assert admitted_at == {11: 2, 33: 2, 22: 3}
    assert t["scores"][orc.hash_find_slow(t, 11)] == 3 and t["scores"][orc.hash_find_slow(t, 33)] == 3
    assert t["scores"][orc.hash_find_slow(t, 22)] == 4          # 1 + 1 + 2 at admission
    assert not np.any(c["counts"][np.isin(c["keys"], k)])      # counts reset on admission
    # (3) STEP eviction: 16 ids admitted at steps 1..16 fill max_keys = 16;
    # three new ids at step 100 evict the three oldest; an old id that is
    # used in the same call is not among them
    cap = 64
    t, c = orc.empty_hash_table(cap), orc.empty_counter_table(256)
    old = _distinct_keys(rng, 16)
    for i, key in enumerate(old):
        orc.hash_admit(t, c, np.array([key]), vals(1), 1, STEP, 1 + i, max_keys=16)
    where = {int(key): orc.hash_find_slow(t, int(key)) for key in old}
    # the first new id's home is the slot of old[1], which this call evicts:
    # it must take that tombstone
    cand_k = _distinct_keys(np.random.default_rng(8), 20000)
    homes = synth.home_slot(synth.splitmix64_mix(cand_k), cap)
    first = cand_k[np.nonzero(homes == where[int(old[1])])[0][0]]
    rest = cand_k[(homes != where[int(old[1])]) & ~np.isin(cand_k, old)][:2]
    new = np.concatenate([[first], rest]).astype(np.int64)
    batch = np.concatenate([new, old[:1]])
    sl, cnt = orc.hash_admit(t, c, batch, vals(4), 1, STEP, 100, max_keys=16)
    assert list(cnt) == [3, 3, 0] and np.all(sl >= 0)
    for i, key in enumerate(old):
        s_ = orc.hash_find_slow(t, int(key))
        assert (s_ < 0) == (i in (1, 2, 3)), i
        if s_ >= 0:
            assert s_ == where[int(key)]                       # survivors keep their slots
    assert t["scores"][where[int(old[0])]] == 100
    assert orc.hash_find_slow(t, int(first)) == where[int(old[1])]
    assert orc.hash_check(t["keys"], t["digests"]) == 0
    stored = (t["keys"] != -1) & (t["keys"] != -2)
    assert stored.sum() == 16 and np.sum(t["keys"] == -2) <= 3
    # new ids sit at the first free slot (empty or tombstone) from their home
    h = synth.splitmix64_mix(new)
    for key, home in zip(new, synth.home_slot(h, cap)):
        s_ = orc.hash_find_slow(t, int(key))
        q = int(home)
        while q != s_:
            assert t["keys"][q] not in (-1, -2)                # passed no free slot
            q = (q + 1) % cap
    # (4) LFU eviction: counts 5, 1, 3, 1 -> the two least used go; scores
    # at or above 2^32 - 2 compare as equal, and equal scores go smaller id
    # first
    t, c = orc.empty_hash_table(16), orc.empty_counter_table(64)
    ks = _distinct_keys(rng, 4)
    for key, n_ in zip(ks, (5, 1, 3, 1)):
        orc.hash_admit(t, c, np.full(n_, key, np.int64), vals(n_), 1, LFU, 0, max_keys=4)
    sl_old = [orc.hash_find_slow(t, int(key)) for key in ks]
    fresh = _distinct_keys(np.random.default_rng(9), 2)
    _, cnt = orc.hash_admit(t, c, fresh, vals(2), 1, LFU, 0, max_keys=4)
    assert list(cnt) == [2, 2, 0]
    assert [orc.hash_find_slow(t, int(key)) >= 0 for key in ks] == [True, False, True, False]
    t, c = orc.empty_hash_table(16), orc.empty_counter_table(64)
    for key in ks[:3]:
        orc.hash_admit(t, c, np.array([key]), vals(1), 1, LFU, 0, max_keys=3)
    sl3 = [orc.hash_find_slow(t, int(key)) for key in ks[:3]]
    t["scores"][sl3[0]], t["scores"][sl3[1]], t["scores"][sl3[2]] = 2**33, 2**40, 7
    orc.hash_admit(t, c, ks[3:4], vals(1), 1, LFU, 0, max_keys=3)
    gone = [i for i in range(3) if orc.hash_find_slow(t, int(ks[i])) < 0]
    assert gone == [2]                                             # 7 is the least
    s3 = orc.hash_find_slow(t, int(ks[3]))
    left = {int(ks[0]): sl3[0], int(ks[1]): sl3[1], int(ks[3]): s3}   # id -> slot
    order = sorted(left)
    # scores all at or above 2^32 - 2: equal after saturation, so the
    # smallest id goes even though its raw score is the largest
    for k_, sc in zip(order, (2**41, 2**34, 2**32 - 2)):
        t["scores"][left[k_]] = sc
    orc.hash_admit(t, c, fresh[:1], vals(1), 1, LFU, 0, max_keys=3)
    gone = [k_ for k_ in left if orc.hash_find_slow(t, k_) < 0]
    assert gone == [order[0]]
    # (5) NO_EVICTION keeps a full table and the counts of those left out
    t, c = orc.empty_hash_table(32), orc.empty_counter_table(64)
    ks = _distinct_keys(rng, 6)
    orc.hash_admit(t, c, ks[:4], vals(4), 1, NONE, max_keys=4)
    before = _stored_map(t)
    sl, cnt = orc.hash_admit(t, c, np.repeat(ks[4:], 2), vals(4), 2, NONE, max_keys=4)
    assert list(cnt) == [0, 0, 2] and np.all(sl == -1) and _stored_map(t) == before
    got = {int(key): int(n_) for key, n_ in zip(c["keys"], c["counts"]) if key != -1}
    assert got[int(ks[4])] == 2 and got[int(ks[5])] == 2
    sl, cnt = orc.hash_admit(t, c, ks[4:5], vals(1), 2, NONE, max_keys=4)    # 2 + 1, still left out
    assert list(cnt) == [0, 0, 1] and sl[0] == -1
    got = {int(key): int(n_) for key, n_ in zip(c["keys"], c["counts"]) if key != -1}
    assert got[int(ks[4])] == 3
    # (6) reserved ids; (7) a full counter table counts no new id
    t, c = orc.empty_hash_table(32), orc.empty_counter_table(2)
    sl, cnt = orc.hash_admit(t, c, np.array([-1, -2, 5, 6, 7, 5], np.int64), vals(6), 3, LFU)
    assert sl[0] == -2 and sl[1] == -2 and np.all(sl[2:] == -1) and list(cnt) == [0, 0, 0]
    assert sorted(c["keys"].tolist()) == [5, 6] and sorted(c["counts"].tolist()) == [1, 2]
    assert not np.any(t["keys"] == -2)


ALL_PINS = [pin_offsets, pin_floor_mod, pin_hash, pin_embbag_direct, pin_embbag_hash,
            pin_din_vs_padded, pin_din_closed_forms, pin_din_hash, pin_towers_closed_forms,
            pin_towers_library, pin_hash_insert, pin_dlrm_interact, pin_embbag_adagrad,
            pin_din_bwd, pin_dlrm_fwd, pin_hash_admit]
