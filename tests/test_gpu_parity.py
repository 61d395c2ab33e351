"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Integers (offsets, resolved rows, hash slots) must match
bit-exactly; floats within the per-row relative tolerance of the MLP's
precision (1e-5 fp32, 2e-2 bf16 matrix cores with fp32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (BF16_TOL, DEV, FP32_TOL, Run, gpu_scores_by_sample, oracle_forward,
                         oracle_rows, row_rel_err, say)
from sparse_embedding_din_amd import pipeline as PL
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def models():
    cache = {}

    def get(i, **kw):
        key = (i, tuple(sorted(kw.items())))
        if key not in cache:
            cache[key] = synth.make_model(synth.WORKLOADS[i], **kw)
        return cache[key]
    return get


def _tol(model):
    return FP32_TOL if model.mlp_dtype == "f32" else BF16_TOL


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [0, 1, 5, 1024, 1025, 4095, 4096, 4097, 131089, 300000])
def test_lengths_to_offsets(n):
    rng = np.random.default_rng(n)
    L = rng.integers(0, 4, size=n).astype(np.int32)
    say(f"scan n={n}")
    lt = torch.from_numpy(L).to(DEV)
    off = torch.full((n + 1,), -5, dtype=torch.int64, device=DEV)
    R.rec_lengths_to_offsets(lt, n, off)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), oracle.get().lengths_to_offsets(L))


@pytest.mark.parametrize("B,max_len,C", [(1, 100, 0), (37, 100, 16), (4096, 100, 32),
                                          (4097, 7, 64), (10000, 128, 4096)])
def test_din_plan(models, B, max_len, C):
    """Plan: jagged offsets, packed starts, per-position entries and
    resolved rows (bit-exact against the oracle)."""
    m = models(1)
    rng = np.random.default_rng(B)
    L = rng.integers(0, 140, size=B).astype(np.int32)
    L[::7] = 0
    orc = oracle.get()
    off = orc.lengths_to_offsets(L)
    stride = int(off[-1])
    seq = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=(3, max(stride, 1)),
                       dtype=np.int64)
    say(f"plan B={B} max_len={max_len} C={C}")
    tabs = PL.DeviceTables([m.tables[k] for k in synth.SEQ_KEYS], DEV)
    lt = torch.from_numpy(L).to(DEV)
    st = torch.from_numpy(seq).to(DEV)
    pb = R.rec_din_plan_bytes(B, max_len)
    plan = torch.zeros(pb, dtype=torch.uint8, device=DEV)
    so = torch.full((B + 1,), -5, dtype=torch.int64, device=DEV)
    rows = torch.full((3, max(stride, 1)), -9, dtype=torch.int64, device=DEV)
    R.rec_din_plan(tabs.array(), st, seq.shape[1], None, lt, B, max_len, C, so, rows, plan, pb)
    torch.cuda.synchronize()
    assert np.array_equal(so.cpu().numpy(), off)
    p = plan.cpu().numpy()
    hdr = p[:64].view(np.int32)
    clamped = np.minimum(L, max_len)
    P = int(clamped.sum())
    assert hdr[0] == B and hdr[1] == max_len and hdr[4] == P
    assert hdr[2] == C
    a16 = lambda x: (x + 15) // 16 * 16
    nb = (B + 1023) // 1024
    off_pos = a16(64 + 8 * 130 * nb)
    pos = p[off_pos: off_pos + 4 * (B + 1)].view(np.int32)
    assert np.array_equal(pos, orc.lengths_to_offsets(clamped))
    pmax = B * max_len
    off_pb = a16(a16(off_pos + 4 * (B + 1)) + 8 * B)
    pos_b = p[off_pb: off_pb + 4 * P].view(np.int32)
    off_pjr = a16(off_pb + 4 * pmax)
    pos_jr = p[off_pjr: off_pjr + 4 * P].view(np.int32)
    off_prows = a16(off_pjr + 4 * pmax)
    exp_b = np.repeat(np.arange(B), clamped)
    exp_j = np.arange(P) - pos[exp_b]
    assert np.array_equal(pos_b, exp_b)
    assert np.array_equal(pos_jr & 0xffff, exp_j)
    assert np.array_equal(pos_jr >> 16, clamped[exp_b] - 1 - exp_j)
    # resolved rows: every id inside the first min(len, max_len) steps, bit-exact
    rg = rows.cpu().numpy()
    gidx = off[exp_b] + exp_j
    for f, k in enumerate(synth.SEQ_KEYS):
        ref = orc.resolve(m.tables[k], seq[f, gidx])
        assert np.array_equal(rg[f, gidx], ref)
        pr = p[off_prows + 4 * f * pmax: off_prows + 4 * (f * pmax + P)].view(np.int32)
        assert np.array_equal(pr, ref)
    # positions past the cap are never read
    mask = np.ones(max(stride, 1), bool)
    mask[gidx] = False
    assert np.all(rg[:, mask] == -9)
    # attention groups: nominal spans of one requested range per wave of an
    # attention workgroup (eight waves), else P over the workgroups (one per
    # CU), each start moved forward to a sample start
    groups = torch.cuda.get_device_properties(0).multi_processor_count
    span = 8 * C if C > 0 else max(1, -(-P // groups))
    ng = -(-P // span)
    assert hdr[3] == ng
    off_group = a16(a16(off_prows + 12 * pmax) + 4 * B)
    gs = p[off_group: off_group + 4 * (ng + 1)].view(np.int32)
    starts = np.append(pos[:B], P)
    exp_gs = [0]
    for g in range(1, ng):
        t = g * span
        nxt = int(starts[np.searchsorted(starts, t, "left")])      # first start >= t
        prv = int(starts[np.searchsorted(starts, t, "right") - 1])  # last start <= t
        exp_gs.append(prv if t - prv <= nxt - t else nxt)
    exp_gs.append(P)
    assert np.array_equal(gs[: ng + 1], np.array(exp_gs[: ng + 1], dtype=np.int32)), (gs, exp_gs)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,B", [(1, 256), (1, 37), (2, 8192), (4, 65536), (5, 8192)])
def test_embbag_parity(models, cfg, B):
    """Offsets derived inside the embedding bags (from the KJT sums), pooled
    output and resolved rows against the oracle; the two-call form (offsets
    scan, then bags) gives bit-identical results."""
    m = models(cfg)
    b = synth.make_batch(m, B=B)
    r = Run(m, b)
    r2 = Run(m, b, fused=False)
    assert np.array_equal(r.offsets, r2.offsets)
    assert np.array_equal(r.pooled, r2.pooled)
    assert np.array_equal(r.emb_rows, r2.emb_rows)
    orc = oracle.get()
    assert np.array_equal(r.offsets, orc.lengths_to_offsets(b.lengths))
    rows, _ = oracle_rows(m, b)
    assert np.array_equal(r.emb_rows, rows)
    ref = orc.embbag(m.tables, B, b.values, b.lengths, r.offsets)
    assert row_rel_err(r.pooled, ref) <= 1e-6


def test_embbag_edges(models):
    """Empty bags, a single id per bag, every id of the signed range's edges."""
    m = models(1)
    b = synth.make_batch(m, B=33)
    L = b.lengths.reshape(synth.T, 33).copy()
    L[:, 0] = 0                       # sample 0: every bag empty
    L[2, 5:9] = 0
    L[4, 10:14] = 1
    i64 = np.iinfo(np.int64)
    edge = np.array([i64.min, i64.max, -1, 0, 1, i64.min + 1, i64.max - 1], np.int64)
    vals = []
    starts = np.concatenate([[0], np.cumsum(b.lengths)])
    for k in range(synth.T):
        for s in range(33):
            i = k * 33 + s
            v = b.values[starts[i]: starts[i] + L[k, s]].copy()
            if k < 15 and v.size:
                v[0] = edge[(k + s) % edge.size]
            vals.append(v)
    b.lengths = L.reshape(-1).astype(np.int32)
    b.values = np.concatenate(vals)
    r = Run(m, b)
    assert np.array_equal(r.offsets, oracle.get().lengths_to_offsets(b.lengths))
    rows, _ = oracle_rows(m, b)
    assert np.array_equal(r.emb_rows, rows)
    ref = oracle.get().embbag(m.tables, 33, b.values, b.lengths, r.offsets)
    assert np.all(r.pooled[0] == 0.0)
    assert row_rel_err(r.pooled, ref) <= 1e-6


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("cfg", [1, 5])
def test_embbag_long_bags(models, cfg, fused):
    """Bags of 0 to 40 ids (a bag lane runs up to 14 rounds of three ids, with
    empty bags beside long ones in every wave), over direct tables and over
    hash tables whose ids keep the workload's mix of hits and misses, with
    offsets given and derived in the bags: resolved rows bit-exact, pooled
    sums within the fp32 tolerance of the oracle's fp64 sums."""
    m = models(cfg)
    B = 300
    b = synth.make_batch(m, B=B)
    rng = np.random.default_rng(40 + cfg)
    L = rng.integers(0, 41, size=(synth.T, B)).astype(np.int32)
    L[rng.random((synth.T, B)) < 0.2] = 0
    starts = np.concatenate([[0], np.cumsum(b.lengths)])
    vals = []
    for k in range(synth.T):
        pool = b.values[starts[k * B]: starts[(k + 1) * B]]      # table k's ids as generated
        vals.append(rng.choice(pool, size=int(L[k].sum())))
    b.lengths = L.reshape(-1)
    b.values = np.concatenate(vals)
    r = Run(m, b, fused=fused)
    orc = oracle.get()
    rows, _ = oracle_rows(m, b)
    assert np.array_equal(r.emb_rows, rows)
    if cfg == 5:
        assert np.any(rows < 0) and np.any(rows >= 0)            # hits and misses both present
    ref = orc.embbag(m.tables, B, b.values, b.lengths, orc.lengths_to_offsets(b.lengths))
    assert row_rel_err(r.pooled, ref) <= FP32_TOL


@pytest.mark.parametrize("T,B", [(1, 1), (5, 2500), (16, 1025), (32, 3000), (3, 4096)])
def test_embbag_kjt_shapes(models, T, B):
    """Offsets derived in the bags for odd table counts, batches that are not
    a multiple of the 32-sample chunk or the 1024-sample block, and up to 32
    tables (the tiny model's tables repeated): bit-exact offsets, pooled
    output against the oracle."""
    m = models(1)
    tables = [m.tables[k % synth.T] for k in range(T)]
    rng = np.random.default_rng(T * 7919 + B)
    L = rng.integers(0, 6, size=T * B).astype(np.int32)
    L[rng.random(T * B) < 0.2] = 0
    nnz = int(L.sum())
    vals = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=max(nnz, 1),
                        dtype=np.int64)
    say(f"kjt T={T} B={B} nnz={nnz}")
    tabs = PL.DeviceTables(tables, DEV)
    lt = torch.from_numpy(L).to(DEV)
    vt = torch.from_numpy(vals).to(DEV)
    sb = R.rec_kjt_sums_bytes(T, B)
    sums = torch.full((sb,), 0x5A, dtype=torch.uint8, device=DEV)
    off = torch.full((T * B + 1,), -5, dtype=torch.int64, device=DEV)
    out = torch.full((B, T * 16), np.nan, dtype=torch.float32, device=DEV)
    R.rec_kjt_sums(lt, T, B, sums, sb)
    R.rec_embbag_fwd_kjt(tabs.array(), T, B, vt, lt, sums, sb, off, out)
    torch.cuda.synchronize()
    orc = oracle.get()
    ref_off = orc.lengths_to_offsets(L)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    ref = orc.embbag(tables, B, vals[:nnz], L, ref_off)
    assert row_rel_err(out.cpu().numpy(), ref) <= 1e-6


def test_hash_lookup(models):
    m = models(5)
    orc = oracle.get()
    for k in m.cfg.hash_keys:
        tab = m.tables[k]
        rng = np.random.default_rng(k)
        hits = tab["stored"][rng.integers(0, tab["stored"].size, 5000)]
        miss = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, 3000, dtype=np.int64)
        keys = np.concatenate([hits, miss, [synth.EMPTY_KEY]])
        rng.shuffle(keys)
        say(f"hash table {k} n={keys.size}")
        vals = torch.from_numpy(tab["values"]).to(DEV)
        kd = torch.from_numpy(tab["keys"]).to(DEV)
        dg = torch.from_numpy(tab["digests"]).to(DEV)
        desc = R.table(R.REC_HASH, tab["rows"], vals, kd, dg, None)
        kt = torch.from_numpy(keys).to(DEV)
        slot = torch.full((keys.size,), -9, dtype=torch.int64, device=DEV)
        rows = torch.full((keys.size, 16), np.nan, dtype=torch.float32, device=DEV)
        R.rec_hash_lookup(desc, kt, keys.size, slot, rows)
        torch.cuda.synchronize()
        ref = orc.resolve(tab, keys)
        got = slot.cpu().numpy()
        assert np.array_equal(got, ref)
        rg = rows.cpu().numpy()
        hit = ref >= 0
        assert np.array_equal(rg[hit], tab["values"][ref[hit]])
        assert np.all(rg[~hit] == 0.0) and not np.any(np.signbit(rg[~hit]))


@pytest.mark.parametrize("cap,nkeys", [(2, 1), (17, 16), (33, 32), (37, 30), (100, 70), (4099, 4000)])
def test_hash_lookup_small_tables(cap, nkeys):
    """Tables around the 32-digest window and nearly full (probes that wrap
    past the end), on the device against the oracle: bit-exact slots, exact
    rows, exact zero rows for misses."""
    rng = np.random.default_rng(cap)
    I64 = np.iinfo(np.int64)
    stored = np.unique(rng.integers(I64.min, I64.max, size=2 * nkeys, dtype=np.int64))
    stored = stored[stored != synth.EMPTY_KEY][:nkeys]
    vals = rng.standard_normal((stored.size, 16)).astype(np.float32)
    tab = synth.build_hash_table(stored, vals, cap)
    miss = rng.integers(I64.min, I64.max, size=500, dtype=np.int64)
    keys = np.concatenate([stored, miss, [synth.EMPTY_KEY]])
    say(f"hash small cap={cap} n={keys.size}")
    dt = PL.DeviceTables([tab], DEV)
    kt = torch.from_numpy(keys).to(DEV)
    slot = torch.full((keys.size,), -9, dtype=torch.int64, device=DEV)
    rows = torch.full((keys.size, 16), np.nan, dtype=torch.float32, device=DEV)
    R.rec_hash_lookup(dt.desc[0], kt, keys.size, slot, rows)
    torch.cuda.synchronize()
    ref = oracle.get().resolve(tab, keys)
    got = slot.cpu().numpy()
    assert np.array_equal(got, ref)
    rg = rows.cpu().numpy()
    hit = ref >= 0
    assert np.array_equal(rg[hit], tab["values"][ref[hit]])
    assert np.all(rg[~hit] == 0.0)


# ---------------------------------------------------------------------------
DIN_CASES = [
    (1, 256, None), (1, 1, None), (1, 37, None),
    (2, 8192, None),
    (3, 8192, 384),      # long sequences: sampled samples for the oracle
    (4, 65536, 768),
    (5, 8192, 2048),
]


@pytest.mark.parametrize("cfg,B,nsample", DIN_CASES)
def test_din_parity(models, cfg, B, nsample):
    m = models(cfg, bias=True)
    b = synth.make_batch(m, B=B)
    r = Run(m, b)
    if m.mlp_dtype == "bf16" and B <= 8192:
        # the plain bf16 weight layout (permuted on chip) gives identical results
        r2 = Run(m, b, packed=False)
        assert np.array_equal(r.att, r2.att)
    samples = None
    if nsample is not None:
        rng = np.random.default_rng(cfg)
        samples = np.sort(rng.choice(B, size=nsample, replace=False))
        samples[0] = 0
        samples[-1] = B - 1
    idx = np.arange(B) if samples is None else samples
    o = oracle_forward(m, b, samples=samples)
    tol = _tol(m)
    assert row_rel_err(r.pooled[idx], o["pooled"]) <= 1e-6
    assert row_rel_err(r.att[idx], o["att"]) <= tol
    # score-level parity and softmax weights
    sc, wt = gpu_scores_by_sample(r, idx, m.cfg.max_len)
    L = np.minimum(b.seq_lengths[idx], m.cfg.max_len)
    mask = np.arange(m.cfg.max_len)[None, :] < L[:, None]
    escale = np.max(np.abs(o["scores"][mask]))
    assert np.max(np.abs(sc[mask] - o["scores"][mask])) <= tol * escale
    assert np.max(np.abs(wt[mask] - o["weights"][mask])) <= tol
    sums = wt.sum(axis=1)
    assert np.all(np.abs(sums[L > 0] - 1.0) <= 1e-5)
    # resolved sequence rows, bit-exact
    _, seq = oracle_rows(m, b)
    assert np.array_equal(r.seq_rows[:, : b.seq_stride], seq)


def test_din_sharp_fp32(models):
    """Peaky softmax (embedding std 1, score weights x20) with the fp32 MLP:
    MLP mistakes cannot hide behind near-uniform weights.  Scores must match
    to the fp32 tolerance; the output bound is the one that score tolerance
    implies: with p = softmax(e), |d att| <= 2 max|de| max_j |s_j| per
    feature, so rows may deviate by 2 * (1e-5 * max|e|) * max|s| / |att|."""
    m = synth.make_model(synth.WORKLOADS[1], bias=True, emb_std=1.0, w3_scale=20.0)
    b = synth.make_batch(m, B=200)
    r = Run(m, b)
    o = oracle_forward(m, b)
    assert o["weights"].max() > 0.9
    sc, _ = gpu_scores_by_sample(r, np.arange(200), 100)
    mask = np.arange(100)[None, :] < b.seq_lengths[:, None]
    emax = np.max(np.abs(o["scores"][mask]))
    assert np.max(np.abs(sc[mask] - o["scores"][mask])) <= FP32_TOL * emax
    _, _, _, S = __import__("oracle_pins").torch_padded_din(m, b, o["query"],
                                                             r.seq_offsets[:-1], 100)
    de = FP32_TOL * emax
    for s in range(200):
        if b.seq_lengths[s] == 0:
            continue
        bound = 2 * de * np.abs(S[s, : b.seq_lengths[s]]).max()
        assert np.max(np.abs(r.att[s] - o["att"][s])) <= bound + FP32_TOL * np.abs(o["att"][s]).max()


def test_din_sharp_bf16_scores(models):
    """Peaky case through the bf16 matrix cores: score-level parity."""
    m = synth.make_model(synth.WORKLOADS[2], bias=True, emb_std=1.0, w3_scale=20.0)
    b = synth.make_batch(m, B=512)
    r = Run(m, b)
    o = oracle_forward(m, b)
    sc, _ = gpu_scores_by_sample(r, np.arange(512), 100)
    mask = np.arange(100)[None, :] < b.seq_lengths[:, None]
    assert np.max(np.abs(sc[mask] - o["scores"][mask])) <= BF16_TOL * np.max(np.abs(o["scores"][mask]))


@pytest.mark.parametrize("cfg", [1, 2])
def test_din_padded_equals_packed(models, cfg):
    """Padding-free means padding-blind: the same samples laid out with a
    stride of 100 positions (garbage ids in the padding) give bit-identical
    output, scores and weights."""
    m = models(cfg, bias=True)
    b = synth.make_batch(m, B=300)
    r1 = Run(m, b)
    lay = synth.padded_seq_layout(b, 100)
    r2 = Run(m, b, layout=lay)
    assert np.array_equal(r1.att, r2.att)
    assert np.array_equal(r1.scores, r2.scores)
    assert np.array_equal(r1.weights, r2.weights)


@pytest.mark.parametrize("cfg,law,C", [(1, "unif100", 16), (1, "unif100", 48), (1, "geom4", 16),
                                        (1, "unif100", 4096), (2, None, 16), (2, None, 32),
                                        (2, None, 64), (2, "unif100", 128)])
def test_din_range_sizes(models, cfg, law, C):
    """Attention ranges small enough that samples are cut between one or
    several waves of a workgroup (merged in LDS), and one group for the whole
    batch: scores do not depend on the split and outputs stay within
    tolerance."""
    m = models(cfg, bias=True)
    b = synth.make_batch(m, B=600, seq_law=law)
    r = Run(m, b, range_positions=C)
    r0 = Run(m, b)
    o = oracle_forward(m, b)
    assert np.array_equal(r.scores, r0.scores)
    assert row_rel_err(r.att, o["att"]) <= _tol(m)
    L = np.minimum(b.seq_lengths, m.cfg.max_len)
    sc, wt = gpu_scores_by_sample(r, np.arange(600), m.cfg.max_len)
    mask = np.arange(m.cfg.max_len)[None, :] < L[:, None]
    assert np.max(np.abs(wt[mask] - o["weights"][mask])) <= _tol(m)
    assert np.all(np.abs(wt.sum(axis=1)[L > 0] - 1.0) <= 1e-5)


@pytest.mark.parametrize("B,C", [(16384, 48), (8192, 48), (16384, 32)])
def test_din_three_tile_ranges(models, B, C):
    """Ranges of 33 to 48 positions (four ranges of C per group), which run
    as a round of 32 and one of 16; at B = 16384 there are more groups than
    workgroups, so a wave's next group is prefetched across the group's
    barriers.  Scores equal the default split's bit for bit; sampled outputs
    match the oracle."""
    m = models(2, bias=True)
    b = synth.make_batch(m, B=B)
    say(f"three-tile ranges B={B} C={C}")
    r = Run(m, b, range_positions=C)
    r0 = Run(m, b)
    assert np.array_equal(r.scores, r0.scores)
    samples = np.sort(np.random.default_rng(B).choice(B, size=1024, replace=False))
    o = oracle_forward(m, b, samples=samples)
    assert row_rel_err(r.att[samples], o["att"]) <= _tol(m)
    assert row_rel_err(r0.att[samples], o["att"]) <= _tol(m)


def test_din_edges(models):
    """Empty sequences, length 1, lengths at and past the cap, one sample."""
    m = models(1, bias=True)
    b = synth.make_batch(m, B=64)
    orig = b.seq_lengths.copy()
    starts = np.concatenate([[0], np.cumsum(orig)])
    L = orig.copy()
    L[0] = 0
    L[1] = 1
    L[2] = 100
    L[3] = 130        # longer than max_len: only the first 100 positions count
    L[10:20] = 0
    L[20:40] = 17
    rng = np.random.default_rng(3)
    parts = []
    for s in range(64):
        if L[s] <= orig[s]:
            parts.append(b.seq_values[:, starts[s]: starts[s] + L[s]])
        else:
            parts.append(rng.integers(-2**62, 2**62, size=(3, L[s]), dtype=np.int64))
    b.seq_values = np.ascontiguousarray(np.concatenate(parts, axis=1))
    b.seq_lengths = L.astype(np.int32)
    b.seq_stride = b.seq_values.shape[1]
    r = Run(m, b)
    o = oracle_forward(m, b)
    assert np.all(r.att[0] == 0.0) and np.all(r.att[10:20] == 0.0)
    assert row_rel_err(r.att, o["att"]) <= FP32_TOL
    # one position: weight exactly 1, output equal to that position's rows
    assert r.weights[r.packed_start[1]] == 1.0
    _, seq = oracle_rows(m, b)
    s1 = np.concatenate([m.tables[k]["values"][seq[i, r.seq_offsets[1]]]
                         for i, k in enumerate(synth.SEQ_KEYS)])
    assert np.array_equal(r.att[1], s1)


@pytest.mark.parametrize("B,nonempty", [(300, 0), (70000, 10)])
def test_din_empty_samples_zeroed(models, B, nonempty):
    """Samples without positions get exact zeros, whatever the output buffer
    held, also when there are no positions at all and when the empty samples
    outnumber the lanes of the whole launch."""
    m = models(1, bias=True)
    b = synth.make_batch(m, B=B)
    L = np.zeros(B, np.int32)
    L[:nonempty] = b.seq_lengths[:nonempty]
    keep = int(L.sum())
    b.seq_values = np.ascontiguousarray(b.seq_values[:, :max(keep, 1)])
    b.seq_lengths = L
    b.seq_stride = b.seq_values.shape[1]
    say(f"empty samples B={B} nonempty={nonempty} P={keep}")
    tabs = PL.DeviceTables(m.tables, DEV)
    fwd = PL.SparseDinForward(tabs, PL.DeviceMLP(m, DEV), B, m.cfg.max_len, DEV)
    fwd.att.fill_(float("nan"))
    fwd.run(PL.DeviceBatch(b, DEV))
    torch.cuda.synchronize()
    att = fwd.att[:B].cpu().numpy()
    assert np.all(att[nonempty:] == 0.0)
    if nonempty:
        o = oracle_forward(m, b, samples=np.arange(nonempty))
        assert row_rel_err(att[:nonempty], o["att"]) <= FP32_TOL


def test_din_deterministic(models):
    m = models(2, bias=True)
    b = synth.make_batch(m, B=4096)
    r1 = Run(m, b)
    r2 = Run(m, b)
    assert np.array_equal(r1.att, r2.att)
    assert np.array_equal(r1.pooled, r2.pooled)
    assert np.array_equal(r1.scores, r2.scores)


@pytest.mark.parametrize("R_pos", [16, 0])
def test_din_repeat_same_plan(models, R_pos):
    """The attention run three times over one plan (the arrival counters
    must come back to zero after every call) with long sequences cut into up
    to seven pieces, a block of empty sequences, and the output buffer
    poisoned between calls: identical results every time, within tolerance
    of the oracle."""
    m = models(1, bias=True)
    b = synth.make_batch(m, B=700, seq_law="unif100")
    L = b.seq_lengths.copy()
    starts = np.concatenate([[0], np.cumsum(L)])
    keep = np.ones(700, bool)
    keep[100:140] = False                      # 40 empty sequences
    parts = [b.seq_values[:, starts[s]: starts[s + 1]] for s in range(700) if keep[s]]
    b.seq_values = np.ascontiguousarray(np.concatenate(parts, axis=1))
    b.seq_lengths = np.where(keep, L, 0).astype(np.int32)
    b.seq_stride = b.seq_values.shape[1]
    r = Run(m, b, range_positions=R_pos)
    o = oracle_forward(m, b)
    assert row_rel_err(r.att, o["att"]) <= FP32_TOL
    assert np.all(r.att[100:140] == 0.0)
    att0 = r.fwd.att[:700].clone()
    for _ in range(2):
        r.fwd.att.fill_(np.nan)
        r.fwd.din_step(r.db)
        torch.cuda.synchronize()
        assert torch.equal(r.fwd.att[:700], att0)


@pytest.mark.parametrize("cfg,B,R_pos", [(1, 256, 0), (1, 37, 16), (2, 8192, 0), (3, 2000, 0),
                                         (4, 65536, 0), (5, 8192, 0), (5, 300, 16)])
def test_whole_forward_equals_calls(models, cfg, B, R_pos):
    """rec_sparse_din_fwd (four launches) against the calls one by one:
    bit-identical offsets, rows, pooled output, attention, scores and
    weights; and the oracle on the pooled output and attention."""
    m = models(cfg, bias=True)
    b = synth.make_batch(m, B=B)
    r1 = Run(m, b, range_positions=R_pos)
    r2 = Run(m, b, range_positions=R_pos, whole=True)
    for name in ("offsets", "seq_offsets", "pooled", "att", "emb_rows", "scores", "weights",
                 "seq_rows"):
        x, y = getattr(r1, name), getattr(r2, name)
        assert np.array_equal(x, y, equal_nan=True), name
    idx = np.arange(B) if B <= 8192 else np.sort(np.random.default_rng(0).choice(B, 512, replace=False))
    o = oracle_forward(m, b, samples=None if B <= 8192 else idx)
    assert row_rel_err(r2.pooled[idx], o["pooled"]) <= 1e-6
    assert row_rel_err(r2.att[idx], o["att"]) <= _tol(m)
