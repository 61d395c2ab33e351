"""GPU parity of the hash table's write side (rec_hash_insert, rec_hash_clear;
"集成 DynamicEmb" §6.4 rebuild from stored key/value pairs, §4.2 STEP / LFU
scores, no eviction when full) against the CPU oracle's sequential insert and
its check of the placement convention.

Inserting one key per call fixes the placement, so that case is compared
with the oracle's table slot by slot, bit for bit.  In a batch, which empty
slot a new key takes depends on the order in which lanes claim slots; there
the unique parts are compared (the stored map: every key with its values and
score, the count, every lookup) and the rest is checked for validity (the
oracle's convention check: digests, no hole between a key's home and its
slot, no key twice)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, say
from sparse_embedding_din_amd import pipeline as PL
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu
I64 = np.iinfo(np.int64)


def _keys(rng, n):
    k = np.unique(rng.integers(I64.min, I64.max, size=2 * n + 8, dtype=np.int64))
    return rng.permutation(k[k != synth.EMPTY_KEY])[:n]


def _vals(rng, n):
    return rng.standard_normal((n, 16)).astype(np.float32)


def _dev_empty(cap):
    return PL.DeviceTables([oracle.Oracle.empty_hash_table(cap)], DEV)


def _insert(dt, keys, vals, mode=R.REC_SCORE_NONE, step=0):
    k = torch.from_numpy(np.ascontiguousarray(keys, np.int64)).to(DEV)
    v = torch.from_numpy(np.ascontiguousarray(vals, np.float32).reshape(-1, 16)).to(DEV)
    slot = torch.full((max(keys.size, 1),), -9, dtype=torch.int64, device=DEV)
    wsb = R.rec_hash_insert_workspace_bytes(keys.size, int(dt.desc[0].rows))
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    R.rec_hash_insert(dt.desc[0], k, v, keys.size, mode, step, slot, ws, wsb)
    torch.cuda.synchronize()
    return slot.cpu().numpy()[: keys.size]


def _stored(tab):
    occ = np.nonzero(tab["keys"] != synth.EMPTY_KEY)[0]
    return {int(tab["keys"][s]): (tab["values"][s].tobytes(), int(tab["scores"][s])) for s in occ}


def _lookup(dt, keys):
    k = torch.from_numpy(np.ascontiguousarray(keys, np.int64)).to(DEV)
    slot = torch.empty(keys.size, dtype=torch.int64, device=DEV)
    rows = torch.empty((keys.size, 16), dtype=torch.float32, device=DEV)
    R.rec_hash_lookup(dt.desc[0], k, keys.size, slot, rows)
    torch.cuda.synchronize()
    return slot.cpu().numpy(), rows.cpu().numpy()


def test_one_key_per_call_matches_oracle():
    """Key by key the placement is unique: the GPU table equals the oracle's
    bit for bit, through new keys, assignments, LFU and STEP scores and a
    crowded cluster (half the keys share a few home slots)."""
    orc = oracle.get()
    rng = np.random.default_rng(5)
    cap = 257
    cand = _keys(rng, 20000)
    homes = synth.home_slot(synth.splitmix64_mix(cand), cap)
    crowd = cand[np.isin(homes, [3, 4, 255, 256])][:60]          # clusters, one wrapping
    keys = np.concatenate([crowd, _keys(rng, 150)])
    keys = keys[np.unique(keys, return_index=True)[1]][:200]
    vals = _vals(rng, keys.size)
    dt = _dev_empty(cap)
    ref = orc.empty_hash_table(cap)
    say(f"one-by-one cap={cap} n={keys.size}")
    for i, k in enumerate(keys):
        mode = R.REC_SCORE_LFU if i % 3 else R.REC_SCORE_STEP
        got = _insert(dt, keys[i:i + 1], vals[i:i + 1], mode, step=1000 + i)
        exp = orc.hash_insert(ref, keys[i:i + 1], vals[i:i + 1], mode, step=1000 + i)
        assert got[0] == exp[0]
    again = rng.permutation(keys)[:80]
    for i, k in enumerate(again):
        nv = _vals(rng, 1)
        assert _insert(dt, again[i:i + 1], nv, R.REC_SCORE_LFU)[0] == \
            orc.hash_insert(ref, again[i:i + 1], nv, R.REC_SCORE_LFU)[0]
    g = dt.to_host(0)
    for f in ("keys", "digests", "scores"):
        assert np.array_equal(g[f], ref[f]), f
    occ = ref["keys"] != synth.EMPTY_KEY
    assert np.array_equal(g["values"][occ], ref["values"][occ])


@pytest.mark.parametrize("cap,n", [(300000, 210000), (4099, 4000), (1000, 999), (1, 1), (64, 0)])
def test_batch_build(cap, n):
    """One call builds the table (the start-up rebuild at the headline
    table size, and nearly full small tables): a valid table holding exactly
    the pairs, every key found where its slot says, misses still miss."""
    orc = oracle.get()
    rng = np.random.default_rng(cap + n)
    keys, vals = _keys(rng, n), _vals(rng, n)
    dt = _dev_empty(cap)
    say(f"batch build cap={cap} n={n}")
    slot = _insert(dt, keys, vals, R.REC_SCORE_STEP, step=7)
    g = dt.to_host(0)
    assert orc.hash_check(g["keys"], g["digests"]) == 0
    assert np.all(slot >= 0) and np.array_equal(g["keys"][slot], keys)
    assert _stored(g) == {int(k): (v.tobytes(), 7) for k, v in zip(keys, vals)}
    if n:
        s2, rows = _lookup(dt, keys)
        assert np.array_equal(s2, slot) and np.array_equal(rows, vals)
    miss = _keys(np.random.default_rng(1), 500)
    miss = miss[~np.isin(miss, keys)]
    s3, rows3 = _lookup(dt, miss)
    assert np.all(s3 == -1) and np.all(rows3 == 0.0)


def test_assign_lfu_step():
    """Insert-or-assign on a built table: keys already stored keep their slots
    and take the new values; LFU adds one per insert, STEP overwrites; new
    keys in the same call are added; the oracle's map is the same."""
    orc = oracle.get()
    rng = np.random.default_rng(9)
    cap, n = 20011, 14000
    keys, vals = _keys(rng, n), _vals(rng, n)
    dt = _dev_empty(cap)
    ref = orc.empty_hash_table(cap)
    slot = _insert(dt, keys, vals, R.REC_SCORE_LFU)
    orc.hash_insert(ref, keys, vals, R.REC_SCORE_LFU)
    upd = rng.choice(keys, 3000, replace=False)
    fresh = _keys(np.random.default_rng(10), 2000)
    fresh = fresh[~np.isin(fresh, keys)][:1000]
    batch = np.concatenate([upd, fresh])
    nv = _vals(rng, batch.size)
    s2 = _insert(dt, batch, nv, R.REC_SCORE_LFU)
    orc.hash_insert(ref, batch, nv, R.REC_SCORE_LFU)
    where = {int(k): int(s) for k, s in zip(keys, slot)}
    assert s2[: upd.size].tolist() == [where[int(k)] for k in upd]
    s3 = _insert(dt, upd[:500], nv[:500], R.REC_SCORE_STEP, step=99)
    orc.hash_insert(ref, upd[:500], nv[:500], R.REC_SCORE_STEP, step=99)
    g = dt.to_host(0)
    assert orc.hash_check(g["keys"], g["digests"]) == 0
    assert _stored(g) == _stored(ref)
    assert np.all(g["scores"][s3] == 99) and np.all(g["scores"][s2[500: upd.size]] == 2)


def test_full_table_stores_no_more():
    """More distinct keys than slots: exactly `capacity` are stored, the rest
    report -1 and change nothing; keys already stored are still assigned."""
    orc = oracle.get()
    rng = np.random.default_rng(11)
    cap = 1000
    keys, vals = _keys(rng, 1300), _vals(rng, 1300)
    dt = _dev_empty(cap)
    slot = _insert(dt, keys, vals)
    g = dt.to_host(0)
    assert np.sum(slot >= 0) == cap and np.sum(slot == -1) == 300
    assert np.all(g["keys"] != synth.EMPTY_KEY)
    assert orc.hash_check(g["keys"], g["digests"]) == 0
    put = slot >= 0
    assert np.array_equal(np.sort(g["keys"]), np.sort(keys[put]))
    assert _stored(g) == {int(k): (v.tobytes(), 0) for k, v in zip(keys[put], vals[put])}
    nv = _vals(rng, 10)
    s2 = _insert(dt, keys[put][:10], nv)
    assert np.array_equal(s2, slot[put][:10])
    assert np.array_equal(dt.to_host(0)["values"][s2], nv)


def test_empty_marker_and_duplicates():
    """The empty marker is refused (-2); a key given twice in one call is
    stored once with the values of its last occurrence (as inserting the
    pairs in order leaves it: the oracle's map), and LFU counts both."""
    orc = oracle.get()
    rng = np.random.default_rng(13)
    base = _keys(rng, 300)
    keys = np.concatenate([base, base[:100], [synth.EMPTY_KEY]])
    vals = _vals(rng, keys.size)
    dt = _dev_empty(1021)
    slot = _insert(dt, keys, vals, R.REC_SCORE_LFU)
    ref = orc.empty_hash_table(1021)
    orc.hash_insert(ref, keys, vals, R.REC_SCORE_LFU)
    g = dt.to_host(0)
    assert slot[-1] == -2 and orc.hash_check(g["keys"], g["digests"]) == 0
    assert np.array_equal(slot[300:400], slot[:100])
    assert np.sum(g["keys"] != synth.EMPTY_KEY) == 300
    for i in range(100):
        assert np.array_equal(g["values"][slot[i]], vals[300 + i])
        assert g["scores"][slot[i]] == 2
    assert np.all(g["scores"][slot[100:300]] == 1)
    assert _stored(g) == _stored(ref)


@pytest.mark.parametrize("reps", [2, 5])
def test_duplicates_across_workgroups_last_wins(reps):
    """Each key appears `reps` times, its occurrences thousands of pairs
    apart (so in different workgroups) with values that differ in every
    16-byte piece: the stored row is exactly that of the last occurrence,
    never a mix, and the map equals the oracle's sequential insert."""
    orc = oracle.get()
    rng = np.random.default_rng(100 + reps)
    base = _keys(rng, 3000)
    keys = np.concatenate([rng.permutation(base) for _ in range(reps)])
    vals = np.repeat(np.arange(keys.size, dtype=np.float32)[:, None], 16, axis=1)
    vals += np.arange(16, dtype=np.float32)[None, :] * 1e-3          # every float4 differs
    cap = 4099
    dt = _dev_empty(cap)
    say(f"duplicates x{reps} across workgroups n={keys.size}")
    slot = _insert(dt, keys, vals, R.REC_SCORE_LFU)
    ref = orc.empty_hash_table(cap)
    orc.hash_insert(ref, keys, vals, R.REC_SCORE_LFU)
    g = dt.to_host(0)
    assert orc.hash_check(g["keys"], g["digests"]) == 0
    assert _stored(g) == _stored(ref)
    last = {int(k): i for i, k in enumerate(keys)}
    for k, i in list(last.items())[:500]:
        assert np.array_equal(g["values"][slot[i]], vals[i])
    assert np.all(g["scores"][slot[:3000]] == reps)


def test_clear_then_rebuild_gives_same_forward():
    """The start-up rebuild: clear each hash table of the hash workload and
    insert its stored pairs on the GPU; the whole forward then gives
    bit-identical pooled and attention outputs to the generator's tables
    (slots may differ, every lookup does not)."""
    orc = oracle.get()
    m = synth.make_model(synth.WORKLOADS[5])
    b = synth.make_batch(m, B=4096)
    say("rebuild hash workload B=4096")
    ref_tabs = PL.DeviceTables(m.tables, DEV)
    gpu_tabs = PL.DeviceTables(m.tables, DEV)
    for k in synth.WORKLOADS[5].hash_keys:
        R.rec_hash_clear(gpu_tabs.desc[k])
        torch.cuda.synchronize()
        cleared = gpu_tabs.to_host(k)
        assert np.all(cleared["keys"] == synth.EMPTY_KEY) and np.all(cleared["digests"] == 0)
        assert np.all(cleared["scores"] == 0)
        t = m.tables[k]
        occ = np.nonzero(t["keys"] != synth.EMPTY_KEY)[0]
        kk = torch.from_numpy(t["keys"][occ]).to(DEV)
        vv = torch.from_numpy(np.ascontiguousarray(t["values"][occ])).to(DEV)
        wsb = R.rec_hash_insert_workspace_bytes(occ.size, int(gpu_tabs.desc[k].rows))
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        R.rec_hash_insert(gpu_tabs.desc[k], kk, vv, occ.size, R.REC_SCORE_STEP, 1, None, ws, wsb)
        torch.cuda.synchronize()
        g = gpu_tabs.to_host(k)
        assert orc.hash_check(g["keys"], g["digests"]) == 0
        assert {kk_: v for kk_, (v, _) in _stored(g).items()} == \
            {int(t["keys"][s]): t["values"][s].tobytes() for s in occ}
    mlp = PL.DeviceMLP(m, DEV)
    outs = []
    for tabs in (ref_tabs, gpu_tabs):
        fwd = PL.SparseDinForward(tabs, mlp, b.B, m.cfg.max_len, DEV)
        fwd.run_whole(PL.DeviceBatch(b, DEV))
        torch.cuda.synchronize()
        outs.append((fwd.pooled[: b.B].cpu().numpy(), fwd.att[: b.B].cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
