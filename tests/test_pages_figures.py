"""Page-printed figures (tests/golden/pages_figures.json) against the
workload definition the generator and the oracle use."""
import json
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _figs():
    with open(GOLD) as f:
        return {d["name"]: d for d in json.load(f)["figures"]}


def _close(got, fig):
    tol = fig.get("tolerance", 0.0)
    want = fig["value"]
    assert abs(got - want) <= tol * abs(want), (fig["name"], got, want)


def test_pages_figures():
    F = _figs()
    assert list(synth.FULL_SIZES[:15]) == F["num_buckets"]["value"]
    total = sum(F["num_buckets"]["value"])
    assert total == F["total_vocab_rows"]["value"]
    _close(total * synth.DIM * 4 / 2**20, F["table_megabytes"])
    assert synth.DIM == F["embedding_dim"]["value"]
    assert synth.MAX_LEN == F["seq_cap"]["value"]
    B = F["batch_size"]["value"]
    assert synth.WORKLOADS[2].B == B
    _close(B * 5 * 3 * synth.DIM, F["real_seq_elements"])
    _close(B * synth.MAX_LEN * 3 * synth.DIM, F["padded_seq_elements"])
    assert 3 * synth.DIM == F["query_width"]["value"] == F["din_output_width"]["value"]
    assert synth.DIN_IN == 4 * 3 * synth.DIM == F["attn_input_width"]["value"]
    assert [synth.HIDDEN1, synth.HIDDEN2] == F["attn_hidden"]["value"]
    assert 128 + 3 * synth.DIM == F["final_concat_width"]["value"]
    macs = synth.MAX_LEN * (synth.DIN_IN * synth.HIDDEN1 + synth.HIDDEN1 * synth.HIDDEN2 + synth.HIDDEN2)
    _close(macs, F["attn_mlp_macs_per_sample_padded"])


def test_hash_slot_layout_bytes():
    F = _figs()
    m = synth.make_model(synth.Config(92, "h", 8, tuple(synth.TINY_SIZES), "u123", "geom4", "f32",
                                      hash_keys=(0,), hash_capacity=128, hash_load=0.5))
    t = m.tables[0]
    per_slot = (t["keys"].itemsize + t["scores"].itemsize + t["digests"].itemsize
                + t["values"].shape[1] * t["values"].itemsize)
    assert per_slot == F["hash_slot_bytes"]["value"]
    _close(128 * per_slot, F["hash_min_capacity_bytes"])


def test_hash_generator_sanity():
    """Generator checks: the layout invariant (every stored key reachable by
    linear probing from its home with no empty slot in between), digests
    marking exactly the occupied slots, and the 80% hit rate of queries."""
    cfg = synth.WORKLOADS[5]
    small = synth.Config(93, "hs", 4096, tuple(synth.TINY_SIZES), "u123", "geom4", "f32",
                         hash_keys=(0, 1), hash_capacity=20000)
    m = synth.make_model(small)
    for k in small.hash_keys:
        t = m.tables[k]
        occ = t["keys"] != synth.EMPTY_KEY
        assert occ.sum() == round(small.hash_load * small.hash_capacity)
        assert np.array_equal(occ, t["digests"] != 0)
        h = synth.splitmix64_mix(t["keys"][occ])
        home = synth.home_slot(h, small.hash_capacity)
        slots = np.nonzero(occ)[0]
        assert np.array_equal(synth.digest_of(h), t["digests"][occ])
        for s, hm in zip(slots[:2000], home[:2000]):
            run = np.arange(hm, s + 1) if s >= hm else np.concatenate(
                [np.arange(hm, small.hash_capacity), np.arange(0, s + 1)])
            assert occ[run].all()
    b = synth.make_batch(m, B=small.B)
    n = b.lengths.reshape(synth.T, small.B)[0].sum()
    ids = b.values[:n]
    hit = np.isin(ids, m.tables[0]["stored"]).mean()
    sd = np.sqrt(0.8 * 0.2 / n)
    assert abs(hit - cfg.hash_hit) < 4 * sd
