"""GPU parity of the DIN attention backward (rec_din_attn_bwd; "当前现状分析"
§4.2, §4.4 forward, differentiated for the run-config table's training step)
against the CPU oracle: the query gradient per sample, the gradient of every
sequence row (zero rows where no position reads), and the six weight
gradients, each per row within the fp32 tolerance.  fp32 and bf16 (plain)
weights, empty sequences, one-position sequences, positions past max_len, a
padded layout with gaps, hash tables, and the same call twice bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, FP32_TOL, row_rel_err, say, settle_relu_ties
from sparse_embedding_din_amd import pipeline as PL
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu

HASH_TINY = synth.Config(91, "hash_tiny", 64, tuple(synth.TINY_SIZES), "u123", "geom4", "f32",
                         hash_keys=(0, 1, 2, 3, 4), hash_capacity=3000)


def _case(cfg, B, seed, max_len=100, lengths=None, pad_to=None, bias=True, emb_std=0.05):
    m = synth.make_model(cfg, bias=bias, emb_std=emb_std)
    b = synth.make_batch(m, B=B)
    if lengths is not None:
        b.seq_lengths = np.asarray(lengths, np.int32)
    P = int(b.seq_lengths.sum())
    seq_values = np.ascontiguousarray(b.seq_values[:, :P]) if b.seq_values.shape[1] >= P else None
    if seq_values is None:                         # longer sequences than generated: draw more ids
        rng = np.random.default_rng(seed)
        seq_values = rng.integers(-10**12, 10**12, size=(3, P), dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(b.seq_lengths.astype(np.int64))[:-1]]).astype(np.int64)
    stride = P
    if pad_to is not None:                         # padded layout: sample b at b * pad_to
        padded = np.random.default_rng(seed + 1).integers(-10**9, 10**9, size=(3, B * pad_to),
                                                          dtype=np.int64)
        for bb in range(B):
            n = int(b.seq_lengths[bb])
            padded[:, bb * pad_to: bb * pad_to + n] = seq_values[:, offs[bb]: offs[bb] + n]
        seq_values, offs, stride = padded, np.arange(B, dtype=np.int64) * pad_to, B * pad_to
    rng = np.random.default_rng(seed)
    query = rng.normal(0, 0.08, (B, 256)).astype(np.float32)      # the pooled rows
    gatt = rng.standard_normal((B, 48)).astype(np.float32)
    return m, b, seq_values, offs, stride, query, gatt


def _gpu(m, b, seq_values, offs, stride, query, gatt, max_len, weights=True, dtype=None):
    tabs = PL.DeviceTables(m.tables, DEV)
    mlp = PL.DeviceMLP(m, DEV, dtype=dtype, packed=False)
    B = b.B
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    gq = torch.full((B, 48), 7.0, dtype=torch.float32, device=DEV)
    gs = torch.full((3, max(stride, 1), 16), 7.0, dtype=torch.float32, device=DEV)
    outs = [torch.full(s, 7.0, dtype=torch.float32, device=DEV)
            for s in ((256, 192), (256,), (64, 256), (64,), (64,), (1,))] if weights else [None] * 6
    wsb = R.rec_din_attn_bwd_workspace_bytes(stride, weights)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    R.rec_din_attn_bwd(tabs.array(list(synth.SEQ_KEYS)), to(seq_values), stride, to(offs),
                       to(b.seq_lengths), max_len, B, to(query), 256, synth.QUERY_COL, mlp.desc,
                       to(gatt), gq, gs, *outs, workspace=ws, workspace_bytes=wsb)
    torch.cuda.synchronize()
    res = dict(gq=gq.cpu().numpy(), gs=gs.cpu().numpy())
    if weights:
        for k, t in zip(("dw1", "db1", "dw2", "db2", "dw3", "db3"), outs):
            res[k] = t.cpu().numpy()
    return res


def _check(m, b, seq_values, offs, stride, query, gatt, max_len=100, weights=True, tag="",
           dtype=None):
    got = _gpu(m, b, seq_values, offs, stride, query, gatt, max_len, weights, dtype)
    q = np.concatenate([query[:, c:c + 16] for c in synth.QUERY_COL], axis=1).astype(np.float64)
    ref = oracle.get().din_bwd([m.tables[k] for k in synth.SEQ_KEYS], seq_values, stride, offs,
                               b.seq_lengths, max_len, q, m.w1, m.b1, m.w2, m.b2, m.w3, m.b3, gatt,
                               gates=True)
    nties = settle_relu_ties(got, ref, m, seq_values, offs, b.seq_lengths, max_len, q, stride)
    if nties:
        say(f"  {tag}: {nties} first-layer gate(s) within rounding of zero")
    # the query gradient sums terms that nearly cancel when a sample's
    # positions look alike (the score gradients of a sample sum to zero): its
    # error is measured per row against the size of those terms
    errs = {"gq": float(np.max(np.abs(got["gq"] - ref["gq"]).max(1) /
                               np.maximum(ref["gq_scale"].max(1), 1e-30)))}
    gs_ref = ref["gs"].reshape(stride, 3, 16).transpose(1, 0, 2)        # [3][stride][16]
    errs["gs"] = row_rel_err(got["gs"].reshape(-1, 16)[:3 * stride], gs_ref.reshape(-1, 16))
    if weights:
        for k in ("dw1", "db1", "dw2", "db2", "dw3"):
            r = ref[k].reshape(ref[k].shape[0], -1) if ref[k].ndim > 1 else ref[k].reshape(1, -1)
            errs[k] = row_rel_err(got[k].reshape(r.shape), r)
        # db3 is zero up to rounding (a common shift of the scores leaves the
        # softmax unchanged): measured against the size of its terms
        errs["db3"] = abs(float(got["db3"][0]) - ref["db3"]) / max(ref["db3_scale"], 1e-30)
    say(f"  {tag}: " + ", ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= FP32_TOL, (tag, k, v)
    return got


def test_din_bwd_tiny_fp32():
    say("din bwd tiny fp32 B=64")
    _check(*_case(synth.WORKLOADS[1], 64, 1), tag="fp32")


def test_din_bwd_sharp():
    say("din bwd sharp (embeddings std 1) B=48")
    _check(*_case(synth.WORKLOADS[1], 48, 2, emb_std=1.0), tag="sharp")


def test_din_bwd_bf16_weights():
    say("din bwd bf16 weights B=64")
    cfg = synth.WORKLOADS[2]
    small = synth.Config(cfg.index, cfg.name, 64, tuple(synth.TINY_SIZES), cfg.bag_law, cfg.seq_law,
                         cfg.mlp_dtype)
    _check(*_case(small, 64, 3), tag="bf16", dtype="bf16")


def test_din_bwd_edges():
    say("din bwd edges: empty, one position, past max_len")
    lengths = [0, 1, 3, 0, 40, 1, 7, 12]
    m, b, sv, offs, stride, q, g = _case(synth.WORKLOADS[1], 8, 4, lengths=lengths)
    got = _check(m, b, sv, offs, stride, q, g, max_len=10, tag="max_len 10")
    assert not got["gq"][0].any() and not got["gq"][3].any()
    # positions 10..39 of sample 4 are past max_len: their rows are zero
    for k in range(3):
        assert not got["gs"][k, offs[4] + 10: offs[4] + 40].any()


def test_din_bwd_long_sequences():
    """Sequences up to and past the largest max_len (128): a sample's
    positions span several workgroups of the position tiles, and the softmax
    wave holds two positions per lane."""
    say("din bwd long sequences, max_len 128")
    lengths = [0, 1, 63, 64, 65, 100, 127, 128, 129, 200, 5, 128, 96, 17, 250, 2]
    _check(*_case(synth.WORKLOADS[1], len(lengths), 10, lengths=lengths), max_len=128, tag="long")


def test_din_bwd_max_len_1024():
    """max_len at its largest (1024): sequences of several hundred positions
    and one past the cap; the softmax wave walks 64 positions per lane step."""
    say("din bwd sequences up to 1100, max_len 1024")
    lengths = [700, 0, 1024, 1, 1100, 129, 300, 64, 1023, 5]
    _check(*_case(synth.WORKLOADS[1], len(lengths), 11, lengths=lengths), max_len=1024,
           tag="max_len 1024")


def test_din_bwd_padded_layout_and_inputs_only():
    say("din bwd padded layout, no weight gradients")
    m, b, sv, offs, stride, q, g = _case(synth.WORKLOADS[1], 32, 5, pad_to=100)
    got = _check(m, b, sv, offs, stride, q, g, weights=False, tag="padded")
    L = b.seq_lengths
    for bb in range(b.B):                          # the gaps get zero rows
        assert not got["gs"][:, offs[bb] + L[bb]: offs[bb] + 100].any()


def test_din_bwd_hash():
    say("din bwd hash tables B=64")
    _check(*_case(HASH_TINY, 64, 6), tag="hash")


def test_din_bwd_deterministic():
    say("din bwd twice, bit-identical")
    args = _case(synth.WORKLOADS[1], 96, 7)
    a = _gpu(*args, 100)
    c = _gpu(*args, 100)
    for k in a:
        assert np.array_equal(a[k].view(np.uint32), c[k].view(np.uint32)), k


def test_din_bwd_full_size():
    """The Taobao-shaped batch (B = 8192, geometric lengths, full tables, bf16
    weights), every gradient against the oracle."""
    say("din bwd full size taobao_B8192")
    _check(*_case(synth.WORKLOADS[2], 8192, 8), tag="taobao_B8192", dtype="bf16")
