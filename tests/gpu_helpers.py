"""Shared helpers for the GPU parity tests: run the HIP forward through the
C ABI on seeded inputs, run the oracle on the same inputs, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from sparse_embedding_din_amd import pipeline as PL

DEV = torch.device("cuda")

FP32_TOL = 1e-5     # max per-row relative error, fp32 MLP
BF16_TOL = 2e-2     # max per-row relative error, bf16 MLP (fp32 accumulate)


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / ||ref||_inf; rows where the
    reference is all zero must be exactly zero."""
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    scale = np.max(np.abs(ref), axis=1)
    zero = scale == 0
    assert np.all(got[zero] == 0.0), "reference-zero rows are not exactly zero"
    if (~zero).sum() == 0:
        return 0.0
    err = np.max(np.abs(got[~zero] - ref[~zero]), axis=1) / scale[~zero]
    return float(err.max())


class Run:
    """One forward on the GPU with every debug output requested."""

    def __init__(self, model, batch, range_positions=0, layout=None, debug=True, mlp_dtype=None,
                 packed=True, fused=True, whole=False):
        self.model, self.batch = model, batch
        B = batch.B
        say(f"cfg={model.cfg.name} B={B} P={batch.seq_stride} nnz={batch.values.size} "
            f"layout={'padded' if layout else 'packed'} R={range_positions} fused={fused} whole={whole}")
        self.tabs = PL.DeviceTables(model.tables, DEV)
        self.mlp = PL.DeviceMLP(model, DEV, dtype=mlp_dtype, packed=packed)
        self.fwd = PL.SparseDinForward(self.tabs, self.mlp, B, model.cfg.max_len, DEV,
                                       range_positions=range_positions, fused=fused)
        if layout is None:
            self.db = PL.DeviceBatch(batch, DEV)
            stride = batch.seq_stride
        else:
            sv, so, stride = layout
            self.db = PL.DeviceBatch(batch, DEV, seq_values=sv, seq_offsets=so, seq_stride=stride)
        self.stride = stride
        dbg = None
        if debug:
            npos = int(np.minimum(batch.seq_lengths, model.cfg.max_len).sum())
            dbg = dict(emb_rows=torch.full((max(batch.values.size, 1),), -7, dtype=torch.int64, device=DEV),
                       scores=torch.full((max(npos, 1),), np.nan, dtype=torch.float32, device=DEV),
                       weights=torch.full((max(npos, 1),), np.nan, dtype=torch.float32, device=DEV),
                       seq_rows=torch.full((3 * max(stride, 1),), -7, dtype=torch.int64, device=DEV))
        self.dbg = dbg
        if whole:
            self.fwd.run_whole(self.db, debug=dbg)
        else:
            self.fwd.run(self.db, debug=dbg)
        torch.cuda.synchronize()
        self.offsets = self.fwd.offsets[: synth.T * B + 1].cpu().numpy()
        self.seq_offsets = self.fwd.seq_offsets[: B + 1].cpu().numpy()
        self.pooled = self.fwd.pooled[:B].cpu().numpy()
        self.att = self.fwd.att[:B].cpu().numpy()
        # packed position of (b, j) = packed_start[b] + j over min(len, max_len)
        self.packed_start = oracle.get().lengths_to_offsets(
            np.minimum(batch.seq_lengths, model.cfg.max_len))
        if debug:
            self.emb_rows = dbg["emb_rows"].cpu().numpy()[: batch.values.size]
            self.scores = dbg["scores"].cpu().numpy()
            self.weights = dbg["weights"].cpu().numpy()
            self.seq_rows = dbg["seq_rows"].cpu().numpy().reshape(3, -1)
        say("done")


def oracle_forward(model, batch, samples=None, want_scores=True):
    return oracle.forward(model, batch, samples=samples, want_scores=want_scores)


def oracle_rows(model, batch):
    """Resolved rows of every deep id (key-major) and every sequence id."""
    orc = oracle.get()
    B = batch.B
    off = orc.lengths_to_offsets(batch.lengths)
    rows = np.empty(batch.values.size, np.int64)
    for k in range(synth.T):
        lo, hi = off[k * B], off[(k + 1) * B]
        rows[lo:hi] = orc.resolve(model.tables[k], batch.values[lo:hi])
    seq = np.empty_like(batch.seq_values)
    for i, k in enumerate(synth.SEQ_KEYS):
        seq[i] = orc.resolve(model.tables[k], batch.seq_values[i])
    return rows, seq


def gpu_scores_by_sample(run: Run, samples, max_len):
    """GPU scores/weights (packed positions) rearranged to [ns][max_len]."""
    b = run.batch
    starts = run.packed_start
    ns = len(samples)
    sc = np.zeros((ns, max_len))
    wt = np.zeros((ns, max_len))
    for i, s in enumerate(samples):
        L = min(int(b.seq_lengths[s]), max_len)
        sc[i, :L] = run.scores[starts[s]: starts[s] + L]
        wt[i, :L] = run.weights[starts[s]: starts[s] + L]
    return sc, wt


# A ReLU gate whose pre-activation z lies within TIE * (the size of z's
# terms) of zero is decided by rounding: fp32 sums in another order may put
# it on either side, and ReLU has no derivative at 0 to prefer one.
TIE = 2e-6


def settle_relu_ties(got, ref, m, seq_values, offs, lengths, max_len, q, stride):
    """Where the first layer's gate of unit u at position p is a tie, both
    decisions are valid: dz1[p][u] is either dh1 = W2^T dz2 (the gate open)
    or 0.  The choice moves dW1[u] by dz1 x_p, db1[u] by dz1, and through
    dx_p = W1^T dz1 the position's sequence-row gradient and its sample's
    query gradient.  For each position with ties, the decisions that bring
    the oracle's row gradient closest to the GPU's are applied to the
    oracle's results, which the usual comparison then checks in full.  A tie
    in a second-layer gate would move every first-layer gradient; those are
    counted and left as the oracle decided them, so the comparison fails if
    the GPU decided one otherwise."""
    L = np.minimum(lengths.astype(np.int64), max_len)
    real = np.concatenate([np.arange(o, o + n) for o, n in zip(offs, L)]) if len(L) else np.zeros(0, int)
    sample = np.repeat(np.arange(len(L)), L)
    ties2 = int((np.abs(ref["r2"][real]) < TIE).sum())
    if ties2:
        say(f"  {ties2} second-layer gate(s) within rounding of zero (taken as the oracle's)")
    ties = np.argwhere(np.abs(ref["r1"][real]) < TIE)
    if not len(ties):
        return 0
    orc = oracle.get()
    w1 = np.asarray(m.w1, np.float64)
    rows = []
    for i, k in enumerate(synth.SEQ_KEYS):
        tab = m.tables[k]
        vals = np.asarray(tab["values"], np.float64)
        rows.append((orc, tab, vals))
    for pi in np.unique(ties[:, 0]):
        p, bb = int(real[pi]), int(sample[pi])
        units = ties[ties[:, 0] == pi, 1]
        s = np.concatenate([(lambda r: np.zeros(16) if r < 0 else vals[r])(
            int(o.resolve(tab, np.array([seq_values[f, p]], np.int64))[0]))
            for f, (o, tab, vals) in enumerate(rows)])
        x = np.concatenate([q[bb], s, q[bb] - s, q[bb] * s])
        deltas = []
        for u in units:                      # dz1 change if the GPU decided otherwise
            v = ref["v1"][p, u]
            deltas.append((int(u), -v if ref["r1"][p, u] > 0 else v))
        best, best_err = (), np.inf
        for mask in range(1 << min(len(deltas), 6)):
            pick = [deltas[i] for i in range(len(deltas)) if mask >> i & 1]
            dx = sum((d * w1[u] for u, d in pick), np.zeros(192))
            gsp = ref["gs"][p] + dx[48:96] - dx[96:144] + q[bb] * dx[144:192]
            err = np.abs(got["gs"][:, p, :].reshape(48) - gsp).max()
            if err < best_err:
                best, best_err = pick, err
        for u, d in best:
            dx = d * w1[u]
            ref["gs"][p] += dx[48:96] - dx[96:144] + q[bb] * dx[144:192]
            ref["gq"][bb] += dx[:48] + dx[96:144] + s * dx[144:192]
            ref["dw1"][u] += d * x
            ref["db1"][u] += d
    return len(ties)
