"""Device-resident tables, MLP and batches, and the whole sparse forward as
four C-ABI calls:

    rec_kjt_sums            (deep KJT lengths -> block and chunk sums)
    rec_din_plan            (sequence lengths/ids -> packed positions, rows)
    rec_embbag_fwd_kjt      (offsets and pooled [B, 256])
    rec_din_attn_fwd_plan   (attention [B, 48], query read from the pooled output)

With fused=False the deep side is rec_lengths_to_offsets + rec_embbag_fwd.
run_whole() makes the same forward one rec_sparse_din_fwd call (three
launches, bit-identical results); din_one_call() is the attention as one
rec_din_attn_fwd call (plan and attention).

torch provides device memory and the stream; every step runs in librec.
Inputs are plain numpy arrays / dicts (as the seeded generator produces).
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np
import torch

from . import rec as R

SEQ_KEYS = (1, 5, 3)             # adgroup, cate, brand: the seq group's sub-features


def _to(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


class DeviceTables:
    """Tables on the device plus their rec_table descriptors."""

    def __init__(self, tables: Sequence[dict], device):
        self.tensors = []
        self.desc = []
        for tab in tables:
            vals = _to(np.asarray(tab["values"], np.float32), device)
            if tab["kind"] == "hash":
                keys = _to(np.asarray(tab["keys"], np.int64), device)
                dig = _to(np.asarray(tab["digests"], np.uint8), device)
                sc = _to(np.asarray(tab["scores"], np.uint64).view(np.int64), device)
                self.tensors.append((vals, keys, dig, sc))
                self.desc.append(R.table(R.REC_HASH, int(tab["rows"]), vals, keys, dig, sc))
            else:
                self.tensors.append((vals,))
                self.desc.append(R.table(R.REC_DIRECT, int(tab["rows"]), vals))

    def to_host(self, i: int) -> dict:
        """Table i copied back to host numpy arrays (the generator's dict form)."""
        t = self.tensors[i]
        out = dict(kind="hash" if len(t) == 4 else "direct", rows=int(self.desc[i].rows),
                   values=t[0].cpu().numpy())
        if len(t) == 4:
            out.update(keys=t[1].cpu().numpy(), digests=t[2].cpu().numpy(),
                       scores=t[3].cpu().numpy().view(np.uint64))
        return out

    def array(self, idx: Optional[Sequence[int]] = None):
        sel = self.desc if idx is None else [self.desc[i] for i in idx]
        arr = (R.rec_table * len(sel))()
        for i, d in enumerate(sel):
            arr[i] = d
        return arr


class DeviceMLP:
    """Attention-MLP weights on the device.  bf16 weights are pre-packed once
    (rec_din_pack_mlp) unless packed=False."""

    def __init__(self, model, device, dtype: Optional[str] = None, packed: bool = True):
        dt = dtype or getattr(model, "mlp_dtype", "f32")
        if dt == "bf16":
            self.dtype = R.REC_BF16
            self.w1 = _to(np.asarray(model.w1_bf16).view(np.int16), device)
            self.w2 = _to(np.asarray(model.w2_bf16).view(np.int16), device)
        else:
            self.dtype = R.REC_F32
            self.w1 = _to(np.asarray(model.w1, np.float32), device)
            self.w2 = _to(np.asarray(model.w2, np.float32), device)
        self.b1 = _to(np.asarray(model.b1, np.float32), device)
        self.b2 = _to(np.asarray(model.b2, np.float32), device)
        self.w3 = _to(np.asarray(model.w3, np.float32), device)
        self.b3 = float(model.b3)
        self.desc = R.din_mlp(self.dtype, self.w1, self.b1, self.w2, self.b2, self.w3, self.b3)
        if self.dtype == R.REC_BF16 and packed:
            self.packed = torch.empty(R.REC_DIN_PACKED_BYTES, dtype=torch.uint8, device=device)
            R.rec_din_pack_mlp(self.desc, self.packed, R.REC_DIN_PACKED_BYTES)
            self.dtype = R.REC_BF16_PACKED
            self.desc = R.din_mlp(self.dtype, self.packed, self.b1, None, self.b2, self.w3, self.b3)


class DeviceTowers:
    """Deep-tower and final-MLP weights on the device (plain nn.Linear layout;
    bf16 bit patterns for a bf16 model, pre-packed once with
    rec_tower_pack_mlp unless packed=False)."""

    def __init__(self, towers, device, dtype: str = "bf16", packed: bool = True):
        if dtype == "bf16":
            self.dtype = R.REC_BF16
            mats = [_to(np.asarray(towers.bits[k]).view(np.int16), device)
                    for k in ("wd1", "wd2", "wd3", "wf")]
        else:
            self.dtype = R.REC_F32
            mats = [_to(np.asarray(getattr(towers, k), np.float32), device)
                    for k in ("wd1", "wd2", "wd3", "wf")]
        self.wd1, self.wd2, self.wd3, self.wf = mats
        self.bd1, self.bd2, self.bd3, self.bf, self.wo = [
            _to(np.asarray(getattr(towers, k), np.float32), device)
            for k in ("bd1", "bd2", "bd3", "bf", "wo")]
        self.bo = float(towers.bo)
        self.desc = R.tower_mlp(self.dtype, self.wd1, self.bd1, self.wd2, self.bd2, self.wd3,
                                self.bd3, self.wf, self.bf, self.wo, self.bo)
        if self.dtype == R.REC_BF16 and packed:
            self.packed = torch.empty(R.REC_TOWER_PACKED_BYTES, dtype=torch.uint8, device=device)
            R.rec_tower_pack_mlp(self.desc, self.packed, R.REC_TOWER_PACKED_BYTES)
            self.dtype = R.REC_BF16_PACKED
            self.desc = R.tower_mlp(self.dtype, self.packed, self.bd1, None, self.bd2, None,
                                    self.bd3, None, self.bf, self.wo, self.bo)


class DeviceBatch:
    def __init__(self, batch, device, seq_values=None, seq_offsets=None, seq_stride=None):
        self.B = int(batch.B)
        self.lengths = _to(np.asarray(batch.lengths, np.int32), device)
        self.values = _to(np.asarray(batch.values, np.int64), device)
        self.nnz = int(batch.values.size)
        self.seq_lengths = _to(np.asarray(batch.seq_lengths, np.int32), device)
        sv = batch.seq_values if seq_values is None else seq_values
        self.seq_values = _to(np.asarray(sv, np.int64), device)
        self.seq_stride = int(batch.seq_stride if seq_stride is None else seq_stride)
        # an explicit sequence layout (e.g. padded); None = packed offsets from the plan
        self.seq_offsets = None if seq_offsets is None else _to(np.asarray(seq_offsets, np.int64), device)


class SparseDinForward:
    """Buffers for batches of up to B_max samples and the four-call forward."""

    def __init__(self, tables: DeviceTables, mlp: DeviceMLP, B_max: int, max_len: int = 100,
                 device="cuda", range_positions: int = 0, T: int = 16, fused: bool = True,
                 towers: Optional[DeviceTowers] = None):
        self.T = T
        self.towers = towers
        self.fused = fused
        self.tables = tables
        self.mlp = mlp
        self.max_len = max_len
        self.range_positions = range_positions
        self.B_max = B_max
        self.tab_arr = tables.array(list(range(T)))
        self.seq_arr = tables.array(list(SEQ_KEYS))
        self.query_col = (C.c_int32 * 3)(*[16 * k for k in SEQ_KEYS])
        self.offsets = torch.empty(T * B_max + 1, dtype=torch.int64, device=device)
        self.kjt_bytes = R.rec_kjt_sums_bytes(T, B_max)
        self.kjt = torch.empty(max(self.kjt_bytes, 8), dtype=torch.uint8, device=device)
        self.plan_bytes = R.rec_din_plan_bytes(B_max, max_len)
        self.plan = torch.empty(self.plan_bytes, dtype=torch.uint8, device=device)
        self.seq_offsets = torch.empty(B_max + 1, dtype=torch.int64, device=device)
        self.pooled = torch.empty(B_max, T * 16, dtype=torch.float32, device=device)
        self.fwd_ws_bytes = R.rec_sparse_din_fwd_workspace_bytes(T, B_max, max_len)
        self.fwd_ws = torch.empty(max(self.fwd_ws_bytes, 16), dtype=torch.uint8, device=device)
        self.att = torch.empty(B_max, 48, dtype=torch.float32, device=device)
        if towers is not None:
            self.deep = torch.empty(B_max, 128, dtype=torch.float32, device=device)
            self.logit = torch.empty(B_max, dtype=torch.float32, device=device)
            self.prob = torch.empty(B_max, dtype=torch.float32, device=device)

    # the four steps, each one C-ABI call
    def offsets_step(self, b: DeviceBatch, stream=None):
        if self.fused:
            R.rec_kjt_sums(b.lengths, self.T, b.B, self.kjt, self.kjt_bytes, stream)
        else:
            R.rec_lengths_to_offsets(b.lengths, self.T * b.B, self.offsets, stream)

    def plan_step(self, b: DeviceBatch, rows_out=None, stream=None):
        R.rec_din_plan(self.seq_arr, b.seq_values, b.seq_stride, b.seq_offsets, b.seq_lengths,
                       b.B, self.max_len, self.range_positions, self.seq_offsets, rows_out,
                       self.plan, self.plan_bytes, stream)

    def embbag_step(self, b: DeviceBatch, rows_out=None, stream=None):
        if self.fused:
            R.rec_embbag_fwd_kjt(self.tab_arr, self.T, b.B, b.values, b.lengths, self.kjt,
                                 self.kjt_bytes, self.offsets, self.pooled, rows_out, stream)
        else:
            R.rec_embbag_fwd(self.tab_arr, self.T, b.B, b.values, b.lengths, self.offsets,
                             self.pooled, rows_out, stream)

    def din_step(self, b: DeviceBatch, scores=None, weights=None, stream=None):
        R.rec_din_attn_fwd_plan(self.seq_arr, self.plan, self.plan_bytes, b.B, self.max_len,
                                self.pooled, self.T * 16, self.query_col, self.mlp.desc, self.att,
                                scores, weights, stream)

    def din_one_call(self, b: DeviceBatch, scores=None, weights=None, rows_out=None, stream=None):
        """The attention as one rec_din_attn_fwd call (plan built inside, in
        the plan buffer), query read from the pooled output."""
        R.rec_din_attn_fwd(self.seq_arr, b.seq_values, b.seq_stride, b.seq_offsets, b.seq_lengths,
                           self.max_len, b.B, self.pooled, self.T * 16, self.query_col,
                           self.mlp.desc, self.att, scores, weights, rows_out, self.plan,
                           self.plan_bytes, stream)

    def tower_step(self, b: DeviceBatch, stream=None):
        R.rec_towers_fwd(self.towers.desc, b.B, self.pooled, self.T * 16, self.att, self.logit,
                         deep_out=self.deep, prob=self.prob, stream=stream)

    def whole_args(self, b: DeviceBatch, debug: Optional[dict] = None) -> R.rec_fwd_args:
        """The rec_fwd_args of a batch."""
        d = debug or {}
        return R.fwd_args(self.T, b.B, self.max_len, self.tab_arr, b.values, b.lengths,
                          self.seq_arr, b.seq_values, b.seq_stride, b.seq_offsets,
                          b.seq_lengths, [16 * k for k in SEQ_KEYS], self.range_positions,
                          self.mlp.desc, self.pooled, self.att, self.fwd_ws, self.fwd_ws_bytes,
                          offsets_out=self.offsets, rows_out=d.get("emb_rows"),
                          seq_offsets_out=self.seq_offsets, seq_rows_out=d.get("seq_rows"),
                          scores_out=d.get("scores"), weights_out=d.get("weights"))

    def run_whole(self, b: DeviceBatch, stream=None, debug: Optional[dict] = None):
        """The forward as one rec_sparse_din_fwd call."""
        assert b.B <= self.B_max
        R.rec_sparse_din_fwd(self.whole_args(b, debug), stream)
        if self.towers is not None:
            self.tower_step(b, stream)
        return self.pooled[: b.B], self.att[: b.B]

    def run(self, b: DeviceBatch, stream=None, debug: Optional[dict] = None, side=None):
        """The forward on torch's current stream.  With `side` (another
        torch stream), the sequence plan runs there, concurrently with the
        offsets scan and the embedding bags, and joins before the attention."""
        assert b.B <= self.B_max
        d = debug or {}
        if side is not None:
            main = torch.cuda.current_stream()
            side.wait_stream(main)
            with torch.cuda.stream(side):
                self.plan_step(b, d.get("seq_rows"))
            self.offsets_step(b)
            self.embbag_step(b, d.get("emb_rows"))
            main.wait_stream(side)
            self.din_step(b, d.get("scores"), d.get("weights"))
            if self.towers is not None:
                self.tower_step(b)
            return self.pooled[: b.B], self.att[: b.B]
        self.offsets_step(b, stream)
        self.plan_step(b, d.get("seq_rows"), stream)
        self.embbag_step(b, d.get("emb_rows"), stream)
        self.din_step(b, d.get("scores"), d.get("weights"), stream)
        if self.towers is not None:
            self.tower_step(b, stream)
        return self.pooled[: b.B], self.att[: b.B]
