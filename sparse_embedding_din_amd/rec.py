"""Thin ctypes binding over librec.so (include/rec.h).

Argument marshalling only: every function here has the C entry point's name
and arguments; device buffers are torch tensors (or raw integer addresses),
host structs are built from plain Python values, and the stream defaults to
torch's current stream.  All computation happens in the HIP library; if it
is not built this module raises on first use, it never falls back.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librec.so")

REC_OK, REC_EINVAL, REC_EUNSUPPORTED, REC_EHIP, REC_EWORKSPACE = 0, -1, -2, -3, -4
REC_DIRECT, REC_HASH = 0, 1
REC_F32, REC_BF16, REC_BF16_PACKED = 0, 1, 2
REC_SCORE_NONE, REC_SCORE_STEP, REC_SCORE_LFU = 0, 1, 2
(REC_TIME_DIN_ATTN, REC_TIME_GATHER, REC_TIME_SUMS, REC_TIME_TOWERS,
 REC_TIME_DLRM_INTERACT, REC_TIME_DLRM_FWD, REC_TIME_KINDS) = range(7)
REC_POOL_SUM, REC_POOL_MEAN = 0, 1
REC_DIN_PACKED_BYTES = 106496
REC_TOWER_PACKED_BYTES = 614400
REC_NOALLOC_SCRATCH_BYTES = 33554432
REC_DIM = 16
REC_EMPTY_KEY = -1
REC_TOMBSTONE_KEY = -2
REC_MAX_TABLES = 32
REC_MAX_SEQ_LEN = 1024
REC_MAX_B = 16777215

EXPORTS = ["rec_din_pack_mlp", "rec_lengths_to_offsets", "rec_embbag_fwd",
           "rec_kjt_sums_bytes", "rec_kjt_sums", "rec_embbag_fwd_kjt", "rec_hash_lookup",
           "rec_hash_insert_workspace_bytes", "rec_hash_insert", "rec_hash_clear",
           "rec_hash_admit_workspace_bytes", "rec_hash_admit",
           "rec_dlrm_interact", "rec_dlrm_fwd",
           "rec_din_plan_bytes", "rec_din_plan", "rec_din_attn_workspace_bytes", "rec_din_attn_fwd",
           "rec_din_attn_fwd_plan",
           "rec_sparse_din_fwd_workspace_bytes", "rec_sparse_din_fwd", "rec_sparse_din_fwd_noalloc",
           "rec_towers_fwd",
           "rec_tower_pack_mlp", "rec_embbag_adagrad_workspace_bytes", "rec_embbag_adagrad",
           "rec_din_attn_bwd_workspace_bytes", "rec_din_attn_bwd",
           "rec_time_next_launch", "rec_last_error", "rec_version", "rec_host_floor_mod", "rec_host_hash_home",
           "rec_host_hash_probe"]


class RecError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {status}: {msg}")
        self.status = status


class rec_table(C.Structure):
    _fields_ = [("kind", C.c_int32), ("dim", C.c_int32), ("rows", C.c_int64),
                ("values", C.c_void_p), ("keys", C.c_void_p), ("digests", C.c_void_p),
                ("scores", C.c_void_p)]


class rec_din_mlp(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("reserved", C.c_int32), ("w1", C.c_void_p),
                ("b1", C.c_void_p), ("w2", C.c_void_p), ("b2", C.c_void_p),
                ("w3", C.c_void_p), ("b3", C.c_float)]


class rec_tower_mlp(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("reserved", C.c_int32),
                ("wd1", C.c_void_p), ("bd1", C.c_void_p), ("wd2", C.c_void_p), ("bd2", C.c_void_p),
                ("wd3", C.c_void_p), ("bd3", C.c_void_p), ("wf", C.c_void_p), ("bf", C.c_void_p),
                ("wo", C.c_void_p), ("bo", C.c_float)]


class rec_dlrm_mlp(C.Structure):
    _fields_ = [("n_dense", C.c_int32), ("dim", C.c_int32), ("S", C.c_int32), ("reserved", C.c_int32),
                ("wb1", C.c_void_p), ("bb1", C.c_void_p), ("wb2", C.c_void_p), ("bb2", C.c_void_p),
                ("wt1", C.c_void_p), ("bt1", C.c_void_p), ("wt2", C.c_void_p), ("bt2", C.c_void_p),
                ("wt3", C.c_void_p), ("bt3", C.c_float)]


class rec_adagrad_table(C.Structure):
    _fields_ = [("weights", C.c_void_p), ("accum", C.c_void_p), ("rows", C.c_int64),
                ("kind", C.c_int32), ("reserved", C.c_int32), ("keys", C.c_void_p),
                ("digests", C.c_void_p)]


class rec_fwd_args(C.Structure):
    _fields_ = [("T", C.c_int32), ("max_len", C.c_int32), ("B", C.c_int64),
                ("tables", C.POINTER(rec_table)), ("values", C.c_void_p), ("lengths", C.c_void_p),
                ("seq_tables", C.POINTER(rec_table)), ("seq_values", C.c_void_p),
                ("seq_stride", C.c_int64), ("seq_offsets", C.c_void_p), ("seq_lengths", C.c_void_p),
                ("query_col", C.c_int32 * 3), ("range_positions", C.c_int32),
                ("mlp", C.POINTER(rec_din_mlp)), ("pooled", C.c_void_p), ("att", C.c_void_p),
                ("offsets_out", C.c_void_p), ("rows_out", C.c_void_p),
                ("seq_offsets_out", C.c_void_p), ("seq_rows_out", C.c_void_p),
                ("scores_out", C.c_void_p), ("weights_out", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t)]


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sparse_embedding_din_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        L.rec_lengths_to_offsets.argtypes = [vp, i64, vp, vp]
        L.rec_embbag_fwd.argtypes = [C.POINTER(rec_table), i32, i64, vp, vp, vp, vp, vp, vp]
        L.rec_kjt_sums_bytes.argtypes = [i32, i64]
        L.rec_kjt_sums_bytes.restype = sz
        L.rec_kjt_sums.argtypes = [vp, i32, i64, vp, sz, vp]
        L.rec_embbag_fwd_kjt.argtypes = [C.POINTER(rec_table), i32, i64, vp, vp, vp, sz, vp, vp, vp,
                                         vp]
        L.rec_hash_lookup.argtypes = [C.POINTER(rec_table), vp, i64, vp, vp, vp]
        L.rec_hash_insert_workspace_bytes.argtypes = [i64, i64]
        L.rec_hash_insert_workspace_bytes.restype = sz
        L.rec_hash_insert.argtypes = [C.POINTER(rec_table), vp, vp, i64, i32, C.c_uint64, vp, vp,
                                      sz, vp]
        L.rec_hash_clear.argtypes = [C.POINTER(rec_table), vp]
        L.rec_hash_admit_workspace_bytes.argtypes = [i64, i64, i32]
        L.rec_hash_admit_workspace_bytes.restype = sz
        L.rec_hash_admit.argtypes = [C.POINTER(rec_table), i64, vp, vp, i64, vp, vp, i64, C.c_uint64,
                                     i32, C.c_uint64, vp, vp, vp, sz, vp]
        L.rec_dlrm_interact.argtypes = [vp, i64, i32, i32, vp, vp]
        L.rec_dlrm_fwd.argtypes = [C.POINTER(rec_dlrm_mlp), C.POINTER(rec_table),
                                   C.POINTER(C.c_int32), i64, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.rec_din_plan_bytes.argtypes = [i64, i32]
        L.rec_din_plan_bytes.restype = sz
        L.rec_din_plan.argtypes = [C.POINTER(rec_table), vp, i64, vp, vp, i64, i32, i32, vp, vp,
                                   vp, sz, vp]
        L.rec_din_attn_fwd_plan.argtypes = [C.POINTER(rec_table), vp, sz, i64, i32, vp, i64,
                                            C.POINTER(C.c_int32), C.POINTER(rec_din_mlp), vp, vp,
                                            vp, vp]
        L.rec_din_attn_workspace_bytes.argtypes = [i64, i32]
        L.rec_din_attn_workspace_bytes.restype = sz
        L.rec_din_attn_fwd.argtypes = [C.POINTER(rec_table), vp, i64, vp, vp, i32, i64, vp, i64,
                                       C.POINTER(C.c_int32), C.POINTER(rec_din_mlp), vp, vp, vp,
                                       vp, vp, sz, vp]
        L.rec_din_pack_mlp.argtypes = [C.POINTER(rec_din_mlp), vp, sz, vp]
        L.rec_sparse_din_fwd_workspace_bytes.argtypes = [i32, i64, i32]
        L.rec_sparse_din_fwd_workspace_bytes.restype = sz
        L.rec_sparse_din_fwd.argtypes = [C.POINTER(rec_fwd_args), vp]
        L.rec_sparse_din_fwd_noalloc.argtypes = [C.POINTER(rec_fwd_args), vp]
        L.rec_towers_fwd.argtypes = [C.POINTER(rec_tower_mlp), i64, vp, i64, vp, vp, vp, vp, vp]
        L.rec_tower_pack_mlp.argtypes = [C.POINTER(rec_tower_mlp), vp, sz, vp]
        L.rec_din_attn_bwd_workspace_bytes.argtypes = [i64, i32]
        L.rec_din_attn_bwd_workspace_bytes.restype = sz
        L.rec_din_attn_bwd.argtypes = [C.POINTER(rec_table), vp, i64, vp, vp, i32, i64, vp, i64,
                                       C.POINTER(C.c_int32), C.POINTER(rec_din_mlp), vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.rec_embbag_adagrad_workspace_bytes.argtypes = [i32, i64, i64, i64]
        L.rec_embbag_adagrad_workspace_bytes.restype = sz
        L.rec_embbag_adagrad.argtypes = [C.POINTER(rec_adagrad_table), i32, i64, vp, vp, vp, i64,
                                         vp, C.POINTER(C.c_int32), vp, i64, i64, vp, C.c_float,
                                         C.c_float, vp, sz, vp]
        for f in ("rec_lengths_to_offsets", "rec_embbag_fwd", "rec_kjt_sums", "rec_embbag_fwd_kjt",
                  "rec_hash_lookup", "rec_hash_insert", "rec_hash_clear", "rec_hash_admit",
                  "rec_dlrm_interact",
                  "rec_dlrm_fwd",
                  "rec_din_plan",
                  "rec_din_attn_fwd", "rec_din_attn_fwd_plan", "rec_din_pack_mlp", "rec_sparse_din_fwd",
                  "rec_sparse_din_fwd_noalloc", "rec_towers_fwd",
                  "rec_tower_pack_mlp", "rec_embbag_adagrad", "rec_din_attn_bwd"):
            getattr(L, f).restype = C.c_int
        L.rec_time_next_launch.argtypes = [i32, vp, vp]
        L.rec_time_next_launch.restype = C.c_int
        L.rec_last_error.argtypes = []
        L.rec_last_error.restype = C.c_char_p
        L.rec_version.restype = C.c_int32
        L.rec_host_floor_mod.argtypes = [i64, i64]
        L.rec_host_floor_mod.restype = i64
        L.rec_host_hash_home.argtypes = [i64, i64, C.POINTER(C.c_uint8)]
        L.rec_host_hash_home.restype = i64
        L.rec_host_hash_probe.argtypes = [vp, vp, i64, i64]
        L.rec_host_hash_probe.restype = i64
        _LIB = L
    return _LIB


def _p(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, fn: str):
    if status != REC_OK:
        raise RecError(status, fn, lib().rec_last_error().decode())


def table(kind: int, rows: int, values, keys=None, digests=None, scores=None,
          dim: int = REC_DIM) -> rec_table:
    """A host rec_table descriptor over device tensors (kept alive by the caller)."""
    return rec_table(kind, dim, rows, _p(values), _p(keys), _p(digests), _p(scores))


def din_mlp(dtype: int, w1, b1, w2, b2, w3, b3: float) -> rec_din_mlp:
    return rec_din_mlp(dtype, 0, _p(w1), _p(b1), _p(w2), _p(b2), _p(w3), float(b3))


def tower_mlp(dtype: int, wd1, bd1, wd2, bd2, wd3, bd3, wf, bf, wo, bo: float) -> rec_tower_mlp:
    return rec_tower_mlp(dtype, 0, _p(wd1), _p(bd1), _p(wd2), _p(bd2), _p(wd3), _p(bd3), _p(wf),
                         _p(bf), _p(wo), float(bo))


def _tables(tabs):
    if isinstance(tabs, C.Array):
        return tabs
    arr = (rec_table * len(tabs))()
    for i, t in enumerate(tabs):
        arr[i] = t
    return arr


def adagrad_table(weights, accum, rows: int, kind: int = REC_DIRECT, keys=None,
                  digests=None) -> rec_adagrad_table:
    """A host rec_adagrad_table over device tensors (kept alive by the caller)."""
    return rec_adagrad_table(_p(weights), _p(accum), rows, kind, 0, _p(keys), _p(digests))


# -- entry points (same names and arguments as include/rec.h) ----------------
def rec_version() -> int:
    return int(lib().rec_version())


def rec_time_next_launch(kernel: int, start=None, stop=None):
    """start/stop: torch.cuda.Event(enable_timing=True) already recorded once
    (so that the HIP event exists), or raw event handles."""
    h = [None if e is None else (e if isinstance(e, int) else e.cuda_event) for e in (start, stop)]
    _check(lib().rec_time_next_launch(kernel, h[0], h[1]), "rec_time_next_launch")


def rec_last_error() -> str:
    return lib().rec_last_error().decode()


def rec_lengths_to_offsets(lengths, n: int, offsets, stream=None):
    _check(lib().rec_lengths_to_offsets(_p(lengths), n, _p(offsets), _stream(stream)),
           "rec_lengths_to_offsets")


def rec_embbag_fwd(tables: Sequence[rec_table], T: int, B: int, values, lengths, offsets, out,
                   rows_out=None, stream=None):
    _check(lib().rec_embbag_fwd(_tables(tables), T, B, _p(values), _p(lengths), _p(offsets),
                                _p(out), _p(rows_out), _stream(stream)), "rec_embbag_fwd")


def rec_kjt_sums_bytes(T: int, B: int) -> int:
    return int(lib().rec_kjt_sums_bytes(T, B))


def rec_kjt_sums(lengths, T: int, B: int, sums, sums_bytes: int, stream=None):
    _check(lib().rec_kjt_sums(_p(lengths), T, B, _p(sums), sums_bytes, _stream(stream)),
           "rec_kjt_sums")


def rec_embbag_fwd_kjt(tables: Sequence[rec_table], T: int, B: int, values, lengths, sums,
                       sums_bytes: int, offsets_out, out, rows_out=None, stream=None):
    _check(lib().rec_embbag_fwd_kjt(_tables(tables), T, B, _p(values), _p(lengths), _p(sums),
                                    sums_bytes, _p(offsets_out), _p(out), _p(rows_out),
                                    _stream(stream)), "rec_embbag_fwd_kjt")


def rec_hash_lookup(table_: rec_table, keys, n: int, slot_out=None, rows_out=None, stream=None):
    _check(lib().rec_hash_lookup(C.byref(table_), _p(keys), n, _p(slot_out), _p(rows_out),
                                 _stream(stream)), "rec_hash_lookup")


def rec_hash_insert_workspace_bytes(n: int, capacity: int) -> int:
    return int(lib().rec_hash_insert_workspace_bytes(n, capacity))


def rec_hash_insert(table_: rec_table, keys, values, n: int, score_mode: int = REC_SCORE_NONE,
                    step: int = 0, slot_out=None, workspace=None, workspace_bytes: int = 0,
                    stream=None):
    _check(lib().rec_hash_insert(C.byref(table_) if table_ is not None else None, _p(keys),
                                 _p(values), n, score_mode, step, _p(slot_out), _p(workspace),
                                 workspace_bytes, _stream(stream)),
           "rec_hash_insert")


def rec_dlrm_interact(z, B: int, F: int, d: int, out, stream=None):
    _check(lib().rec_dlrm_interact(_p(z), B, F, d, _p(out), _stream(stream)), "rec_dlrm_interact")


def dlrm_mlp(n_dense: int, dim: int, S: int, wb1, bb1, wb2, bb2, wt1, bt1, wt2, bt2, wt3,
             bt3: float) -> rec_dlrm_mlp:
    return rec_dlrm_mlp(n_dense, dim, S, 0, _p(wb1), _p(bb1), _p(wb2), _p(bb2), _p(wt1), _p(bt1),
                        _p(wt2), _p(bt2), _p(wt3), float(bt3))


def rec_dlrm_fwd(mlp: rec_dlrm_mlp, tables: Sequence[rec_table], modes: Sequence[int], B: int,
                 dense, values, lengths, offsets, z, inter, logit, prob=None, stream=None):
    md = None if modes is None else (C.c_int32 * len(modes))(*[int(x) for x in modes])
    _check(lib().rec_dlrm_fwd(C.byref(mlp) if mlp is not None else None,
                              _tables(tables) if tables is not None else None, md, B, _p(dense),
                              _p(values), _p(lengths), _p(offsets), _p(z), _p(inter), _p(logit),
                              _p(prob), _stream(stream)),
           "rec_dlrm_fwd")


def rec_hash_admit_workspace_bytes(n: int, capacity: int, score_mode: int) -> int:
    return int(lib().rec_hash_admit_workspace_bytes(n, capacity, score_mode))


def rec_hash_admit(table_: rec_table, max_keys: int, counter_keys, counter_counts,
                   counter_capacity: int, keys, init_values, n: int, threshold: int,
                   score_mode: int, step: int = 0, slot_out=None, counts_out=None, workspace=None,
                   workspace_bytes: int = 0, stream=None):
    _check(lib().rec_hash_admit(C.byref(table_) if table_ is not None else None, max_keys,
                                _p(counter_keys), _p(counter_counts), counter_capacity, _p(keys),
                                _p(init_values), n, threshold, score_mode, step, _p(slot_out),
                                _p(counts_out), _p(workspace), workspace_bytes, _stream(stream)),
           "rec_hash_admit")


def rec_hash_clear(table_: rec_table, stream=None):
    _check(lib().rec_hash_clear(C.byref(table_) if table_ is not None else None, _stream(stream)),
           "rec_hash_clear")


def rec_din_pack_mlp(mlp: rec_din_mlp, packed, packed_bytes: int, stream=None):
    _check(lib().rec_din_pack_mlp(C.byref(mlp) if mlp is not None else None, _p(packed),
                                  packed_bytes, _stream(stream)), "rec_din_pack_mlp")


def rec_din_plan_bytes(B: int, max_len: int) -> int:
    return int(lib().rec_din_plan_bytes(B, max_len))


def rec_din_plan(seq_tables: Sequence[rec_table], seq_values, seq_stride: int, seq_offsets,
                 seq_lengths, B: int, max_len: int, range_positions: int, seq_offsets_out,
                 rows_out, plan, plan_bytes: int, stream=None):
    _check(lib().rec_din_plan(_tables(seq_tables), _p(seq_values), seq_stride, _p(seq_offsets),
                              _p(seq_lengths), B, max_len, range_positions, _p(seq_offsets_out),
                              _p(rows_out), _p(plan), plan_bytes, _stream(stream)),
           "rec_din_plan")


def rec_din_attn_workspace_bytes(B: int, max_len: int) -> int:
    return int(lib().rec_din_attn_workspace_bytes(B, max_len))


def rec_din_attn_fwd(seq_tables: Sequence[rec_table], seq_values, seq_stride: int, seq_offsets,
                     seq_lengths, max_len: int, B: int, query, query_ld: int,
                     query_col: Sequence[int], mlp: rec_din_mlp, out, scores_out=None,
                     weights_out=None, rows_out=None, workspace=None, workspace_bytes: int = 0,
                     stream=None):
    qc = None if query_col is None else (C.c_int32 * 3)(*query_col)
    _check(lib().rec_din_attn_fwd(_tables(seq_tables) if seq_tables is not None else None,
                                  _p(seq_values), seq_stride, _p(seq_offsets), _p(seq_lengths),
                                  max_len, B, _p(query), query_ld, qc,
                                  C.byref(mlp) if mlp is not None else None, _p(out),
                                  _p(scores_out), _p(weights_out), _p(rows_out), _p(workspace),
                                  workspace_bytes, _stream(stream)),
           "rec_din_attn_fwd")


def rec_din_attn_fwd_plan(seq_tables: Sequence[rec_table], plan, plan_bytes: int, B: int,
                          max_len: int, query, query_ld: int, query_col: Sequence[int],
                          mlp: rec_din_mlp, out, scores_out=None, weights_out=None, stream=None):
    qc = None if query_col is None else (C.c_int32 * 3)(*query_col)
    _check(lib().rec_din_attn_fwd_plan(_tables(seq_tables), _p(plan), plan_bytes, B, max_len,
                                       _p(query), query_ld, qc,
                                       C.byref(mlp) if mlp is not None else None, _p(out),
                                       _p(scores_out), _p(weights_out), _stream(stream)),
           "rec_din_attn_fwd_plan")


def rec_towers_fwd(mlp: rec_tower_mlp, B: int, pooled, pooled_ld: int, att, logit,
                   deep_out=None, prob=None, stream=None):
    _check(lib().rec_towers_fwd(C.byref(mlp) if mlp is not None else None, B, _p(pooled),
                                pooled_ld, _p(att), _p(deep_out), _p(logit), _p(prob),
                                _stream(stream)),
           "rec_towers_fwd")


def rec_tower_pack_mlp(mlp: rec_tower_mlp, packed, packed_bytes: int, stream=None):
    _check(lib().rec_tower_pack_mlp(C.byref(mlp) if mlp is not None else None, _p(packed),
                                    packed_bytes, _stream(stream)),
           "rec_tower_pack_mlp")


def rec_sparse_din_fwd_workspace_bytes(T: int, B: int, max_len: int) -> int:
    return int(lib().rec_sparse_din_fwd_workspace_bytes(T, B, max_len))


def fwd_args(T: int, B: int, max_len: int, tables, values, lengths, seq_tables, seq_values,
             seq_stride: int, seq_offsets, seq_lengths, query_col: Sequence[int],
             range_positions: int, mlp: rec_din_mlp, pooled, att, workspace, workspace_bytes: int,
             offsets_out=None, rows_out=None, seq_offsets_out=None, seq_rows_out=None,
             scores_out=None, weights_out=None) -> rec_fwd_args:
    """A host rec_fwd_args; `tables`/`seq_tables`/`mlp` must stay alive with it."""
    a = rec_fwd_args()
    a.T, a.max_len, a.B = T, max_len, B
    a.tables = C.cast(_tables(tables), C.POINTER(rec_table))
    a.seq_tables = C.cast(_tables(seq_tables), C.POINTER(rec_table))
    a.values, a.lengths = _p(values), _p(lengths)
    a.seq_values, a.seq_stride = _p(seq_values), seq_stride
    a.seq_offsets, a.seq_lengths = _p(seq_offsets), _p(seq_lengths)
    a.query_col = (C.c_int32 * 3)(*query_col)
    a.range_positions = range_positions
    a.mlp = C.pointer(mlp)
    a.pooled, a.att = _p(pooled), _p(att)
    a.offsets_out, a.rows_out = _p(offsets_out), _p(rows_out)
    a.seq_offsets_out, a.seq_rows_out = _p(seq_offsets_out), _p(seq_rows_out)
    a.scores_out, a.weights_out = _p(scores_out), _p(weights_out)
    a.workspace, a.workspace_bytes = _p(workspace), workspace_bytes
    return a


def rec_sparse_din_fwd(args: Optional[rec_fwd_args], stream=None):
    _check(lib().rec_sparse_din_fwd(C.byref(args) if args is not None else None, _stream(stream)),
           "rec_sparse_din_fwd")


def rec_sparse_din_fwd_noalloc(args: Optional[rec_fwd_args], stream=None):
    _check(lib().rec_sparse_din_fwd_noalloc(C.byref(args) if args is not None else None,
                                            _stream(stream)),
           "rec_sparse_din_fwd_noalloc")


def rec_host_floor_mod(x: int, n: int) -> int:
    return int(lib().rec_host_floor_mod(x, n))


def rec_host_hash_probe(keys, digests, capacity: int, key: int) -> int:
    """keys/digests: host numpy arrays (int64, uint8; digests 16-byte aligned)."""
    return int(lib().rec_host_hash_probe(keys.ctypes.data, digests.ctypes.data, capacity, key))


def rec_host_hash_home(x: int, capacity: int):
    d = C.c_uint8(0)
    home = int(lib().rec_host_hash_home(x, capacity, C.byref(d)))
    return home, int(d.value)


def rec_embbag_adagrad_workspace_bytes(T: int, B: int, nnz: int, P: int) -> int:
    return int(lib().rec_embbag_adagrad_workspace_bytes(T, B, nnz, P))


def rec_embbag_adagrad(tables, T: int, B: int, values, lengths, offsets, nnz: int, grad_pooled,
                       seq_table, seq_values, seq_stride: int, P: int, grad_seq, lr: float,
                       eps: float, workspace, workspace_bytes: int, stream=None):
    if isinstance(tables, C.Array):
        arr = tables
    else:
        arr = (rec_adagrad_table * len(tables))()
        for i, t in enumerate(tables):
            arr[i] = t
    st = None if seq_table is None else (C.c_int32 * 3)(*[int(x) for x in seq_table])
    _check(lib().rec_embbag_adagrad(arr, T, B, _p(values), _p(lengths), _p(offsets), nnz,
                                    _p(grad_pooled), st, _p(seq_values), seq_stride, P,
                                    _p(grad_seq), float(lr), float(eps), _p(workspace),
                                    workspace_bytes, _stream(stream)), "rec_embbag_adagrad")


def rec_din_attn_bwd_workspace_bytes(seq_stride: int, weight_grads: bool) -> int:
    return int(lib().rec_din_attn_bwd_workspace_bytes(seq_stride, int(bool(weight_grads))))


def rec_din_attn_bwd(seq_tables: Sequence[rec_table], seq_values, seq_stride: int, seq_offsets,
                     seq_lengths, max_len: int, B: int, query, query_ld: int, query_col,
                     mlp: rec_din_mlp, grad_att, grad_query, grad_seq=None, dw1=None, db1=None,
                     dw2=None, db2=None, dw3=None, db3=None, workspace=None,
                     workspace_bytes: int = 0, stream=None):
    qc = (C.c_int32 * 3)(*[int(x) for x in query_col])
    _check(lib().rec_din_attn_bwd(_tables(seq_tables), _p(seq_values), seq_stride, _p(seq_offsets),
                                  _p(seq_lengths), max_len, B, _p(query), query_ld, qc,
                                  C.byref(mlp), _p(grad_att), _p(grad_query), _p(grad_seq),
                                  _p(dw1), _p(db1), _p(dw2), _p(db2), _p(dw3), _p(db3),
                                  _p(workspace), workspace_bytes, _stream(stream)),
           "rec_din_attn_bwd")
