"""CPU oracle (test infrastructure only).

Python face of oracle/oracle.c, a plain fp64 C statement of the sparse
embedding + DIN attention forward.  Only tests, the smoke check and the
benchmark's CPU-baseline leg may import this package; the HIP library never
does, and this package imports nothing from it.

Inputs are numpy arrays from the seeded generator (synth); results are fp64.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

P64 = C.POINTER(C.c_int64)
P32 = C.POINTER(C.c_int32)
PF = C.POINTER(C.c_float)
PD = C.POINTER(C.c_double)
P8 = C.POINTER(C.c_uint8)
PU = C.POINTER(C.c_uint64)


class OrcTable(C.Structure):
    _fields_ = [("kind", C.c_int32), ("pad_", C.c_int32), ("rows", C.c_int64),
                ("values", PF), ("sorted_keys", P64), ("sorted_slots", P64),
                ("count", C.c_int64)]


def build(src: str = SRC, out: str = LIB) -> str:
    """gcc -O2, no fast-math: IEEE fp64 in source order."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class Oracle:
    def __init__(self, path: Optional[str] = None):
        path = path or LIB
        if path == LIB and (not os.path.exists(LIB) or
                            os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build()
        self.lib = L = C.CDLL(path)
        L.orc_lengths_to_offsets.argtypes = [P32, C.c_int64, P64]
        L.orc_lengths_to_offsets.restype = None
        L.orc_floor_mod.argtypes = [C.c_int64, C.c_int64]
        L.orc_floor_mod.restype = C.c_int64
        L.orc_hash_index.argtypes = [P64, C.c_int64, P64, P64]
        L.orc_hash_index.restype = C.c_int64
        L.orc_hash_find.argtypes = [P64, P64, C.c_int64, C.c_int64]
        L.orc_hash_find.restype = C.c_int64
        L.orc_resolve_many.argtypes = [C.POINTER(OrcTable), P64, C.c_int64, P64]
        L.orc_resolve_many.restype = None
        L.orc_embbag.argtypes = [C.c_int32, C.c_int64, C.POINTER(OrcTable), P64, P32, P64,
                                 P64, C.c_int64, PD]
        L.orc_embbag.restype = None
        L.orc_din.argtypes = [C.POINTER(OrcTable), P64, C.c_int64, P64, P32, C.c_int32,
                              PD, PD, PD, PD, PD, PD, C.c_double, P64, C.c_int64, PD, PD, PD]
        L.orc_din.restype = None
        L.orc_towers.argtypes = [C.c_int64, PD, C.c_int64, PD, PD, PD, PD, PD, PD, PD, PD, PD,
                                 PD, C.c_double, PD, PD, PD, PD]
        L.orc_towers.restype = None
        L.orc_hash_insert.argtypes = [P64, P8, PU, PF, C.c_int64, P64, PF, C.c_int64, C.c_int32,
                                      C.c_uint64, P64]
        L.orc_hash_insert.restype = None
        L.orc_hash_check.argtypes = [P64, P8, C.c_int64]
        L.orc_hash_check.restype = C.c_int64
        L.orc_dlrm_interact.argtypes = [PF, C.c_int64, C.c_int32, C.c_int32, PD, PD]
        L.orc_dlrm_interact.restype = None
        L.orc_embbag_adagrad.argtypes = [C.c_int32, C.c_int64, C.POINTER(OrcTable), P64, P64, P32,
                                         P64, PF,
                                         C.c_int64, P32, P64, C.c_int64, PF, C.c_double,
                                         C.c_double, PD, PD, PD, P8]
        L.orc_embbag_adagrad.restype = C.c_int64
        L.orc_din_bwd.argtypes = [C.POINTER(OrcTable), P64, C.c_int64, P64, P32, C.c_int32,
                                  C.c_int64, PD, PD, PD, PD, PD, PD, C.c_double, PD, PD, PD,
                                  PD, PD, PD, PD, PD, PD, PD, PD, PD]
        L.orc_din_bwd.restype = None
        L.orc_dlrm_fwd.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.c_int32, PD, PD, PD, PD, PD,
                                   P64, C.POINTER(PF), P32, P64, P32, P64, PD, PD, PD, PD, PD,
                                   C.c_double, PD, PD, PD, PD, PD, PD]
        L.orc_dlrm_fwd.restype = None
        L.orc_hash_admit.argtypes = [P64, P8, PU, PF, C.c_int64, C.c_int64, P64, PU, C.c_int64, P64,
                                     PF, C.c_int64, C.c_uint64, C.c_int32, C.c_uint64, P64, P64]
        L.orc_hash_admit.restype = None
        self._keep = []

    # -- bookkeeping ---------------------------------------------------------
    def lengths_to_offsets(self, lengths: np.ndarray) -> np.ndarray:
        lengths = np.ascontiguousarray(lengths, dtype=np.int32)
        out = np.empty(lengths.size + 1, dtype=np.int64)
        self.lib.orc_lengths_to_offsets(_ptr(lengths, P32), lengths.size, _ptr(out, P64))
        return out

    def floor_mod(self, raw: int, n: int) -> int:
        return int(self.lib.orc_floor_mod(int(raw), int(n)))

    # -- hash tables: the insert side ------------------------------------------
    SCORE_NONE, SCORE_STEP, SCORE_LFU = 0, 1, 2

    @staticmethod
    def empty_hash_table(capacity: int) -> dict:
        """An empty table in the generator's dict form (keys -1, digests 0,
        scores 0; values NaN so that a read of an empty slot shows)."""
        return dict(kind="hash", rows=capacity,
                    keys=np.full(capacity, -1, np.int64), digests=np.zeros(capacity, np.uint8),
                    scores=np.zeros(capacity, np.uint64),
                    values=np.full((capacity, 16), np.nan, np.float32))

    def hash_insert(self, tab: dict, keys: np.ndarray, vals: np.ndarray, mode: int = 0,
                    step: int = 0) -> np.ndarray:
        """Insert-or-assign (keys[i], vals[i]) in order into `tab` in place
        (its keys, digests, scores and values arrays); returns each key's
        slot, -1 when the table was full, -2 for the empty marker."""
        keys = np.ascontiguousarray(keys, np.int64)
        vals = np.ascontiguousarray(vals, np.float32).reshape(-1, 16)
        assert vals.shape[0] == keys.size
        for k, t in (("keys", np.int64), ("digests", np.uint8), ("scores", np.uint64),
                     ("values", np.float32)):
            assert tab[k].dtype == t and tab[k].flags.c_contiguous, k
        cap = int(tab["rows"])
        out = np.empty(keys.size, np.int64)
        self.lib.orc_hash_insert(_ptr(tab["keys"], P64), _ptr(tab["digests"], P8),
                                 _ptr(tab["scores"], PU), _ptr(tab["values"], PF), cap,
                                 _ptr(keys, P64), _ptr(vals, PF), keys.size, int(mode),
                                 int(step), _ptr(out, P64))
        return out

    @staticmethod
    def empty_counter_table(capacity: int) -> dict:
        """An empty admission counter table: keys -1, counts 0."""
        return dict(rows=capacity, keys=np.full(capacity, -1, np.int64),
                    counts=np.zeros(capacity, np.uint64))

    def hash_admit(self, tab: dict, counter: dict, keys: np.ndarray, init_vals: np.ndarray,
                   threshold: int, mode: int, step: int = 0, max_keys: Optional[int] = None):
        """One admission step ("集成 DynamicEmb" §4.1, §4.2) in place on `tab`
        (keys, digests, scores, values) and `counter` (keys, counts).
        Returns (slot of every key after the call, [admitted, evicted,
        candidates left out])."""
        keys = np.ascontiguousarray(keys, np.int64)
        init_vals = np.ascontiguousarray(init_vals, np.float32).reshape(-1, 16)
        assert init_vals.shape[0] == keys.size
        for k, t in (("keys", np.int64), ("digests", np.uint8), ("scores", np.uint64),
                     ("values", np.float32)):
            assert tab[k].dtype == t and tab[k].flags.c_contiguous, k
        assert counter["keys"].dtype == np.int64 and counter["counts"].dtype == np.uint64
        cap = int(tab["rows"])
        mk = cap if max_keys is None else int(max_keys)
        out = np.empty(keys.size, np.int64)
        counts = np.zeros(3, np.int64)
        self.lib.orc_hash_admit(_ptr(tab["keys"], P64), _ptr(tab["digests"], P8),
                                _ptr(tab["scores"], PU), _ptr(tab["values"], PF), cap, mk,
                                _ptr(counter["keys"], P64), _ptr(counter["counts"], PU),
                                int(counter["rows"]), _ptr(keys, P64), _ptr(init_vals, PF),
                                keys.size, int(threshold), int(mode), int(step), _ptr(out, P64),
                                _ptr(counts, P64))
        return out, counts

    @staticmethod
    def hash_find_slow(tab: dict, key: int) -> int:
        """The slot holding `key`, by a scan of every slot (-1 if none)."""
        hit = np.nonzero(tab["keys"] == key)[0]
        return int(hit[0]) if hit.size else -1

    def hash_check(self, keys: np.ndarray, digests: np.ndarray) -> int:
        """Number of slots that break the table convention (0 for a valid table)."""
        keys = np.ascontiguousarray(keys, np.int64)
        digests = np.ascontiguousarray(digests, np.uint8)
        return int(self.lib.orc_hash_check(_ptr(keys, P64), _ptr(digests, P8), keys.size))

    # -- backward of the bags + sparse AdaGrad ------------------------------------
    def embbag_adagrad(self, tabs, B: int, values, lengths, offsets, dpooled, weights, accums,
                       lr: float = 1e-3, eps: float = 1e-10, seq=None):
        """One sparse AdaGrad step of T tables from the gradient of the
        sum-pooled output, dpooled [B][T*16] (fp32), and optionally of the
        unpooled sequence rows: seq = (seq_table [3], seq_values [3][>=P],
        dseq [3][P][16] fp32).  tabs: generator table dicts (direct or hash;
        a hash table's rows are its slots), or plain row counts for direct
        tables.  weights / accums: T arrays [rows][16] (not modified).
        Returns (new weights, new accums, summed gradient, touched mask),
        lists of T fp64 arrays (mask: bool)."""
        T = len(tabs)
        tabs = [dict(kind="direct", rows=int(t), values=np.zeros((1, 16), np.float32))
                if isinstance(t, (int, np.integer)) else t for t in tabs]
        wrapped = self.tables(tabs)
        rows = np.array([int(t["rows"]) for t in tabs], dtype=np.int64)
        base = np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(np.int64)
        R = int(rows.sum())
        values = np.ascontiguousarray(values, dtype=np.int64)
        lengths = np.ascontiguousarray(lengths, dtype=np.int32)
        offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        dp = np.ascontiguousarray(dpooled, dtype=np.float32).reshape(B, T * 16)
        assert lengths.size == T * B and offsets.size >= T * B
        w = np.concatenate([np.asarray(a, np.float64).reshape(-1, 16) for a in weights])
        G = np.concatenate([np.asarray(a, np.float64).reshape(-1, 16) for a in accums])
        assert w.shape == (R, 16) and G.shape == (R, 16)
        grad = np.zeros((R, 16), np.float64)
        touched = np.zeros(R, np.uint8)
        if seq is None:
            P, st, sv, ds, stride = 0, np.zeros(3, np.int32), np.zeros(1, np.int64), \
                np.zeros(1, np.float32), 0
        else:
            st = np.ascontiguousarray(seq[0], dtype=np.int32)
            sv = np.ascontiguousarray(seq[1], dtype=np.int64)
            ds = np.ascontiguousarray(seq[2], dtype=np.float32)
            P = ds.shape[1]
            stride = sv.shape[1]
            assert st.shape == (3,) and ds.shape == (3, P, 16) and sv.shape[0] == 3 and stride >= P
            assert np.all((st >= 0) & (st < T))
        outside = self.lib.orc_embbag_adagrad(T, B, wrapped, _ptr(base, P64), _ptr(values, P64),
                                    _ptr(lengths, P32), _ptr(offsets, P64), _ptr(dp, PF), P,
                                    _ptr(st, P32), _ptr(sv, P64), stride, _ptr(ds, PF),
                                    float(lr), float(eps), _ptr(w, PD), _ptr(G, PD),
                                    _ptr(grad, PD), _ptr(touched, P8))
        assert outside == 0, f"{outside} reads resolved to a row outside their table"
        cut = lambda a: [a[base[t]: base[t] + rows[t]] for t in range(T)]  # noqa: E731
        return cut(w), cut(G), cut(grad), cut(touched.astype(bool))

    def din_bwd(self, seq_tabs, seq_values, seq_stride, seq_offsets, seq_lengths, max_len, query,
                w1, b1, w2, b2, w3, b3, gatt, wrapped=None, gates=False):
        """Backward of the DIN attention for all B samples given the gradient
        of its output gatt [B][48].  Returns a dict of fp64 arrays: gq [B][48],
        gs [seq_stride][48] (by position index), dw1 [256][192], db1 [256],
        dw2 [64][256], db2 [64], dw3 [64], db3 (a float), db3_scale (sum |de_j|,
        the size of db3's terms: db3 itself is zero up to rounding), gq_scale
        [B][48] (the size of each query-gradient entry's terms).  With gates,
        also r1 [seq_stride][256] = z1 / (the size of z1's terms), v1
        [seq_stride][256] = W2^T dz2 before the first ReLU gate, r2
        [seq_stride][64] = z2 / (the size of its terms): the ReLU gates within
        rounding of zero, where either derivative is valid."""
        seq_values = np.ascontiguousarray(seq_values, dtype=np.int64)
        seq_offsets = np.ascontiguousarray(seq_offsets, dtype=np.int64)
        seq_lengths = np.ascontiguousarray(seq_lengths, dtype=np.int32)
        B = seq_lengths.size
        q = np.ascontiguousarray(query, dtype=np.float64).reshape(B, 48)
        g = np.ascontiguousarray(gatt, dtype=np.float64).reshape(B, 48)
        d = [np.ascontiguousarray(a, dtype=np.float64) for a in (w1, b1, w2, b2, w3)]
        assert d[0].shape == (256, 192) and d[2].shape == (64, 256)
        arr = wrapped if wrapped is not None else self.tables(seq_tabs)
        out = dict(gq=np.empty((B, 48)), gs=np.empty((int(seq_stride), 48)),
                   dw1=np.zeros((256, 192)), db1=np.zeros(256), dw2=np.zeros((64, 256)),
                   db2=np.zeros(64), dw3=np.zeros(64), db3=np.zeros(1), db3_scale=np.zeros(1),
                   gq_scale=np.empty((B, 48)))
        gate = np.empty((int(seq_stride), 576)) if gates else None
        self.lib.orc_din_bwd(arr, _ptr(seq_values, P64), int(seq_stride), _ptr(seq_offsets, P64),
                             _ptr(seq_lengths, P32), int(max_len), B, _ptr(q, PD),
                             *[_ptr(x, PD) for x in d], float(b3), _ptr(g, PD),
                             *[_ptr(out[k], PD) for k in ("gq", "gs", "dw1", "db1", "dw2", "db2",
                                                          "dw3", "db3", "db3_scale", "gq_scale")],
                             _ptr(gate, PD) if gates else None)
        if gates:
            out["r1"], out["v1"], out["r2"] = gate[:, :256], gate[:, 256:512], gate[:, 512:]
        out["db3"] = float(out["db3"][0])
        out["db3_scale"] = float(out["db3_scale"][0])
        return out

    # -- DLRM interaction --------------------------------------------------------
    def dlrm_interact(self, z: np.ndarray, want_scale: bool = False):
        """z [B][F][d] fp32 -> the upper triangle (with the diagonal) of each
        sample's Gram matrix, [B][F(F+1)/2] fp64, row by row; with want_scale
        also sum_k |z_ik z_jk| per entry."""
        z = np.ascontiguousarray(z, np.float32)
        B, F, d = z.shape
        out = np.empty((B, F * (F + 1) // 2), np.float64)
        sc = np.empty_like(out) if want_scale else None
        self.lib.orc_dlrm_interact(_ptr(z, PF), B, F, d, _ptr(out, PD),
                                   None if sc is None else _ptr(sc, PD))
        return (out, sc) if want_scale else out

    # -- DLRM forward ------------------------------------------------------------
    def dlrm_fwd(self, m, dense, values, lengths, offsets=None):
        """The DLRM forward of a model m (attributes wb1, bb1, wb2, bb2, tables
        (S arrays [rows][d] fp32), modes (S ints: 0 sum, 1 mean), wt1, bt1,
        wt2, bt2, wt3, bt3; weights as the GPU receives them) on dense [B][nd]
        and the key-major KJT (values, lengths [S*B], offsets [S*B] or None
        for the exclusive scan of lengths).  Returns a dict of fp64 arrays:
        z [B][S+1][d], inter [B][npairs], logit [B], prob [B], lscale [B]
        (|bt3| + sum |wt3_i t2_i|) and iscale [B][npairs] (sum_k |z_ik z_jk|)."""
        dense = np.ascontiguousarray(dense, np.float64)
        B, nd = dense.shape
        S = len(m.tables)
        d = int(m.tables[0].shape[1])
        F = S + 1
        npairs = F * (F + 1) // 2
        values = np.ascontiguousarray(values, np.int64)
        lengths = np.ascontiguousarray(lengths, np.int32)
        assert lengths.size == S * B
        if offsets is None:
            offsets = self.lengths_to_offsets(lengths)[:-1]
        offsets = np.ascontiguousarray(offsets, np.int64)
        tabs = [np.ascontiguousarray(t, np.float32) for t in m.tables]
        assert all(t.ndim == 2 and t.shape[1] == d for t in tabs)
        rows = np.array([t.shape[0] for t in tabs], np.int64)
        ptrs = (PF * S)(*[_ptr(t, PF) for t in tabs])
        modes = np.ascontiguousarray(m.modes, np.int32)
        w = [np.ascontiguousarray(getattr(m, k), np.float64)
             for k in ("wb1", "bb1", "wb2", "bb2", "wt1", "bt1", "wt2", "bt2", "wt3")]
        assert w[0].shape == (128, nd) and w[2].shape == (d, 128)
        assert w[4].shape == (128, npairs) and w[6].shape == (64, 128) and w[8].shape == (64,)
        out = dict(z=np.empty((B, F, d)), inter=np.empty((B, npairs)), logit=np.empty(B),
                   prob=np.empty(B), lscale=np.empty(B), iscale=np.empty((B, npairs)))
        self.lib.orc_dlrm_fwd(B, nd, d, S, _ptr(dense, PD), *[_ptr(x, PD) for x in w[:4]],
                              _ptr(rows, P64), ptrs, _ptr(modes, P32), _ptr(values, P64),
                              _ptr(lengths, P32), _ptr(offsets, P64),
                              *[_ptr(x, PD) for x in w[4:]], float(m.bt3),
                              *[_ptr(out[k], PD) for k in ("z", "inter", "logit", "prob", "lscale",
                                                           "iscale")])
        return out

    # -- tables --------------------------------------------------------------
    def table(self, tab: dict) -> OrcTable:
        """Wrap one generator table (dict from synth) for the C side."""
        vals = np.ascontiguousarray(tab["values"], dtype=np.float32)
        t = OrcTable()
        t.rows = int(tab["rows"])
        t.values = _ptr(vals, PF)
        keep = [vals]
        if tab["kind"] == "hash":
            keys = np.ascontiguousarray(tab["keys"], dtype=np.int64)
            sk = np.empty(keys.size, dtype=np.int64)
            sl = np.empty(keys.size, dtype=np.int64)
            cnt = self.lib.orc_hash_index(_ptr(keys, P64), keys.size, _ptr(sk, P64), _ptr(sl, P64))
            t.kind = 1
            t.sorted_keys = _ptr(sk, P64)
            t.sorted_slots = _ptr(sl, P64)
            t.count = cnt
            keep += [keys, sk, sl]
        else:
            t.kind = 0
            t.count = 0
        t._keep = keep
        return t

    def tables(self, tabs: Sequence[dict]):
        arr = (OrcTable * len(tabs))()
        keep = []
        for i, tab in enumerate(tabs):
            w = self.table(tab)
            arr[i] = w
            keep.append(w._keep)
        arr._keep = keep
        return arr

    def resolve(self, tab: dict, raw: np.ndarray, wrapped=None) -> np.ndarray:
        raw = np.ascontiguousarray(raw, dtype=np.int64)
        t = wrapped if wrapped is not None else self.table(tab)
        out = np.empty(raw.size, dtype=np.int64)
        self.lib.orc_resolve_many(C.byref(t), _ptr(raw, P64), raw.size, _ptr(out, P64))
        return out

    # -- forward pieces ------------------------------------------------------
    def embbag(self, tabs, B: int, values, lengths, offsets, samples=None, wrapped=None):
        T = len(tabs)
        values = np.ascontiguousarray(values, dtype=np.int64)
        lengths = np.ascontiguousarray(lengths, dtype=np.int32)
        offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        samples = np.arange(B, dtype=np.int64) if samples is None else \
            np.ascontiguousarray(samples, dtype=np.int64)
        arr = wrapped if wrapped is not None else self.tables(tabs)
        out = np.empty((samples.size, T * 16), dtype=np.float64)
        self.lib.orc_embbag(T, B, arr, _ptr(values, P64), _ptr(lengths, P32),
                            _ptr(offsets, P64), _ptr(samples, P64), samples.size,
                            _ptr(out, PD))
        return out

    def din(self, seq_tabs, seq_values, seq_stride, seq_offsets, seq_lengths, max_len,
            query, w1, b1, w2, b2, w3, b3, samples=None, wrapped=None,
            want_scores=False):
        """query: [ns][48] fp64 for the sampled samples (in `samples` order)."""
        seq_values = np.ascontiguousarray(seq_values, dtype=np.int64)
        seq_offsets = np.ascontiguousarray(seq_offsets, dtype=np.int64)
        seq_lengths = np.ascontiguousarray(seq_lengths, dtype=np.int32)
        B = seq_lengths.size
        samples = np.arange(B, dtype=np.int64) if samples is None else \
            np.ascontiguousarray(samples, dtype=np.int64)
        q = np.ascontiguousarray(query, dtype=np.float64).reshape(samples.size, 48)
        d = [np.ascontiguousarray(a, dtype=np.float64) for a in (w1, b1, w2, b2, w3)]
        assert d[0].shape == (256, 192) and d[2].shape == (64, 256)
        arr = wrapped if wrapped is not None else self.tables(seq_tabs)
        att = np.empty((samples.size, 48), dtype=np.float64)
        sc = np.empty((samples.size, max(max_len, 1)), dtype=np.float64) if want_scores else None
        wt = np.empty((samples.size, max(max_len, 1)), dtype=np.float64) if want_scores else None
        self.lib.orc_din(arr, _ptr(seq_values, P64), int(seq_stride), _ptr(seq_offsets, P64),
                         _ptr(seq_lengths, P32), int(max_len), _ptr(q, PD),
                         _ptr(d[0], PD), _ptr(d[1], PD), _ptr(d[2], PD), _ptr(d[3], PD),
                         _ptr(d[4], PD), float(b3), _ptr(samples, P64), samples.size,
                         _ptr(att, PD), _ptr(sc, PD) if sc is not None else None,
                         _ptr(wt, PD) if wt is not None else None)
        if want_scores:
            return att, sc, wt
        return att


    def towers(self, pooled, att, tw, want_scale=False):
        """Deep tower + final MLP.  pooled: [ns][>=256] (the first 256 columns
        are the deep input), att: [ns][48]; tw has wd1, bd1, wd2, bd2, wd3, bd3,
        wf, bf, wo, bo (values as the GPU receives them).  Returns deep_out
        [ns][128], logit [ns] and prob [ns], fp64; with want_scale also
        |bo| + sum_i |wo_i f_i| per sample (the size of the logit's terms)."""
        x = np.ascontiguousarray(pooled, dtype=np.float64)
        a = np.ascontiguousarray(att, dtype=np.float64).reshape(x.shape[0], 48)
        assert x.ndim == 2 and x.shape[1] >= 256
        ns = x.shape[0]
        d = [np.ascontiguousarray(getattr(tw, k), dtype=np.float64)
             for k in ("wd1", "bd1", "wd2", "bd2", "wd3", "bd3", "wf", "bf", "wo")]
        assert d[0].shape == (512, 256) and d[2].shape == (256, 512)
        assert d[4].shape == (128, 256) and d[6].shape == (64, 176) and d[8].shape == (64,)
        deep = np.empty((ns, 128), dtype=np.float64)
        logit = np.empty(ns, dtype=np.float64)
        prob = np.empty(ns, dtype=np.float64)
        scale = np.empty(ns, dtype=np.float64)
        self.lib.orc_towers(ns, _ptr(x, PD), x.shape[1], _ptr(a, PD),
                            *[_ptr(v, PD) for v in d], float(tw.bo),
                            _ptr(deep, PD), _ptr(logit, PD), _ptr(prob, PD), _ptr(scale, PD))
        if want_scale:
            return deep, logit, prob, scale
        return deep, logit, prob


_DEFAULT: Optional[Oracle] = None


def get() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


# ---------------------------------------------------------------------------
# Whole-forward convenience used by tests and the CPU-baseline leg.
def forward(model, batch, samples=None, orc: Optional[Oracle] = None, want_scores=False,
            towers=False):
    """Oracle forward for one generator batch: returns dict with offsets,
    pooled [ns, 256], att [ns, 48] (+ scores/weights) for `samples`; with
    towers=True also deep [ns, 128], logit [ns] and prob [ns]."""
    import synth
    orc = orc or get()
    B = batch.B
    samples = np.arange(B, dtype=np.int64) if samples is None else np.asarray(samples, np.int64)
    offsets = orc.lengths_to_offsets(batch.lengths)
    wrapped = orc.tables(model.tables)
    pooled = orc.embbag(model.tables, B, batch.values, batch.lengths, offsets, samples,
                        wrapped=wrapped)
    q = np.concatenate([pooled[:, c:c + 16] for c in synth.QUERY_COL], axis=1)
    seq_off = orc.lengths_to_offsets(batch.seq_lengths)[:-1]
    seq_tabs = [model.tables[k] for k in synth.SEQ_KEYS]
    seq_wrapped = orc.tables(seq_tabs)
    r = orc.din(seq_tabs, batch.seq_values, batch.seq_stride, seq_off, batch.seq_lengths,
                model.cfg.max_len, q, model.w1, model.b1, model.w2, model.b2, model.w3,
                model.b3, samples=samples, wrapped=seq_wrapped, want_scores=want_scores)
    out = dict(offsets=offsets, pooled=pooled, query=q)
    if want_scores:
        out["att"], out["scores"], out["weights"] = r
    else:
        out["att"] = r
    if towers:
        out["deep"], out["logit"], out["prob"], out["logit_scale"] = orc.towers(
            pooled, out["att"], model.towers, want_scale=True)
    return out
