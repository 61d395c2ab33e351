"""The C ABI without a GPU: librec.so loads, exports every function that
include/rec.h declares, agrees with the binding's constants, rejects bad
arguments with the documented status before touching a device, and its
host twins of the device index arithmetic (floor modulo by an invariant
divisor, the hash home slot and digest) agree with independent definitions.

Device pointers here are fake aligned addresses: every call below fails (or
is a documented no-op) in host validation, before the first HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth
from sparse_embedding_din_amd import build as BUILD
from sparse_embedding_din_amd import rec as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rec.h")
FAKE = 0x10000          # a 16-byte aligned, never dereferenced address
FAKE_ODD = 0x10004      # 4-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(R.LIB_PATH):
        BUILD.build()
    return R.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(rec_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in rec.h but not exported"
    assert sorted(R.EXPORTS) == names


def test_header_constants_match_binding(lib):
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(REC_\w+)\s+\(?(-?\w+)", text))
    for name in ("REC_DIM", "REC_MAX_TABLES", "REC_MAX_SEQ_LEN", "REC_MAX_B", "REC_DIN_PACKED_BYTES",
                 "REC_TOWER_PACKED_BYTES", "REC_NOALLOC_SCRATCH_BYTES"):
        assert int(defs[name], 0) == getattr(R, name), name
    enums = dict((k, int(v)) for k, v in re.findall(r"\b(REC_[A-Z0-9_]+)\s*=\s*(-?\d+)", text))
    for name in ("REC_OK", "REC_EINVAL", "REC_EUNSUPPORTED", "REC_EHIP", "REC_EWORKSPACE",
                 "REC_DIRECT", "REC_HASH", "REC_F32", "REC_BF16", "REC_BF16_PACKED"):
        assert enums[name] == getattr(R, name), name
    assert lib.rec_version() >= 100


def _status(fn, *args):
    s = fn(*args)
    return s, R.rec_last_error()


def _table(kind=R.REC_DIRECT, rows=100, dim=16, values=FAKE, keys=None, digests=None):
    return R.table(kind, rows, values, keys, digests, None, dim=dim)


def test_scan_errors(lib):
    s, msg = _status(lib.rec_lengths_to_offsets, FAKE, -1, FAKE, None)
    assert s == R.REC_EINVAL and "n < 0" in msg
    s, msg = _status(lib.rec_lengths_to_offsets, FAKE, 10, None, None)
    assert s == R.REC_EINVAL and "offsets" in msg
    s, msg = _status(lib.rec_lengths_to_offsets, None, 10, FAKE, None)
    assert s == R.REC_EINVAL and "lengths" in msg
    s, msg = _status(lib.rec_lengths_to_offsets, FAKE, 10, FAKE + 4, None)
    assert s == R.REC_EINVAL and "aligned" in msg


def test_embbag_errors(lib):
    tabs = R._tables([_table() for _ in range(16)])
    ok = dict(tables=tabs, T=16, B=4, values=FAKE, lengths=FAKE, offsets=FAKE, out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return _status(lib.rec_embbag_fwd, a["tables"], a["T"], a["B"], a["values"], a["lengths"],
                       a["offsets"], a["out"], None, None)
    assert call(tables=None)[0] == R.REC_EINVAL
    assert call(T=0)[0] == R.REC_EINVAL
    assert call(T=R.REC_MAX_TABLES + 1)[0] == R.REC_EUNSUPPORTED
    assert call(B=-1)[0] == R.REC_EINVAL
    assert call(values=None)[0] == R.REC_EINVAL
    assert call(out=FAKE_ODD)[0] == R.REC_EINVAL
    bad = R._tables([_table() for _ in range(15)] + [_table(dim=8)])
    s, msg = call(tables=bad)
    assert s == R.REC_EINVAL and "dim" in msg
    bad = R._tables([_table(rows=0)] + [_table() for _ in range(15)])
    assert call(tables=bad)[0] == R.REC_EINVAL
    bad = R._tables([_table(kind=7)] + [_table() for _ in range(15)])
    assert call(tables=bad)[0] == R.REC_EINVAL
    bad = R._tables([_table(kind=R.REC_HASH)] + [_table() for _ in range(15)])
    s, msg = call(tables=bad)
    assert s == R.REC_EINVAL and "keys" in msg
    bad = R._tables([_table(values=FAKE_ODD)] + [_table() for _ in range(15)])
    assert call(tables=bad)[0] == R.REC_EINVAL
    # B == 0 is a documented no-op (no device work)
    s, msg = call(B=0)
    assert s == R.REC_OK and msg == ""


def test_kjt_errors(lib):
    assert R.rec_kjt_sums_bytes(16, 8192) >= 8 * 16 * 8 * 33
    assert R.rec_kjt_sums_bytes(0, 10) == 0 and R.rec_kjt_sums_bytes(4, -1) == 0
    sb = R.rec_kjt_sums_bytes(16, 100)
    assert _status(lib.rec_kjt_sums, FAKE, 0, 100, FAKE, sb, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_kjt_sums, FAKE, 33, 100, FAKE, sb, None)[0] == R.REC_EUNSUPPORTED
    assert _status(lib.rec_kjt_sums, FAKE, 16, -1, FAKE, sb, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_kjt_sums, None, 16, 100, FAKE, sb, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_kjt_sums, FAKE, 16, 100, None, sb, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_kjt_sums, FAKE, 16, 100, FAKE + 4, sb, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_kjt_sums, FAKE, 16, 100, FAKE, sb - 8, None)[0] == R.REC_EWORKSPACE
    assert _status(lib.rec_kjt_sums, FAKE, 16, 0, FAKE, 0, None)[0] == R.REC_OK
    tabs = R._tables([_table() for _ in range(16)])

    def call(**kw):
        a = dict(tables=tabs, T=16, B=100, values=FAKE, lengths=FAKE, sums=FAKE, sb=sb, out=FAKE)
        a.update(kw)
        return _status(lib.rec_embbag_fwd_kjt, a["tables"], a["T"], a["B"], a["values"],
                       a["lengths"], a["sums"], a["sb"], None, a["out"], None, None)
    assert call(tables=None)[0] == R.REC_EINVAL
    assert call(T=0)[0] == R.REC_EINVAL
    assert call(T=33)[0] == R.REC_EUNSUPPORTED
    assert call(B=-3)[0] == R.REC_EINVAL
    assert call(sums=None)[0] == R.REC_EINVAL
    assert call(sums=FAKE + 4)[0] == R.REC_EINVAL
    assert call(sb=sb - 8)[0] == R.REC_EWORKSPACE
    assert call(out=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(B=0, sb=0)[0] == R.REC_OK


def test_hash_lookup_errors(lib):
    h = _table(kind=R.REC_HASH, keys=FAKE, digests=FAKE)
    d = _table()
    assert _status(lib.rec_hash_lookup, None, FAKE, 4, FAKE, None, None)[0] == R.REC_EINVAL
    s, msg = _status(lib.rec_hash_lookup, C.byref(d), FAKE, 4, FAKE, None, None)
    assert s == R.REC_EINVAL and "REC_HASH" in msg
    assert _status(lib.rec_hash_lookup, C.byref(h), FAKE, 4, None, None, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_hash_lookup, C.byref(h), None, 4, FAKE, None, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_hash_lookup, C.byref(h), FAKE, -1, FAKE, None, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_hash_lookup, C.byref(h), FAKE, 4, None, FAKE_ODD, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_hash_lookup, C.byref(h), FAKE, 0, FAKE, None, None)[0] == R.REC_OK


def test_hash_insert_errors(lib):
    """Every bad argument is refused before any device call; n == 0 is a no-op."""
    def tab(**kw):
        t = _table(kind=R.REC_HASH, keys=FAKE, digests=FAKE)
        for k, v in kw.items():
            setattr(t, k, v)
        return t
    h, hs = tab(), tab(scores=FAKE)
    ins = lib.rec_hash_insert
    assert _status(ins, None, FAKE, FAKE, 4, 0, 0, None, None, 0, None)[0] == R.REC_EINVAL
    s, msg = _status(ins, C.byref(_table()), FAKE, FAKE, 4, 0, 0, None, None, 0, None)
    assert s == R.REC_EINVAL and "REC_HASH" in msg
    assert _status(ins, C.byref(h), FAKE, FAKE, -1, 0, 0, None, None, 0, None)[0] == R.REC_EINVAL
    s, msg = _status(ins, C.byref(hs), FAKE, FAKE, 4, 3, 0, None, None, 0, None)
    assert s == R.REC_EINVAL and "score_mode" in msg
    for mode in (R.REC_SCORE_STEP, R.REC_SCORE_LFU):
        s, msg = _status(ins, C.byref(h), FAKE, FAKE, 4, mode, 0, None, None, 0, None)
        assert s == R.REC_EINVAL and "scores" in msg
    assert _status(ins, C.byref(tab(scores=FAKE_ODD)), FAKE, FAKE, 4, 1, 0, None, None, 0, None)[0] == \
        R.REC_EINVAL
    assert _status(ins, C.byref(h), None, FAKE, 4, 0, 0, None, None, 0, None)[0] == R.REC_EINVAL
    assert _status(ins, C.byref(h), FAKE, None, 4, 0, 0, None, None, 0, None)[0] == R.REC_EINVAL
    assert _status(ins, C.byref(h), FAKE, FAKE_ODD, 4, 0, 0, None, None, 0, None)[0] == R.REC_EINVAL
    assert _status(ins, C.byref(tab(digests=FAKE_ODD)), FAKE, FAKE, 4, 0, 0, None, None, 0, None)[0] == \
        R.REC_EINVAL
    assert _status(ins, C.byref(tab(rows=0)), FAKE, FAKE, 4, 0, 0, None, None, 0, None)[0] == R.REC_EINVAL
    assert _status(ins, C.byref(tab(dim=8)), FAKE, FAKE, 4, 0, 0, None, None, 0, None)[0] == R.REC_EINVAL
    assert _status(ins, C.byref(hs), None, None, 0, 2, 5, None, None, 0, None)[0] == R.REC_OK
    need = R.rec_hash_insert_workspace_bytes(4, 100)
    assert need >= 4 * 4 + 4 * 100 and R.rec_hash_insert_workspace_bytes(-1, 100) == 0
    assert R.rec_hash_insert_workspace_bytes((1 << 30) + 1, 100) == 0
    assert R.rec_hash_insert_workspace_bytes(4, 0) == 0
    s, msg = _status(ins, C.byref(h), FAKE, FAKE, 4, 0, 0, None, None, 0, None)
    assert s == R.REC_EWORKSPACE and "workspace" in msg
    assert _status(ins, C.byref(h), FAKE, FAKE, 4, 0, 0, None, FAKE, need - 1, None)[0] == R.REC_EWORKSPACE
    assert _status(ins, C.byref(h), FAKE, FAKE, 4, 0, 0, None, FAKE + 16, need, None)[0] == R.REC_EINVAL
    assert _status(ins, C.byref(h), FAKE, FAKE, (1 << 30) + 1, 0, 0, None, FAKE, need, None)[0] == \
        R.REC_EUNSUPPORTED
    with pytest.raises(R.RecError):
        R.rec_hash_insert(_table(), FAKE, FAKE, 4)


def test_hash_clear_errors(lib):
    clr = lib.rec_hash_clear
    assert _status(clr, None, None)[0] == R.REC_EINVAL
    s, msg = _status(clr, C.byref(_table()), None)
    assert s == R.REC_EINVAL and "REC_HASH" in msg
    t = _table(kind=R.REC_HASH, keys=FAKE, digests=FAKE)
    t.scores = FAKE_ODD
    assert _status(clr, C.byref(t), None)[0] == R.REC_EINVAL
    assert _status(clr, C.byref(_table(kind=R.REC_HASH, keys=None, digests=FAKE)), None)[0] == \
        R.REC_EINVAL


def test_dlrm_interact_errors(lib):
    f = lib.rec_dlrm_interact
    assert _status(f, FAKE, -1, 5, 16, FAKE, None)[0] == R.REC_EINVAL
    assert _status(f, FAKE, 4, 0, 16, FAKE, None)[0] == R.REC_EINVAL
    for d in (0, 8, 24, 100):
        s, msg = _status(f, FAKE, 4, 5, d, FAKE, None)
        assert s == R.REC_EINVAL and "multiple of 16" in msg
    assert _status(f, FAKE, 4, 257, 16, FAKE, None)[0] == R.REC_EUNSUPPORTED
    assert _status(f, FAKE, 4, 5, 528, FAKE, None)[0] == R.REC_EUNSUPPORTED
    s, msg = _status(f, FAKE, 4, 217, 176, FAKE, None)              # 224 x 180 floats > 144 KiB
    assert s == R.REC_EUNSUPPORTED and "LDS" in msg
    assert _status(f, None, 4, 5, 16, FAKE, None)[0] == R.REC_EINVAL
    assert _status(f, FAKE, 4, 5, 16, None, None)[0] == R.REC_EINVAL
    assert _status(f, FAKE_ODD, 4, 5, 16, FAKE, None)[0] == R.REC_EINVAL
    assert _status(f, None, 0, 217, 160, None, None)[0] == R.REC_OK   # the largest width at F = 217
    with pytest.raises(R.RecError):
        R.rec_dlrm_interact(FAKE, 4, 5, 8, FAKE)


def test_din_pack_errors(lib):
    m = R.din_mlp(R.REC_F32, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0)
    assert _status(lib.rec_din_pack_mlp, C.byref(m), FAKE, R.REC_DIN_PACKED_BYTES, None)[0] == R.REC_EINVAL
    m = R.din_mlp(R.REC_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0)
    assert _status(lib.rec_din_pack_mlp, None, FAKE, R.REC_DIN_PACKED_BYTES, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_din_pack_mlp, C.byref(m), None, R.REC_DIN_PACKED_BYTES, None)[0] == R.REC_EINVAL
    assert _status(lib.rec_din_pack_mlp, C.byref(m), FAKE_ODD, R.REC_DIN_PACKED_BYTES, None)[0] == R.REC_EINVAL
    assert (_status(lib.rec_din_pack_mlp, C.byref(m), FAKE, R.REC_DIN_PACKED_BYTES - 16, None)[0]
            == R.REC_EWORKSPACE)


def test_din_plan_errors(lib):
    seq = R._tables([_table() for _ in range(3)])
    B, ml = 64, 100
    pb = R.rec_din_plan_bytes(B, ml)
    assert pb > 20 * B * ml
    assert R.rec_din_plan_bytes(-1, 100) == 0 and R.rec_din_plan_bytes(4, 0) == 0
    assert R.rec_din_plan_bytes(4, R.REC_MAX_SEQ_LEN + 1) == 0
    assert R.rec_din_plan_bytes(R.REC_MAX_B + 1, 1) == 0

    def call(**kw):
        a = dict(tables=seq, values=FAKE, stride=B * 4, offsets=None, lengths=FAKE, B=B, ml=ml,
                 rp=0, plan=FAKE, pb=pb)
        a.update(kw)
        return _status(lib.rec_din_plan, a["tables"], a["values"], a["stride"], a["offsets"],
                       a["lengths"], a["B"], a["ml"], a["rp"], None, None, a["plan"], a["pb"], None)
    assert call(B=-1)[0] == R.REC_EINVAL
    assert call(B=R.REC_MAX_B + 1)[0] == R.REC_EUNSUPPORTED
    assert call(ml=0)[0] == R.REC_EINVAL
    assert call(ml=R.REC_MAX_SEQ_LEN + 1)[0] == R.REC_EINVAL
    for rp in (8, 24, -16, (1 << 20) + 16):
        s, msg = call(rp=rp)
        assert s == R.REC_EINVAL and "range_positions" in msg
    assert call(tables=None)[0] == R.REC_EINVAL
    assert call(lengths=None)[0] == R.REC_EINVAL
    assert call(values=None)[0] == R.REC_EINVAL
    assert call(stride=-1)[0] == R.REC_EINVAL
    assert call(plan=None)[0] == R.REC_EWORKSPACE
    assert call(plan=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(pb=pb - 1)[0] == R.REC_EWORKSPACE
    bad = R._tables([_table(), _table(dim=4), _table()])
    assert call(tables=bad)[0] == R.REC_EINVAL
    assert call(B=0, pb=R.rec_din_plan_bytes(0, ml))[0] == R.REC_OK


def test_din_attn_errors(lib):
    seq = R._tables([_table() for _ in range(3)])
    B, ml = 64, 100
    pb = R.rec_din_plan_bytes(B, ml)
    good = R.din_mlp(R.REC_BF16_PACKED, FAKE, FAKE, None, FAKE, FAKE, 0.0)

    def call(**kw):
        a = dict(tables=seq, plan=FAKE, pb=pb, B=B, ml=ml, q=FAKE, qld=256, qcol=(16, 80, 48),
                 mlp=good, out=FAKE, scores=None, weights=None)
        a.update(kw)
        qc = None if a["qcol"] is None else (C.c_int32 * 3)(*a["qcol"])
        mlp = None if a["mlp"] is None else C.byref(a["mlp"])
        return _status(lib.rec_din_attn_fwd_plan, a["tables"], a["plan"], a["pb"], a["B"], a["ml"],
                       a["q"], a["qld"], qc, mlp, a["out"], a["scores"], a["weights"], None)
    assert call(B=-1)[0] == R.REC_EINVAL
    assert call(B=R.REC_MAX_B + 1)[0] == R.REC_EUNSUPPORTED
    assert call(ml=0)[0] == R.REC_EINVAL
    assert call(q=None)[0] == R.REC_EINVAL
    assert call(qcol=None)[0] == R.REC_EINVAL
    assert call(q=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(qld=250)[0] == R.REC_EINVAL
    assert call(qcol=(16, 82, 48))[0] == R.REC_EINVAL
    assert call(qcol=(16, 80, 248))[0] == R.REC_EINVAL
    assert call(mlp=None)[0] == R.REC_EINVAL
    assert call(mlp=R.din_mlp(9, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0))[0] == R.REC_EINVAL
    assert call(mlp=R.din_mlp(R.REC_BF16, FAKE, FAKE, None, FAKE, FAKE, 0.0))[0] == R.REC_EINVAL
    assert call(mlp=R.din_mlp(R.REC_F32, FAKE_ODD, FAKE, FAKE, FAKE, FAKE, 0.0))[0] == R.REC_EINVAL
    assert call(out=None)[0] == R.REC_EINVAL
    assert call(out=FAKE_ODD)[0] == R.REC_EINVAL
    s, msg = call(weights=FAKE)
    assert s == R.REC_EINVAL and "scores_out" in msg
    assert call(plan=None)[0] == R.REC_EWORKSPACE
    assert call(pb=pb - 1)[0] == R.REC_EWORKSPACE
    assert call(B=0, pb=R.rec_din_plan_bytes(0, ml))[0] == R.REC_OK


def test_din_attn_one_call_errors(lib):
    """rec_din_attn_fwd (plan built inside the caller's workspace): every
    argument error is caught on the host before any launch."""
    seq = R._tables([_table() for _ in range(3)])
    B, ml = 64, 100
    wb = R.rec_din_attn_workspace_bytes(B, ml)
    assert wb == R.rec_din_plan_bytes(B, ml) and wb > 20 * B * ml
    assert R.rec_din_attn_workspace_bytes(4, R.REC_MAX_SEQ_LEN) > 20 * 4 * R.REC_MAX_SEQ_LEN
    assert R.rec_din_attn_workspace_bytes(4, R.REC_MAX_SEQ_LEN + 1) == 0
    assert R.rec_din_attn_workspace_bytes(-1, ml) == 0 and R.rec_din_attn_workspace_bytes(4, 0) == 0
    good = R.din_mlp(R.REC_BF16_PACKED, FAKE, FAKE, None, FAKE, FAKE, 0.0)

    def call(**kw):
        a = dict(tables=seq, values=FAKE, stride=B * 4, offsets=None, lengths=FAKE, ml=ml, B=B,
                 q=FAKE, qld=256, qcol=(16, 80, 48), mlp=good, out=FAKE, scores=None,
                 weights=None, rows=None, ws=FAKE, wb=wb)
        a.update(kw)
        qc = None if a["qcol"] is None else (C.c_int32 * 3)(*a["qcol"])
        mlp = None if a["mlp"] is None else C.byref(a["mlp"])
        return _status(lib.rec_din_attn_fwd, a["tables"], a["values"], a["stride"], a["offsets"],
                       a["lengths"], a["ml"], a["B"], a["q"], a["qld"], qc, mlp, a["out"],
                       a["scores"], a["weights"], a["rows"], a["ws"], a["wb"], None)
    assert call(B=-1)[0] == R.REC_EINVAL
    assert call(B=R.REC_MAX_B + 1)[0] == R.REC_EUNSUPPORTED
    for bad_ml in (0, R.REC_MAX_SEQ_LEN + 1):
        s, msg = call(ml=bad_ml, wb=R.rec_din_attn_workspace_bytes(B, R.REC_MAX_SEQ_LEN))
        assert s == R.REC_EINVAL and "max_len" in msg
    assert call(tables=None)[0] == R.REC_EINVAL
    assert call(values=None)[0] == R.REC_EINVAL
    assert call(lengths=None)[0] == R.REC_EINVAL
    assert call(stride=-1)[0] == R.REC_EINVAL
    assert call(q=None)[0] == R.REC_EINVAL
    assert call(qcol=None)[0] == R.REC_EINVAL
    assert call(q=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(qcol=(16, 82, 48))[0] == R.REC_EINVAL
    assert call(mlp=None)[0] == R.REC_EINVAL
    assert call(out=None)[0] == R.REC_EINVAL
    s, msg = call(weights=FAKE)
    assert s == R.REC_EINVAL and "scores_out" in msg
    s, msg = call(ws=None)
    assert s == R.REC_EWORKSPACE and "workspace" in msg
    s, msg = call(wb=wb - 1)
    assert s == R.REC_EWORKSPACE and "rec_din_attn_workspace_bytes" in msg
    assert call(ws=FAKE_ODD)[0] == R.REC_EINVAL
    bad = R._tables([_table(), _table(kind=7), _table()])
    assert call(tables=bad)[0] == R.REC_EINVAL
    assert call(B=0, wb=R.rec_din_attn_workspace_bytes(0, ml))[0] == R.REC_OK


def test_whole_forward_errors(lib):
    tabs = R._tables([_table() for _ in range(16)])
    seq = R._tables([_table() for _ in range(3)])
    B, ml = 64, 100
    wb = R.rec_sparse_din_fwd_workspace_bytes(16, B, ml)
    assert wb >= R.rec_kjt_sums_bytes(16, B) + R.rec_din_plan_bytes(B, ml)
    assert R.rec_sparse_din_fwd_workspace_bytes(0, B, ml) == 0
    assert R.rec_sparse_din_fwd_workspace_bytes(16, B, 0) == 0
    mlp = R.din_mlp(R.REC_BF16_PACKED, FAKE, FAKE, None, FAKE, FAKE, 0.0)

    def args(**kw):
        a = dict(T=16, B=B, max_len=ml, tables=tabs, values=FAKE, lengths=FAKE, seq_tables=seq,
                 seq_values=FAKE, seq_stride=B * 4, seq_offsets=None, seq_lengths=FAKE,
                 query_col=(16, 80, 48), range_positions=0, mlp=mlp, pooled=FAKE, att=FAKE,
                 workspace=FAKE, workspace_bytes=wb)
        a.update(kw)
        return R.fwd_args(**a)
    assert lib.rec_sparse_din_fwd(None, None) == R.REC_EINVAL
    assert lib.rec_sparse_din_fwd(C.byref(args(workspace=None)), None) == R.REC_EINVAL
    assert lib.rec_sparse_din_fwd(C.byref(args(workspace=FAKE_ODD)), None) == R.REC_EINVAL
    assert lib.rec_sparse_din_fwd(C.byref(args(workspace_bytes=wb - 16)), None) == R.REC_EWORKSPACE
    assert lib.rec_sparse_din_fwd(C.byref(args(T=0)), None) == R.REC_EINVAL
    assert lib.rec_sparse_din_fwd(C.byref(args(pooled=FAKE_ODD)), None) == R.REC_EINVAL
    assert lib.rec_sparse_din_fwd(C.byref(args(range_positions=8)), None) == R.REC_EINVAL
    assert lib.rec_sparse_din_fwd(C.byref(args(query_col=(16, 80, 250))), None) == R.REC_EINVAL
    s, msg = _status(lib.rec_sparse_din_fwd, C.byref(args(weights_out=FAKE)), None)
    assert s == R.REC_EINVAL and "rec_sparse_din_fwd" in msg and "scores_out" in msg
    bad = R._tables([_table(), _table(dim=3), _table()])
    assert lib.rec_sparse_din_fwd(C.byref(args(seq_tables=bad)), None) == R.REC_EINVAL
    zb = R.rec_sparse_din_fwd_workspace_bytes(16, 0, ml)
    assert lib.rec_sparse_din_fwd(C.byref(args(B=0, workspace_bytes=zb)), None) == R.REC_OK


def test_towers_errors(lib):
    def mlp(**kw):
        a = dict(dtype=R.REC_BF16, wd1=FAKE, bd1=FAKE, wd2=FAKE, bd2=FAKE, wd3=FAKE, bd3=FAKE,
                 wf=FAKE, bf=FAKE, wo=FAKE, bo=0.0)
        a.update(kw)
        return R.tower_mlp(**a)

    def call(m=None, B=64, pooled=FAKE, ld=256, att=FAKE, deep=None, logit=FAKE, prob=None):
        return _status(lib.rec_towers_fwd, C.byref(m if m is not None else mlp()), B, pooled, ld,
                       att, deep, logit, prob, None)
    assert lib.rec_towers_fwd(None, 4, FAKE, 256, FAKE, None, FAKE, None, None) == R.REC_EINVAL
    assert call(mlp(dtype=7))[0] == R.REC_EINVAL
    # a packed image replaces wd2, wd3 and wf: they may be NULL then
    pk = mlp(dtype=R.REC_BF16_PACKED, wd2=None, wd3=None, wf=None)
    assert call(pk, B=0)[0] == R.REC_OK
    assert call(mlp(dtype=R.REC_BF16_PACKED, wd1=None), B=0)[0] == R.REC_EINVAL
    assert call(mlp(dtype=R.REC_BF16_PACKED, wd1=FAKE_ODD), B=0)[0] == R.REC_EINVAL
    for k in ("wd1", "bd1", "wd2", "bd2", "wd3", "bd3", "wf", "bf", "wo"):
        assert call(mlp(**{k: None}))[0] == R.REC_EINVAL, k
        s, msg = call(mlp(**{k: FAKE_ODD}))
        assert s == R.REC_EINVAL and "aligned" in msg, k
    assert call(B=-1)[0] == R.REC_EINVAL
    assert call(pooled=None)[0] == R.REC_EINVAL
    assert call(att=None)[0] == R.REC_EINVAL
    assert call(logit=None)[0] == R.REC_EINVAL
    assert call(ld=255)[0] == R.REC_EINVAL
    assert call(ld=258)[0] == R.REC_EINVAL
    assert call(pooled=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(att=FAKE_ODD)[0] == R.REC_EINVAL
    s, msg = call(deep=FAKE_ODD)
    assert s == R.REC_EINVAL and "rec_towers_fwd" in msg
    assert call(B=0)[0] == R.REC_OK
    assert call(m=mlp(dtype=R.REC_F32), B=0)[0] == R.REC_OK


def test_tower_pack_errors(lib):
    def m(**kw):
        a = dict(dtype=R.REC_BF16, wd1=FAKE, bd1=FAKE, wd2=FAKE, bd2=FAKE, wd3=FAKE, bd3=FAKE,
                 wf=FAKE, bf=FAKE, wo=FAKE, bo=0.0)
        a.update(kw)
        return C.byref(R.tower_mlp(**a))
    n = R.REC_TOWER_PACKED_BYTES
    assert lib.rec_tower_pack_mlp(None, FAKE, n, None) == R.REC_EINVAL
    assert lib.rec_tower_pack_mlp(m(dtype=R.REC_F32), FAKE, n, None) == R.REC_EINVAL
    assert lib.rec_tower_pack_mlp(m(dtype=R.REC_BF16_PACKED), FAKE, n, None) == R.REC_EINVAL
    for k in ("wd1", "wd2", "wd3", "wf"):
        assert lib.rec_tower_pack_mlp(m(**{k: None}), FAKE, n, None) == R.REC_EINVAL, k
        assert lib.rec_tower_pack_mlp(m(**{k: FAKE_ODD}), FAKE, n, None) == R.REC_EINVAL, k
    assert lib.rec_tower_pack_mlp(m(), None, n, None) == R.REC_EINVAL
    assert lib.rec_tower_pack_mlp(m(), FAKE_ODD, n, None) == R.REC_EINVAL
    s, msg = _status(lib.rec_tower_pack_mlp, m(), FAKE, n - 16, None)
    assert s == R.REC_EWORKSPACE and "REC_TOWER_PACKED_BYTES" in msg


def test_binding_raises_with_message(lib):
    with pytest.raises(R.RecError) as ei:
        R.rec_hash_lookup(_table(), FAKE, 4, FAKE)
    assert ei.value.status == R.REC_EINVAL and "REC_HASH" in str(ei.value)


# -- host twins of the device index arithmetic --------------------------------
I64 = np.iinfo(np.int64)
EDGE_X = [0, 1, -1, 2, -2, 99, 100, 101, -100, -101, I64.max, I64.min, I64.min + 1, I64.max - 1,
          2**32, -2**32, 2**62 + 12345, -(2**62) - 12345]
EDGE_N = [1, 2, 3, 5, 7, 98, 101, 12961, 255877, 846812, 1141730, 2**31 - 1, 2**32 + 15,
          2**62 + 1, I64.max]


def test_host_floor_mod_edges(lib):
    """Invariant-divisor floor modulo against Python's % (floor semantics)."""
    for n in EDGE_N:
        for x in EDGE_X:
            assert R.rec_host_floor_mod(x, n) == x % n, (x, n)


def test_host_floor_mod_random(lib):
    rng = np.random.default_rng(7)
    ns = np.concatenate([rng.integers(1, 2**20, 40), rng.integers(1, I64.max, 40, dtype=np.int64)])
    xs = rng.integers(I64.min, I64.max, 60, dtype=np.int64, endpoint=True)
    for n in ns:
        for x in xs:
            assert R.rec_host_floor_mod(int(x), int(n)) == int(x) % int(n)


def test_host_hash_home_matches_generator(lib):
    """Home slot and digest against the generator's table layout (the format
    both sides of a hash table share)."""
    rng = np.random.default_rng(11)
    keys = np.concatenate([rng.integers(I64.min, I64.max, 500, dtype=np.int64),
                           np.array([0, 1, -2, I64.max, I64.min], np.int64)])
    for cap in (1, 7, 300000, 2**31 - 1):
        h = synth.splitmix64_mix(keys)
        home = synth.home_slot(h, cap)
        dig = synth.digest_of(h)
        for k, h, d in zip(keys, home, dig):
            got_h, got_d = R.rec_host_hash_home(int(k), cap)
            assert got_h == int(h) and got_d == int(d)
            assert 0 <= got_h < cap and got_d != 0


def _aligned_u8(n):
    buf = np.zeros(n + 64, np.uint8)
    off = (-buf.ctypes.data) % 16
    return buf[off: off + n]


@pytest.mark.parametrize("cap,nkeys", [(1, 0), (2, 1), (5, 4), (16, 15), (17, 16), (31, 20),
                                       (32, 31), (33, 32), (37, 30), (64, 60), (100, 70),
                                       (1000, 700), (4099, 4000)])
def test_host_hash_probe_windowed(lib, cap, nkeys):
    """The device's windowed probe (32 digests per read, byte reads with wrap
    near the table's end), run on the host, against set membership on tables
    of every size around the window, including full and nearly full ones:
    every stored key is found in its slot, every other key misses.  (The
    table layout needs at least one empty slot.)"""
    rng = np.random.default_rng(cap * 1000 + nkeys)
    I64 = np.iinfo(np.int64)
    stored = np.unique(rng.integers(I64.min, I64.max, size=nkeys * 2 + 1, dtype=np.int64))
    stored = stored[stored != synth.EMPTY_KEY][:nkeys]
    vals = np.zeros((max(stored.size, 1), 16), np.float32)
    tab = synth.build_hash_table(stored, vals[: stored.size], cap)
    keys = np.ascontiguousarray(tab["keys"], np.int64)
    dig = _aligned_u8(cap)
    dig[:] = tab["digests"]
    for k in stored:
        slot = R.rec_host_hash_probe(keys, dig, cap, int(k))
        assert slot >= 0 and keys[slot] == k
    misses = rng.integers(I64.min, I64.max, size=300, dtype=np.int64)
    for k in misses:
        if k in set(stored.tolist()):
            continue
        assert R.rec_host_hash_probe(keys, dig, cap, int(k)) == -1
    if cap > 1:
        assert R.rec_host_hash_probe(keys, dig[1:], cap - 1, 0) == -2     # misaligned digests


def test_embbag_adagrad_errors(lib):
    f = lib.rec_embbag_adagrad

    def tabs(n=2, rows=10, w=FAKE, g=FAKE):
        arr = (R.rec_adagrad_table * n)()
        for i in range(n):
            arr[i] = R.rec_adagrad_table(w, g, rows)
        return arr

    st = (C.c_int32 * 3)(0, 1, 1)

    def call(t=None, T=2, B=4, nnz=8, P=3, seq=st, gp=FAKE, gs=FAKE, ws=FAKE, wsb=1 << 20):
        t = tabs() if t is None else t
        return _status(f, t, T, B, FAKE, FAKE, FAKE, nnz, gp, seq, FAKE, max(P, 1), P, gs,
                       1e-3, 1e-10, ws, wsb, None)

    assert call(t=C.cast(None, C.POINTER(R.rec_adagrad_table)))[0] == R.REC_EINVAL
    assert call(T=0)[0] == R.REC_EINVAL
    assert call(t=tabs(33), T=33)[0] == R.REC_EUNSUPPORTED
    assert call(B=-1)[0] == R.REC_EINVAL
    assert call(nnz=-1)[0] == R.REC_EINVAL
    assert call(P=-1)[0] == R.REC_EINVAL
    assert call(t=tabs(rows=0))[0] == R.REC_EINVAL
    assert call(t=tabs(w=None))[0] == R.REC_EINVAL
    assert call(t=tabs(g=FAKE_ODD))[0] == R.REC_EINVAL
    bad_kind = tabs()
    bad_kind[1].kind = 7
    assert call(t=bad_kind)[0] == R.REC_EINVAL
    no_keys = tabs()
    no_keys[0].kind, no_keys[0].digests = R.REC_HASH, FAKE
    assert call(t=no_keys)[0] == R.REC_EINVAL
    odd_dig = tabs()
    odd_dig[0].kind, odd_dig[0].keys, odd_dig[0].digests = R.REC_HASH, FAKE, FAKE + 4
    assert call(t=odd_dig)[0] == R.REC_EINVAL
    s, msg = call(t=tabs(rows=1 << 31))
    assert s == R.REC_EUNSUPPORTED and "2^32" in msg
    assert call(gp=None)[0] == R.REC_EINVAL
    assert call(gp=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(seq=None)[0] == R.REC_EINVAL
    assert call(gs=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(seq=(C.c_int32 * 3)(0, 2, 1))[0] == R.REC_EINVAL       # table 2 of T = 2
    assert call(seq=(C.c_int32 * 3)(-1, 0, 1))[0] == R.REC_EINVAL
    assert call(nnz=1 << 31)[0] == R.REC_EUNSUPPORTED
    assert call(nnz=0, P=0, seq=None, gp=None, gs=None, ws=None, wsb=0)[0] == R.REC_OK
    wsb = R.rec_embbag_adagrad_workspace_bytes(2, 4, 8, 3)
    assert wsb >= 4 * 4 * 17 and wsb % 256 == 0          # four 4-byte arrays of 17 reads
    assert call(ws=FAKE, wsb=wsb - 1)[0] == R.REC_EWORKSPACE
    assert call(ws=None, wsb=wsb)[0] == R.REC_EWORKSPACE
    assert call(ws=FAKE + 16, wsb=wsb)[0] == R.REC_EINVAL              # not 256-byte aligned
    big = R.rec_embbag_adagrad_workspace_bytes(16, 8192, 253952, 32768)
    assert 24 * (253952 + 3 * 32768) <= big <= 26 * (253952 + 3 * 32768)
    assert R.rec_embbag_adagrad_workspace_bytes(0, 4, 8, 3) == 0
    assert R.rec_embbag_adagrad_workspace_bytes(2, 4, 0, 0) == 0
    with pytest.raises(R.RecError):
        R.rec_embbag_adagrad([R.adagrad_table(FAKE, FAKE, 10)], 1, 4, FAKE, FAKE, FAKE, 8, None,
                             None, None, 0, 0, None, 1e-3, 1e-10, FAKE, 1 << 20)


def test_din_attn_bwd_errors(lib):
    f = lib.rec_din_attn_bwd
    seq = R._tables([_table() for _ in range(3)])
    mlp = R.din_mlp(R.REC_F32, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0)
    qc = (C.c_int32 * 3)(16, 80, 48)
    W = [FAKE] * 6

    def call(B=4, max_len=100, stride=64, seq_=seq, mlp_=mlp, qc_=qc, ld=256, gq=FAKE, gs=FAKE,
             w=W, ws=FAKE, wsb=1 << 30):
        return _status(f, seq_, FAKE, stride, FAKE, FAKE, max_len, B, FAKE, ld, qc_, C.byref(mlp_),
                       FAKE, gq, gs, *w, ws, wsb, None)

    assert call(B=-1)[0] == R.REC_EINVAL
    assert call(max_len=0)[0] == R.REC_EINVAL
    assert call(max_len=R.REC_MAX_SEQ_LEN + 1)[0] == R.REC_EINVAL
    assert call(stride=-1)[0] == R.REC_EINVAL
    assert call(qc_=(C.c_int32 * 3)(16, 250, 48))[0] == R.REC_EINVAL     # 250 + 16 > 256
    assert call(gq=None)[0] == R.REC_EINVAL
    assert call(gs=FAKE_ODD)[0] == R.REC_EINVAL
    s, msg = call(w=[FAKE, FAKE, None, FAKE, FAKE, FAKE])
    assert s == R.REC_EINVAL and "all six" in msg
    packed = R.din_mlp(R.REC_BF16_PACKED, FAKE, FAKE, None, FAKE, FAKE, 0.0)
    assert call(mlp_=packed)[0] == R.REC_EUNSUPPORTED
    need = R.rec_din_attn_bwd_workspace_bytes(64, True)
    small = R.rec_din_attn_bwd_workspace_bytes(64, False)
    assert small > (192 + 64) * 256 * 4 + 64 * 3700 and need > small + 4 * 65921
    assert call(wsb=need - 1)[0] == R.REC_EWORKSPACE
    assert call(w=[None] * 6, wsb=small - 1)[0] == R.REC_EWORKSPACE
    assert call(ws=FAKE + 16, wsb=need)[0] == R.REC_EINVAL
    assert call(B=0, wsb=small, w=[None] * 6)[0] == R.REC_OK


def test_noalloc_limit_checked_before_the_device(lib):
    """rec_sparse_din_fwd_noalloc refuses a batch beyond its static scratch
    with REC_EWORKSPACE before any HIP call (this runs without a GPU)."""
    assert _status(lib.rec_sparse_din_fwd_noalloc, None, None)[0] == R.REC_EINVAL
    a = R.rec_fwd_args()
    a.T, a.max_len, a.B = 16, 100, 1 << 20
    assert R.rec_sparse_din_fwd_workspace_bytes(16, 1 << 20, 100) > R.REC_NOALLOC_SCRATCH_BYTES
    s, msg = _status(lib.rec_sparse_din_fwd_noalloc, C.byref(a), None)
    assert s == R.REC_EWORKSPACE and "REC_NOALLOC_SCRATCH_BYTES" in msg
    assert R.rec_sparse_din_fwd_workspace_bytes(16, 8192, 100) <= R.REC_NOALLOC_SCRATCH_BYTES
    a.B = 8192                    # fits: the argument checks come next (no tables given)
    s, msg = _status(lib.rec_sparse_din_fwd_noalloc, C.byref(a), None)
    assert s == R.REC_EINVAL and "rec_sparse_din_fwd_noalloc" in msg


def test_dlrm_fwd_errors(lib):
    """rec_dlrm_fwd: every bad argument is refused on the host."""
    S, d, nd = 8, 96, 13
    good = R.dlrm_mlp(nd, d, S, *([FAKE] * 9), 0.0)
    tabs = [_table(rows=100, dim=d) for _ in range(S)]
    modes = [R.REC_POOL_SUM] * S

    def call(mlp=good, tables=tabs, md=modes, B=4, dense=FAKE, values=FAKE, lengths=FAKE,
             offsets=FAKE, z=FAKE, inter=None, logit=FAKE, prob=None):
        m = None if mlp is None else C.byref(mlp)
        t = None if tables is None else R._tables(tables)
        mm = None if md is None else (C.c_int32 * len(md))(*md)
        return _status(lib.rec_dlrm_fwd, m, t, mm, B, dense, values, lengths, offsets, z, inter,
                       logit, prob, None)
    assert call(mlp=None)[0] == R.REC_EINVAL
    assert call(tables=None)[0] == R.REC_EINVAL
    assert call(md=None)[0] == R.REC_EINVAL
    assert call(B=-1)[0] == R.REC_EINVAL
    for kw in (dict(S=0), dict(S=256), dict(dim=48), dict(dim=16), dict(dim=288), dict(n_dense=0),
               dict(n_dense=129)):
        m = R.dlrm_mlp(kw.get("n_dense", nd), kw.get("dim", d), kw.get("S", S), *([FAKE] * 9), 0.0)
        s, msg = call(mlp=m, tables=[_table(rows=100, dim=kw.get("dim", d))] * max(kw.get("S", S), 1),
                      md=[0] * max(kw.get("S", S), 1))
        assert s == R.REC_EINVAL, kw
    # wide models ((S+1) * dim above 1024, or more than 31 tables) need inter
    m = R.dlrm_mlp(nd, 128, 8, *([FAKE] * 9), 0.0)               # (S+1) * dim = 1152 > 1024
    assert call(mlp=m, tables=[_table(rows=100, dim=128)] * 8)[0] == R.REC_EINVAL
    m = R.dlrm_mlp(nd, 96, 216, *([FAKE] * 9), 0.0)              # the 217-feature model
    assert call(mlp=m, tables=[_table(rows=100, dim=96)] * 216, md=[0] * 216)[0] == R.REC_EINVAL
    m = R.dlrm_mlp(nd, 224, 216, *([FAKE] * 9), 0.0)             # beyond the interaction's LDS stage
    s, msg = call(mlp=m, tables=[_table(rows=100, dim=224)] * 216, md=[0] * 216, inter=FAKE)
    assert s == R.REC_EUNSUPPORTED, msg
    m = R.dlrm_mlp(nd, d, S, *([FAKE] * 8), None, 0.0)
    assert call(mlp=m)[0] == R.REC_EINVAL
    m = R.dlrm_mlp(nd, d, S, FAKE_ODD, *([FAKE] * 8), 0.0)
    assert call(mlp=m)[0] == R.REC_EINVAL
    bad = list(tabs)
    bad[3] = _table(rows=100, dim=16)
    assert call(tables=bad)[0] == R.REC_EINVAL
    bad[3] = _table(kind=R.REC_HASH, rows=100, dim=d, keys=FAKE, digests=FAKE)
    assert call(tables=bad)[0] == R.REC_EINVAL
    bad[3] = _table(rows=0, dim=d)
    assert call(tables=bad)[0] == R.REC_EINVAL
    assert call(md=[0] * 7 + [2])[0] == R.REC_EINVAL
    for k in ("dense", "values", "lengths", "offsets", "z", "logit"):
        assert call(**{k: None})[0] == R.REC_EINVAL, k
    assert call(z=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(B=0, dense=None, values=None, lengths=None, offsets=None, z=None, logit=None)[0] == R.REC_OK


def test_hash_admit_errors(lib):
    """rec_hash_admit: argument errors are refused on the host."""
    def tab(**kw):
        t = _table(kind=R.REC_HASH, rows=1000, keys=FAKE, digests=FAKE)
        t.scores = FAKE
        for k, v in kw.items():
            setattr(t, k, v)
        return t
    wb = R.rec_hash_admit_workspace_bytes(10, 1000, R.REC_SCORE_LFU)
    assert wb > 0 and R.rec_hash_admit_workspace_bytes(10, 1000, R.REC_SCORE_NONE) < wb
    assert R.rec_hash_admit_workspace_bytes(-1, 1000, 1) == 0
    assert R.rec_hash_admit_workspace_bytes(10, 0, 1) == 0

    def call(t=None, mk=1000, ck=FAKE, cc=FAKE, ccap=64, keys=FAKE, iv=FAKE, n=10, th=3,
             mode=R.REC_SCORE_LFU, ws=FAKE, wsb=wb):
        t = tab() if t is None else t
        return _status(lib.rec_hash_admit, C.byref(t) if t != "null" else None, mk, ck, cc, ccap, keys,
                       iv, n, th, mode, 7, None, None, ws, wsb, None)
    assert call(t="null")[0] == R.REC_EINVAL
    assert call(t=_table())[0] == R.REC_EINVAL                       # direct table
    assert call(t=tab(scores=None))[0] == R.REC_EINVAL                # LFU needs scores
    assert call(t=tab(scores=None), mode=R.REC_SCORE_NONE,
                wsb=R.rec_hash_admit_workspace_bytes(10, 1000, 0), ws=None)[0] == R.REC_EWORKSPACE
    assert call(mode=5)[0] == R.REC_EINVAL
    assert call(mk=-1)[0] == R.REC_EINVAL and call(mk=1001)[0] == R.REC_EINVAL
    assert call(th=0)[0] == R.REC_EINVAL
    assert call(ck=None)[0] == R.REC_EINVAL and call(cc=None)[0] == R.REC_EINVAL
    assert call(ccap=0)[0] == R.REC_EINVAL and call(ck=FAKE + 4)[0] == R.REC_EINVAL
    assert call(n=-1)[0] == R.REC_EINVAL
    assert call(n=(1 << 30) + 1)[0] == R.REC_EUNSUPPORTED
    assert call(keys=None)[0] == R.REC_EINVAL and call(iv=None)[0] == R.REC_EINVAL
    assert call(iv=FAKE_ODD)[0] == R.REC_EINVAL
    assert call(ws=None)[0] == R.REC_EWORKSPACE and call(wsb=wb - 1)[0] == R.REC_EWORKSPACE
    assert call(ws=FAKE + 16)[0] == R.REC_EINVAL
    assert call(n=0, keys=None, iv=None, ws=None)[0] == R.REC_OK
