"""The forward entry point that allocates nothing (rec_sparse_din_fwd_noalloc,
its workspace in the library's static device scratch) against the one that
takes a caller's workspace (rec_sparse_din_fwd): bit-identical pooled
output, attention output, scores, softmax weights, offsets and resolved rows,
on two calls in a row, the second with a smaller batch (the scratch keeps
the first call's contents)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import DEV, say
from sparse_embedding_din_amd import pipeline as PL
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu


def _outputs(fwd, b, db, noalloc):
    B = db.B
    P = int(np.minimum(b.seq_lengths, fwd.max_len).sum())
    dbg = dict(emb_rows=torch.full((db.nnz,), -7, dtype=torch.int64, device=DEV),
               seq_rows=torch.full((3 * max(db.seq_stride, 1),), -7, dtype=torch.int64, device=DEV),
               scores=torch.full((max(P, 1),), np.nan, dtype=torch.float32, device=DEV),
               weights=torch.full((max(P, 1),), np.nan, dtype=torch.float32, device=DEV))
    fwd.pooled.fill_(np.nan)
    fwd.att.fill_(np.nan)
    fwd.offsets.fill_(-7)
    fwd.seq_offsets.fill_(-7)
    args = fwd.whole_args(db, dbg)
    if noalloc:
        args.workspace, args.workspace_bytes = None, 0      # ignored by the no-alloc call
        R.rec_sparse_din_fwd_noalloc(args)
    else:
        R.rec_sparse_din_fwd(args)
    torch.cuda.synchronize()
    out = dict(pooled=fwd.pooled[:B], att=fwd.att[:B], offsets=fwd.offsets[: fwd.T * B + 1],
               seq_offsets=fwd.seq_offsets[: B + 1], **dbg)
    return {k: v.cpu().numpy().copy() for k, v in out.items()}


def test_noalloc_matches_workspace_call_twice():
    m = synth.make_model(synth.WORKLOADS[2], bias=True)
    tabs = PL.DeviceTables(m.tables, DEV)
    mlp = PL.DeviceMLP(m, DEV)
    fwd = PL.SparseDinForward(tabs, mlp, 8192, m.cfg.max_len, DEV)
    assert R.rec_sparse_din_fwd_workspace_bytes(16, 8192, 100) <= R.REC_NOALLOC_SCRATCH_BYTES
    for call, B in enumerate((8192, 1500)):
        b = synth.make_batch(m, batch_index=call, B=B)
        db = PL.DeviceBatch(b, DEV)
        say(f"no-alloc forward, call {call}: taobao tables, B={B}")
        ref = _outputs(fwd, b, db, noalloc=False)
        got = _outputs(fwd, b, db, noalloc=True)
        for k in ref:
            assert got[k].shape == ref[k].shape, k
            assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), k
        assert np.isfinite(got["att"]).all() and np.isfinite(got["pooled"]).all()


def test_noalloc_rejects_batch_beyond_scratch():
    """A batch whose workspace exceeds the static scratch is refused before
    anything is launched; the library keeps working afterwards."""
    m = synth.make_model(synth.WORKLOADS[1], bias=True)
    tabs = PL.DeviceTables(m.tables, DEV)
    mlp = PL.DeviceMLP(m, DEV)
    fwd = PL.SparseDinForward(tabs, mlp, 256, m.cfg.max_len, DEV)
    b = synth.make_batch(m, B=256)
    db = PL.DeviceBatch(b, DEV)
    args = fwd.whole_args(db)
    args.B = 1 << 20
    with pytest.raises(R.RecError) as e:
        R.rec_sparse_din_fwd_noalloc(args)
    assert e.value.status == R.REC_EWORKSPACE and "REC_NOALLOC_SCRATCH_BYTES" in str(e.value)
    ref = _outputs(fwd, b, db, noalloc=False)
    got = _outputs(fwd, b, db, noalloc=True)
    for k in ref:
        assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), k
