"""The forward as the benchmark times it: rec_sparse_din_fwd captured in HIP
graphs (one stream holding every batch's step, and batch k on stream k mod n
with one graph per stream) and replayed several times, with the program's
own eager work and synchronisations between the replays.  Every replay must
rewrite the outputs (poisoned before it) bit for bit as the eager calls
wrote them."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import DEV, say
from sparse_embedding_din_amd import pipeline as PL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,B,nb,ns", [(2, 2048, 4, 1), (2, 2048, 8, 4), (5, 1024, 4, 2)])
def test_graph_replays_equal_eager(cfg, B, nb, ns):
    m = synth.make_model(synth.WORKLOADS[cfg])
    batches = [synth.make_batch(m, B=B, batch_index=i) for i in range(nb)]
    tabs, mlp = PL.DeviceTables(m.tables, DEV), PL.DeviceMLP(m, DEV)
    dbs = [PL.DeviceBatch(b, DEV) for b in batches]
    fws = [PL.SparseDinForward(tabs, mlp, B, m.cfg.max_len, DEV) for _ in dbs]
    say(f"graph replay cfg={cfg} B={B} batches={nb} streams={ns}")
    ref = []
    for f, db in zip(fws, dbs):
        f.run_whole(db)
        torch.cuda.synchronize()
        ref.append((f.pooled[:B].clone(), f.att[:B].clone()))
    strs = [torch.cuda.Stream() for _ in range(ns)]
    graphs = [torch.cuda.CUDAGraph() for _ in range(ns)]
    for i in range(ns):
        with torch.cuda.graph(graphs[i], stream=strs[i]):
            for k in range(i, nb, ns):
                fws[k].run_whole(dbs[k])
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device=DEV)
    for rep in range(4):
        for f in fws:                                   # poison every output
            f.pooled.fill_(float("nan"))
            f.att.fill_(float("nan"))
        scratch.uniform_()                              # eager work between replays
        torch.cuda.synchronize()
        for i in range(ns):
            strs[i].wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(strs[i]):
                graphs[i].replay()
        torch.cuda.synchronize()
        for k, f in enumerate(fws):
            assert torch.equal(f.pooled[:B], ref[k][0]), (rep, k, "pooled")
            assert torch.equal(f.att[:B], ref[k][1]), (rep, k, "att")
        # an eager call of one batch between replays leaves the rest unchanged
        fws[rep % nb].run_whole(dbs[rep % nb])
        torch.cuda.synchronize()
        assert torch.equal(fws[rep % nb].att[:B], ref[rep % nb][1])
