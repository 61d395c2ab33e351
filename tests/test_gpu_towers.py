"""GPU parity of the deep tower + final MLP (rec_towers_fwd) against the CPU
oracle on the same seeded inputs, and of the forward with the towers
attached.  deep_out is compared per row (1e-5 fp32, 2e-2 bf16).  The logit
is one dot product per sample that may cancel to near zero, so its error is
measured against the size of its terms, |bo| + sum_i |wo_i f_i| (from the
oracle); the probability's error, at most a quarter of the logit's (the
logistic function's slope is at most 1/4), against a quarter of that."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import BF16_TOL, DEV, FP32_TOL, row_rel_err, say
from sparse_embedding_din_amd import pipeline as PL
from sparse_embedding_din_amd import rec as R

pytestmark = pytest.mark.gpu


def _inputs(B, ld, std, seed):
    """Pooled rows shaped like sums of ~2 N(0, std) rows, attention output
    like one row; columns past 256 hold values the towers must not read."""
    rng = np.random.default_rng(seed)
    pooled = (rng.standard_normal((B, ld)) * std * 1.4).astype(np.float32)
    pooled[:, 256:] = 1e30
    att = (rng.standard_normal((B, 48)) * std).astype(np.float32)
    return pooled, att


def _run(tw, pooled, att, ld, want_deep=True, want_prob=True):
    B = pooled.shape[0]
    p = torch.from_numpy(pooled).to(DEV)
    a = torch.from_numpy(att).to(DEV)
    logit = torch.full((B + 1,), 7.0, dtype=torch.float32, device=DEV)
    deep = torch.full((B + 1, 128), 7.0, dtype=torch.float32, device=DEV) if want_deep else None
    prob = torch.full((B + 1,), 7.0, dtype=torch.float32, device=DEV) if want_prob else None
    R.rec_towers_fwd(tw.desc, B, p, ld, a, logit, deep_out=deep, prob=prob)
    torch.cuda.synchronize()
    out = dict(logit=logit.cpu().numpy())
    assert out["logit"][B] == 7.0, "logit written past B"
    if want_deep:
        out["deep"] = deep.cpu().numpy()
        assert np.all(out["deep"][B] == 7.0), "deep_out written past B"
    if want_prob:
        out["prob"] = prob.cpu().numpy()
        assert out["prob"][B] == 7.0, "prob written past B"
    return out


def _logit_errs(g_logit, g_prob, logit, prob, scale):
    el = float(np.max(np.abs(g_logit.astype(np.float64) - logit) / scale))
    ep = float(np.max(np.abs(g_prob.astype(np.float64) - prob) / (0.25 * scale)))
    return el, ep


CASES = [  # cfg, B, pooled_ld, input std, rows checked (None = all), packed bf16 weights
    (1, 256, 256, 0.05, None, False),
    (1, 37, 260, 0.05, None, False),
    (1, 100, 256, 1.0, None, False),
    (2, 8192, 256, 0.05, None, True),
    (2, 8192, 256, 0.05, None, False),
    (2, 1000, 272, 0.05, None, True),
    (2, 1, 256, 0.05, None, True),
    (2, 33, 256, 1.0, None, True),
    (2, 33, 256, 1.0, None, False),
    (4, 65536, 256, 0.05, 1024, True),
]


@pytest.mark.parametrize("cfg,B,ld,std,nsample,packed", CASES)
def test_towers_parity(cfg, B, ld, std, nsample, packed):
    say(f"towers cfg={cfg} B={B} ld={ld} std={std} packed={packed}")
    m = synth.make_model(synth.WORKLOADS[cfg], bias=True)
    tw = PL.DeviceTowers(m.towers, DEV, dtype=m.mlp_dtype, packed=packed)
    tol = FP32_TOL if m.mlp_dtype == "f32" else BF16_TOL
    pooled, att = _inputs(B, ld, std, seed=100 + cfg)
    g = _run(tw, pooled, att, ld)
    idx = np.arange(B) if nsample is None else \
        np.sort(np.random.default_rng(1).choice(B, nsample, replace=False))
    deep, logit, prob, scale = oracle.get().towers(pooled[idx], att[idx], m.towers, want_scale=True)
    e_deep = row_rel_err(g["deep"][idx], deep)
    e_logit, e_prob = _logit_errs(g["logit"][idx], g["prob"][idx], logit, prob, scale)
    say(f"  deep {e_deep:.3e} logit {e_logit:.3e} prob {e_prob:.3e} (tol {tol})")
    assert e_deep <= tol and e_logit <= tol and e_prob <= tol
    # the probability is the logistic function of the GPU's own logit
    lg = g["logit"][:B].astype(np.float64)
    assert np.max(np.abs(g["prob"][:B] - 1.0 / (1.0 + np.exp(-lg)))) < 1e-6


def test_towers_optional_outputs_and_determinism():
    """Same inputs -> same bits; the outputs do not depend on which optional
    outputs are asked for, nor on whether the weights are packed (the packed
    image only moves the same operands)."""
    m = synth.make_model(synth.WORKLOADS[2], bias=True)
    tw = PL.DeviceTowers(m.towers, DEV)
    plain = PL.DeviceTowers(m.towers, DEV, packed=False)
    assert tw.dtype == R.REC_BF16_PACKED and plain.dtype == R.REC_BF16
    pooled, att = _inputs(3000, 256, 0.05, seed=9)
    full = _run(tw, pooled, att, 256)
    again = _run(tw, pooled, att, 256)
    bare = _run(tw, pooled, att, 256, want_deep=False, want_prob=False)
    unpacked = _run(plain, pooled, att, 256)
    for k in ("logit", "deep", "prob"):
        assert np.array_equal(full[k], again[k]), k
        assert np.array_equal(full[k], unpacked[k]), k
    assert np.array_equal(full["logit"], bare["logit"])


def test_tower_pack_image():
    """The packed image holds every weight exactly once (plus the zero
    padding of wf's columns 176..191), bit for bit."""
    m = synth.make_model(synth.WORKLOADS[2], bias=True)
    tw = PL.DeviceTowers(m.towers, DEV)
    torch.cuda.synchronize()
    img = tw.packed.cpu().numpy().view(np.uint16)
    bits = m.towers.bits
    want = np.concatenate([bits[k].ravel() for k in ("wd1", "wd2", "wd3", "wf")])
    nz = img[img != 0]
    assert img.size == R.REC_TOWER_PACKED_BYTES // 2
    assert np.array_equal(np.sort(nz), np.sort(want[want != 0]))
    assert img.size - want.size == 64 * 16       # wf padding: 64 rows x 16 zero columns


def test_towers_sample_independence():
    """A sample's outputs depend on its own row only: a permuted batch gives
    the permuted outputs, bit for bit (each workgroup holds 32 samples, so
    this also moves samples across workgroups and ragged tails)."""
    m = synth.make_model(synth.WORKLOADS[2], bias=True)
    tw = PL.DeviceTowers(m.towers, DEV)
    pooled, att = _inputs(1500, 256, 0.05, seed=4)
    perm = np.random.default_rng(2).permutation(1500)
    a = _run(tw, pooled, att, 256)
    b = _run(tw, np.ascontiguousarray(pooled[perm]), np.ascontiguousarray(att[perm]), 256)
    for k in ("logit", "deep", "prob"):
        assert np.array_equal(a[k][:1500][perm], b[k][:1500]), k


def test_towers_zero_batch():
    m = synth.make_model(synth.WORKLOADS[2], bias=True)
    tw = PL.DeviceTowers(m.towers, DEV)
    logit = torch.full((4,), 7.0, device=DEV)
    p = torch.zeros(1, 256, device=DEV)
    a = torch.zeros(1, 48, device=DEV)
    R.rec_towers_fwd(tw.desc, 0, p, 256, a, logit)
    torch.cuda.synchronize()
    assert torch.all(logit == 7.0)


@pytest.mark.parametrize("cfg,B,whole", [(1, 256, False), (2, 8192, True), (5, 2000, True)])
def test_forward_with_towers(cfg, B, whole):
    """Sparse forward + towers against the oracle's whole forward (pooled and
    attention in fp64 feed the oracle's towers)."""
    m = synth.make_model(synth.WORKLOADS[cfg], bias=True)
    b = synth.make_batch(m, B=B)
    say(f"forward+towers cfg={cfg} B={B} whole={whole}")
    tabs = PL.DeviceTables(m.tables, DEV)
    mlp = PL.DeviceMLP(m, DEV)
    tw = PL.DeviceTowers(m.towers, DEV, dtype=m.mlp_dtype)
    fwd = PL.SparseDinForward(tabs, mlp, B, m.cfg.max_len, DEV, towers=tw)
    db = PL.DeviceBatch(b, DEV)
    (fwd.run_whole if whole else fwd.run)(db)
    torch.cuda.synchronize()
    o = oracle.forward(m, b, towers=True)
    tol = FP32_TOL if m.mlp_dtype == "f32" else BF16_TOL
    e_deep = row_rel_err(fwd.deep[:B].cpu().numpy(), o["deep"])
    e_logit, _ = _logit_errs(fwd.logit[:B].cpu().numpy(), fwd.prob[:B].cpu().numpy(), o["logit"],
                             o["prob"], o["logit_scale"])
    say(f"  deep {e_deep:.3e} logit {e_logit:.3e}")
    assert e_deep <= tol and e_logit <= tol
