"""Seeded synthetic inputs shaped like the pages' Taobao-ads MultiTowerDIN workload.

This module is the ONE piece shared by the CPU oracle side and the HIP side: it
draws tables, KeyedJaggedTensor-style id batches, click sequences, attention-MLP
weights and pre-filled lookup-only hash tables.  It holds none of the forward's
arithmetic (no floor-mod, no pooling, no attention): it only produces inputs.

Sources for the shapes (page titles, sections):
  * "MultiTowerDIN：当前现状分析" §1 (feature table: 16 features, dim 16,
    num_buckets per feature; feature groups deep / seq), §4.1 (click sequence
    capped at 100, real lengths ~3-5), §2 (id features arrive as values/lengths).
  * "MultiTowerDIN：集成 DynamicEmb" §1 (slot = key 8 B + score 8 B + digest
    1 B + 16 fp32), §2.1 (initializer NORMAL std_dev 0.05), §3.2 (a miss
    returns the constant 0 vector).
  * DLRM essay (wmrh.cn/news/12459) §5.1: Xavier-uniform init, gain 1.

The hash-table layout convention (hash, home slot, digest, probing) is a data
format and is stated in include/rec.h; the builder below places keys by it.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# ----------------------------------------------------------------------------
# Feature order (the deep group's 16 features as the pages' feature table lists
# them; price last).  k is the key index used everywhere.
FEATURES = [
    "user_id", "adgroup_id", "campaign_id", "brand", "customer", "cate_id",
    "cms_segid", "cms_group_id", "final_gender_code", "age_level",
    "pvalue_level", "shopping_level", "occupation", "new_user_class_level",
    "pid", "price",
]
T = 16
DIM = 16
# The seq group's three sub-features (adgroup, cate, brand), sharing the
# top-level tables of the same name.
SEQ_KEYS = (1, 5, 3)
# Column of each seq sub-feature's slice inside the pooled [B, T*16] output.
QUERY_COL = tuple(16 * k for k in SEQ_KEYS)          # (16, 80, 48)

FULL_SIZES = [1141730, 846812, 423438, 461498, 255877, 12961, 98, 14, 3, 8,
              5, 5, 3, 6, 20, 101]
TINY_SIZES = [11417, 8468, 4234, 4615, 2559, 1296, 98, 14, 3, 8, 5, 5, 3, 6,
              20, 101]

HIDDEN1, HIDDEN2, DIN_IN = 256, 64, 192
# deep tower [256] -> 512 -> 256 -> 128; final MLP [128 + 48] -> 64 -> 1
TOWER_IN, TOWER_H = 256, (512, 256, 128)
FINAL_IN, FINAL_H = 176, 64
MAX_LEN = 100
EMPTY_KEY = -1
SEED_BASE = 20261202

U64 = np.uint64
MASK64 = (1 << 64) - 1


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    B: int
    sizes: tuple
    bag_law: str            # "u123": U{1,2,3}; "binom": 1 + Bin(4, 1/4)
    seq_law: str            # "geom4", "geom5": Geometric(1/mean) on {1,..}; "unif100": U{1..100}
    mlp_dtype: str          # "f32" or "bf16"
    zipf_keys: tuple = ()   # keys whose ids (deep and seq) follow Zipf(1.05)
    hash_keys: tuple = ()   # keys stored as lookup-only hash tables
    hash_capacity: int = 300000
    hash_load: float = 0.7
    hash_hit: float = 0.8
    max_len: int = MAX_LEN


WORKLOADS: Dict[int, Config] = {
    1: Config(1, "tiny_fp32_B256", 256, tuple(TINY_SIZES), "u123", "geom4", "f32"),
    2: Config(2, "taobao_B8192", 8192, tuple(FULL_SIZES), "u123", "geom4", "bf16"),
    3: Config(3, "long_seq_B8192", 8192, tuple(FULL_SIZES), "u123", "unif100", "bf16"),
    4: Config(4, "zipf_B65536", 65536, tuple(FULL_SIZES), "binom", "geom5", "bf16",
              zipf_keys=(0, 1, 2, 3, 4, 5)),
    5: Config(5, "hash_B8192", 8192, tuple(FULL_SIZES), "u123", "geom4", "bf16",
              hash_keys=(0, 1, 2, 3, 4)),
}


_BAG_DESC = {"u123": "bags U{1,2,3} ids", "binom": "bags 1+Bin(4,1/4) ids (mean 2)"}
_SEQ_DESC = {"geom4": "click sequences Geom(mean 4)", "geom5": "click sequences Geom(mean 5)",
             "unif100": "click sequences U{1..100}"}


def describe(cfg: Config) -> str:
    """One-line description of a workload's shapes and laws."""
    s = (f"B={cfg.B}, 16 dim-16 fp32 tables ({sum(cfg.sizes)} rows), {_BAG_DESC[cfg.bag_law]} "
         f"(price 1), {_SEQ_DESC[cfg.seq_law]} cap {cfg.max_len}, 3 sub-features")
    if cfg.zipf_keys:
        s += f", Zipf(1.05) ids for tables {list(cfg.zipf_keys)}"
    if cfg.hash_keys:
        s += (f", tables {list(cfg.hash_keys)} as lookup-only hash tables (capacity "
              f"{cfg.hash_capacity}, load {cfg.hash_load}, {int(cfg.hash_hit * 100)}% hits)")
    s += (", attn MLP 192-256-64-1 " +
          ("bf16 with fp32 accumulate" if cfg.mlp_dtype == "bf16" else "fp32"))
    return s


# ----------------------------------------------------------------------------
# Hash-table layout convention (a data format, documented in include/rec.h):
#   h      = SplitMix64 output mix of the key's 64 bits (Steele, Lea & Flood,
#            "Fast splittable pseudorandom number generators", OOPSLA 2014;
#            the mixing function with Stafford's "Mix13" shifts/multipliers)
#   home   = floor(h * capacity / 2^64)   (Lemire's multiply-high range map)
#   digest = h & 0xFF, with 0 replaced by 1 (0 marks an empty slot)
#   probe  = linear, wrapping, from home; no deletes, so no tombstones
def splitmix64_mix(keys: np.ndarray) -> np.ndarray:
    z = keys.astype(np.int64).view(U64).copy()
    z ^= z >> U64(30)
    z *= U64(0xBF58476D1CE4E5B9)
    z ^= z >> U64(27)
    z *= U64(0x94D049BB133111EB)
    z ^= z >> U64(31)
    return z


def home_slot(h: np.ndarray, capacity: int) -> np.ndarray:
    """floor(h * capacity / 2^64) for capacity < 2^32, in 64-bit pieces."""
    assert 0 < capacity < (1 << 32)
    cap = U64(capacity)
    hi = h >> U64(32)
    lo = h & U64(0xFFFFFFFF)
    return ((hi * cap + ((lo * cap) >> U64(32))) >> U64(32)).astype(np.int64)


def digest_of(h: np.ndarray) -> np.ndarray:
    d = (h & U64(0xFF)).astype(np.uint8)
    d[d == 0] = 1
    return d


def build_hash_table(keys: np.ndarray, vals: np.ndarray, capacity: int) -> dict:
    """Place distinct keys by the layout convention above (insertion in rounds:
    every pending key tries its current probe slot; the lowest-indexed key wins
    a free slot; losers move one slot on).  A key only ever moves past occupied
    slots, so every key is reachable from its home by linear probing."""
    n = keys.shape[0]
    assert n < capacity
    assert not np.any(keys == EMPTY_KEY)
    tab_keys = np.full(capacity, EMPTY_KEY, dtype=np.int64)
    tab_dig = np.zeros(capacity, dtype=np.uint8)
    tab_scores = np.zeros(capacity, dtype=np.uint64)
    # Empty slots hold NaN so that a lookup which reads one poisons its output.
    tab_vals = np.full((capacity, DIM), np.nan, dtype=np.float32)
    h = splitmix64_mix(keys)
    pos = home_slot(h, capacity)
    dig = digest_of(h)
    slot_of = np.full(n, -1, dtype=np.int64)
    pending = np.arange(n, dtype=np.int64)
    while pending.size:
        cand = pos[pending]
        free = tab_keys[cand] == EMPTY_KEY
        fidx = pending[free]
        fc = cand[free]
        uc, first = np.unique(fc, return_index=True)
        win = fidx[first]
        tab_keys[uc] = keys[win]
        slot_of[win] = uc
        won = np.zeros(n, dtype=bool)
        won[win] = True
        pending = pending[~won[pending]]
        pos[pending] = (pos[pending] + 1) % capacity
    tab_dig[slot_of] = dig
    tab_vals[slot_of] = vals
    tab_scores[slot_of] = np.arange(1, n + 1, dtype=np.uint64)  # insertion step, never read
    return dict(kind="hash", rows=capacity, keys=tab_keys, digests=tab_dig,
                scores=tab_scores, values=tab_vals, stored=keys.copy())


# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Model:
    cfg: Config
    tables: List[dict]          # per key: dict(kind, rows, values[, keys, digests, scores, stored])
    w1: np.ndarray              # fp32 [256,192] (values the kernel receives, bf16-representable for bf16)
    b1: np.ndarray              # fp32 [256]
    w2: np.ndarray              # fp32 [64,256]
    b2: np.ndarray              # fp32 [64]
    w3: np.ndarray              # fp32 [64]
    b3: float
    w1_bf16: Optional[np.ndarray] = None   # uint16 bit patterns when mlp_dtype == bf16
    w2_bf16: Optional[np.ndarray] = None
    zipf_perm: Optional[dict] = None
    zipf_cdf: Optional[dict] = None
    towers: Optional["Towers"] = None


@dataclasses.dataclass
class Towers:
    """Deep-tower and final-MLP parameters, output-major like nn.Linear.weight.
    Matrices hold the values the GPU receives (bf16-representable when the
    model's MLP dtype is bf16); *_bits are their bf16 bit patterns then."""
    wd1: np.ndarray             # fp32 [512,256]
    bd1: np.ndarray             # fp32 [512]
    wd2: np.ndarray             # fp32 [256,512]
    bd2: np.ndarray
    wd3: np.ndarray             # fp32 [128,256]
    bd3: np.ndarray
    wf: np.ndarray              # fp32 [64,176]
    bf: np.ndarray
    wo: np.ndarray              # fp32 [64]
    bo: float
    bits: Optional[dict] = None  # name -> uint16 bit patterns (bf16 models)


@dataclasses.dataclass
class Batch:
    B: int
    lengths: np.ndarray         # int32 [T*B], key-major (i = k*B + b)
    values: np.ndarray          # int64 [nnz], key-major
    seq_lengths: np.ndarray     # int32 [B]
    seq_values: np.ndarray      # int64 [3, P] packed (sample-major positions)
    seq_stride: int             # P


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 (round-to-nearest-even, torch's conversion); returns
    the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an fp32 bit pattern."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _xavier(rng, fan_out, fan_in):
    bound = np.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-bound, bound, size=(fan_out, fan_in)).astype(np.float32)


def make_model(cfg: Config, *, emb_std: float = 0.05, bias: bool = False,
               w3_scale: float = 1.0, mlp_dtype: Optional[str] = None,
               seed_offset: int = 0) -> Model:
    """Tables, MLP weights and (for hash keys) pre-filled hash tables.
    bias=False gives the zero biases of the benchmark; bias=True draws
    U(-0.1, 0.1) biases so that bias mistakes show in parity tests."""
    ss = np.random.SeedSequence(SEED_BASE + cfg.index + 1000 * seed_offset)
    s_tab, s_mlp, s_hash = ss.spawn(3)
    rng_t = np.random.default_rng(s_tab)
    tables = []
    zipf_perm, zipf_cdf = {}, {}
    for k in range(T):
        n = cfg.sizes[k]
        if k in cfg.hash_keys:
            rng_h = np.random.default_rng(np.random.SeedSequence([s_hash.entropy, k]))
            nkeys = int(round(cfg.hash_load * cfg.hash_capacity))
            keys = _distinct_keys(rng_h, nkeys)
            vals = (rng_t.standard_normal((nkeys, DIM), dtype=np.float32) * np.float32(emb_std))
            tables.append(build_hash_table(keys, vals, cfg.hash_capacity))
        else:
            vals = rng_t.standard_normal((n, DIM), dtype=np.float32) * np.float32(emb_std)
            tables.append(dict(kind="direct", rows=n, values=vals))
        if k in cfg.zipf_keys:
            rng_z = np.random.default_rng(np.random.SeedSequence([s_tab.entropy, 77, k]))
            zipf_perm[k] = rng_z.permutation(n).astype(np.int64)
            w = np.arange(1, n + 1, dtype=np.float64) ** -1.05
            c = np.cumsum(w)
            zipf_cdf[k] = c / c[-1]
    rng_m = np.random.default_rng(s_mlp)
    w1 = _xavier(rng_m, HIDDEN1, DIN_IN)
    w2 = _xavier(rng_m, HIDDEN2, HIDDEN1)
    w3 = _xavier(rng_m, 1, HIDDEN2).reshape(HIDDEN2) * np.float32(w3_scale)
    if bias:
        b1 = rng_m.uniform(-0.1, 0.1, HIDDEN1).astype(np.float32)
        b2 = rng_m.uniform(-0.1, 0.1, HIDDEN2).astype(np.float32)
        b3 = float(np.float32(rng_m.uniform(-0.1, 0.1)))
    else:
        b1 = np.zeros(HIDDEN1, np.float32)
        b2 = np.zeros(HIDDEN2, np.float32)
        b3 = 0.0
    dt = mlp_dtype or cfg.mlp_dtype
    w1b = w2b = None
    if dt == "bf16":
        w1b = _round_bf16(w1)
        w2b = _round_bf16(w2)
        w1 = bf16_bits_to_f32(w1b)
        w2 = bf16_bits_to_f32(w2b)
    m = Model(cfg, tables, w1, b1, w2, b2, w3, b3, w1b, w2b, zipf_perm, zipf_cdf)
    m.mlp_dtype = dt
    m.towers = make_towers(cfg, bias=bias, mlp_dtype=dt, seed_offset=seed_offset)
    return m


def make_towers(cfg: Config, *, bias: bool = False, mlp_dtype: Optional[str] = None,
                seed_offset: int = 0) -> Towers:
    """Xavier-uniform tower weights from a seed stream of their own (the
    tables and the attention MLP draw nothing different because of them)."""
    rng = np.random.default_rng(np.random.SeedSequence(
        [SEED_BASE + cfg.index + 1000 * seed_offset, 4096]))
    dims = [(TOWER_H[0], TOWER_IN), (TOWER_H[1], TOWER_H[0]), (TOWER_H[2], TOWER_H[1]),
            (FINAL_H, FINAL_IN)]
    ws = [_xavier(rng, o, i) for o, i in dims]
    wo = _xavier(rng, 1, FINAL_H).reshape(FINAL_H)
    if bias:
        bs = [rng.uniform(-0.1, 0.1, o).astype(np.float32) for o, _ in dims]
        bo = float(np.float32(rng.uniform(-0.1, 0.1)))
    else:
        bs = [np.zeros(o, np.float32) for o, _ in dims]
        bo = 0.0
    bits = None
    if (mlp_dtype or cfg.mlp_dtype) == "bf16":
        bits = {}
        for name, k in zip(("wd1", "wd2", "wd3", "wf"), range(4)):
            bits[name] = _round_bf16(ws[k])
            ws[k] = bf16_bits_to_f32(bits[name])
    return Towers(ws[0], bs[0], ws[1], bs[1], ws[2], bs[2], ws[3], bs[3], wo, bo, bits)


def _distinct_keys(rng, n):
    out = np.unique(rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max,
                                 size=n + n // 8 + 16, dtype=np.int64, endpoint=True))
    out = out[out != EMPTY_KEY]
    assert out.size >= n
    out = rng.permutation(out)[:n]
    return out


def _uniform_ids(rng, n):
    return rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=n,
                        dtype=np.int64, endpoint=True)


def _ids_for_key(model: Model, k: int, n: int, rng, rng_hash) -> np.ndarray:
    cfg = model.cfg
    if k in cfg.hash_keys:
        tab = model.tables[k]
        stored = tab["stored"]
        hit = rng_hash.random(n) < cfg.hash_hit
        out = np.empty(n, dtype=np.int64)
        out[hit] = stored[rng_hash.integers(0, stored.size, size=int(hit.sum()))]
        nm = int((~hit).sum())
        miss = _uniform_ids(rng_hash, nm)
        bad = np.isin(miss, stored) | (miss == EMPTY_KEY)
        while bad.any():
            miss[bad] = _uniform_ids(rng_hash, int(bad.sum()))
            bad = np.isin(miss, stored) | (miss == EMPTY_KEY)
        out[~hit] = miss
        return out
    if k in cfg.zipf_keys:
        rank = np.searchsorted(model.zipf_cdf[k], rng.random(n), side="right")
        rank = np.minimum(rank, cfg.sizes[k] - 1)
        return model.zipf_perm[k][rank]
    if k == T - 1:                       # price: already bucketized to [0, 101)
        return rng.integers(0, cfg.sizes[k], size=n, dtype=np.int64)
    return _uniform_ids(rng, n)


def make_batch(model: Model, batch_index: int = 0, B: Optional[int] = None,
               seq_law: Optional[str] = None) -> Batch:
    cfg = model.cfg
    B = cfg.B if B is None else B
    ss = np.random.SeedSequence([SEED_BASE + cfg.index, 1 + batch_index, B])
    s_len, s_ids, s_slen, s_sids, s_hq = ss.spawn(5)
    r_len = np.random.default_rng(s_len)
    r_ids = np.random.default_rng(s_ids)
    r_slen = np.random.default_rng(s_slen)
    r_sids = np.random.default_rng(s_sids)
    r_hq = np.random.default_rng(s_hq)
    lengths = np.empty((T, B), dtype=np.int32)
    for k in range(T):
        if k == T - 1:
            lengths[k] = 1
        elif cfg.bag_law == "u123":
            lengths[k] = r_len.integers(1, 4, size=B)
        elif cfg.bag_law == "binom":
            lengths[k] = 1 + r_len.binomial(4, 0.25, size=B)
        else:
            raise ValueError(cfg.bag_law)
    vals = []
    for k in range(T):
        vals.append(_ids_for_key(model, k, int(lengths[k].sum()), r_ids, r_hq))
    law = seq_law or cfg.seq_law
    if law == "geom4":
        sl = r_slen.geometric(1 / 4, size=B)
    elif law == "geom5":
        sl = r_slen.geometric(1 / 5, size=B)
    elif law == "unif100":
        sl = r_slen.integers(1, 101, size=B)
    else:
        raise ValueError(law)
    sl = np.minimum(sl, cfg.max_len).astype(np.int32)
    P = int(sl.sum())
    seq = np.empty((3, P), dtype=np.int64)
    for i, k in enumerate(SEQ_KEYS):
        seq[i] = _ids_for_key(model, k, P, r_sids, r_hq)
    return Batch(B, lengths.reshape(-1).copy(), np.concatenate(vals), sl, seq, P)


def padded_seq_layout(batch: Batch, pad_to: int, rng_seed: int = 7):
    """Re-lay the packed click sequences with a fixed stride of `pad_to`
    positions per sample (sample b starts at b*pad_to); the padding holds
    random ids that must never be read.  Returns (seq_values[3, B*pad_to],
    seq_offsets int64[B], stride)."""
    B = batch.B
    rng = np.random.default_rng(rng_seed)
    out = _uniform_ids(rng, 3 * B * pad_to).reshape(3, B * pad_to)
    starts = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(batch.seq_lengths, out=starts[1:])
    for b in range(B):
        n = int(batch.seq_lengths[b])
        out[:, b * pad_to: b * pad_to + n] = batch.seq_values[:, starts[b]:starts[b] + n]
    return out, (np.arange(B, dtype=np.int64) * pad_to), B * pad_to


# ----------------------------------------------------------------------------
# DLRM workload (DLRM essay, wmrh.cn/news/12459): §4.2's minimal model -- 13
# dense features (the Criteo layout it names), 8 sparse features with tables
# of 100000, 50000, 20000, 10000, 5000, 2000, 1000 and 500 rows, embedding
# width 96, bottom MLP 13 -> 128 -> 96, top MLP (S+1)(S+2)/2 -> 128 -> 64 -> 1;
# §3.2: each bag pools several ids (e.g. the last five clicked items) by sum
# or mean; §4.3: dense features are log-transformed and standardised (so
# N(0, 1) here) and ids are remapped to 0 .. rows-1; §5.1: Xavier-uniform
# weights, gain 1, for the tables too.
DLRM_SIZES = (100000, 50000, 20000, 10000, 5000, 2000, 1000, 500)
DLRM_DENSE = 13
DLRM_DIM = 96


@dataclasses.dataclass(frozen=True)
class DlrmConfig:
    index: int
    name: str
    B: int
    sizes: tuple = DLRM_SIZES
    n_dense: int = DLRM_DENSE
    dim: int = DLRM_DIM
    modes: tuple = (0,) * len(DLRM_SIZES)     # 0 sum, 1 mean, per table
    bag_max: int = 5                           # bags hold 1 .. bag_max ids (uniform)


DLRM_WORKLOADS: Dict[int, DlrmConfig] = {
    1: DlrmConfig(101, "dlrm_sum_B8192", 8192),
    2: DlrmConfig(102, "dlrm_mixed_B8192", 8192, modes=(0, 1, 0, 1, 0, 1, 0, 1)),
    # the interaction's measured shape (217 features of width 96): 216 tables
    # (their sizes are not given; 5000 rows each here) and the dense vector
    3: DlrmConfig(103, "dlrm_wide_F217_B4096", 4096, sizes=(5000,) * 216, modes=(0,) * 216),
}


@dataclasses.dataclass
class DlrmModel:
    cfg: DlrmConfig
    tables: List[np.ndarray]     # S arrays [rows][d] fp32
    modes: tuple
    wb1: np.ndarray
    bb1: np.ndarray
    wb2: np.ndarray
    bb2: np.ndarray
    wt1: np.ndarray
    bt1: np.ndarray
    wt2: np.ndarray
    bt2: np.ndarray
    wt3: np.ndarray
    bt3: float


@dataclasses.dataclass
class DlrmBatch:
    B: int
    dense: np.ndarray            # fp32 [B][n_dense]
    lengths: np.ndarray          # int32 [S*B], key-major
    values: np.ndarray           # int64 [nnz], key-major, ids in [0, rows)


def make_dlrm(cfg: DlrmConfig, *, bias: bool = False, emb_scale: float = 1.0) -> DlrmModel:
    """Xavier-uniform tables and layers; bias=True draws U(-0.1, 0.1) biases
    (parity tests), else zeros."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED_BASE, cfg.index]))
    S = len(cfg.sizes)
    npairs = (S + 1) * (S + 2) // 2
    tables = [_xavier(rng, n, cfg.dim) * np.float32(emb_scale) for n in cfg.sizes]
    wb1 = _xavier(rng, 128, cfg.n_dense)
    wb2 = _xavier(rng, cfg.dim, 128)
    wt1 = _xavier(rng, 128, npairs)
    wt2 = _xavier(rng, 64, 128)
    wt3 = _xavier(rng, 1, 64).reshape(64)

    def b(n):
        return (rng.uniform(-0.1, 0.1, n).astype(np.float32) if bias else np.zeros(n, np.float32))
    bb1, bb2, bt1, bt2 = b(128), b(cfg.dim), b(128), b(64)
    bt3 = float(np.float32(rng.uniform(-0.1, 0.1))) if bias else 0.0
    return DlrmModel(cfg, tables, tuple(cfg.modes), wb1, bb1, wb2, bb2, wt1, bt1, wt2, bt2, wt3, bt3)


def make_dlrm_batch(model: DlrmModel, batch_index: int = 0, B: Optional[int] = None) -> DlrmBatch:
    cfg = model.cfg
    B = cfg.B if B is None else B
    rng = np.random.default_rng(np.random.SeedSequence([SEED_BASE, cfg.index, 1 + batch_index, B]))
    S = len(cfg.sizes)
    dense = rng.standard_normal((B, cfg.n_dense)).astype(np.float32)
    lengths = rng.integers(1, cfg.bag_max + 1, size=(S, B)).astype(np.int32)
    vals = [rng.integers(0, cfg.sizes[t], size=int(lengths[t].sum()), dtype=np.int64)
            for t in range(S)]
    return DlrmBatch(B, dense, lengths.reshape(-1).copy(), np.concatenate(vals))
