// Backward of the sum-pooled embedding bags and of the sequence rows, with one
// sparse AdaGrad step ("当前现状分析": run-config table, sparse AdaGrad with
// lr 1e-3; §3, an accumulator as large as the table; "集成 DynamicEmb" §3.3,
// fp32 gradient accumulation).
//
// Every read of a table row in the forward is one contribution: (the row, the
// output gradient of the read).  The step needs, per distinct row, the sum of
// its contributions before the square of AdaGrad, so duplicates must meet.
// They meet by sorting, which also fixes the order of every sum:
//
//   1. k_bwd_keys: one 32-bit key per contribution, the row in a flat row
//      space over all tables (table t owns base[t] .. base[t] + rows[t] - 1),
//      and one 32-bit source index: b*T + t for id reads of bag (t, b) (the
//      row of grad_pooled viewed as [B*T][16]), B*T + k*P + j for sequence
//      position j of sub-feature k (a row of grad_seq).  One wave per table
//      and 64 bags (or per sub-feature and 64 positions), so the table's
//      descriptor is wave-uniform.
//   2. a stable LSD radix sort of (key, source) pairs over the key's bits,
//      8 bits per pass, each pass three launches: k_sort_hist (per tile of
//      1024 pairs, the count of each digit), k_sort_scan (per digit, the
//      exclusive scan of its counts over the tiles, and its total), and
//      k_sort_scatter (each pair to its digit's place, stable: a tile is
//      ranked in 4 rounds of 256 pairs in order, each wave matching equal
//      digits by ballots, waves and rounds ordered by counters in LDS).
//      Every counter is written by a kernel: no memset, no atomics.
//   3. k_bwd_chunks: the sorted contributions in chunks of 16, one 16-lane
//      group per chunk, lane d owning component d.  The group loads its 16
//      gradient rows (64 contiguous bytes each) and sums each run of equal
//      keys in sorted order.  A run that begins and ends inside the chunk is
//      complete: the group applies its AdaGrad step at once.  A run that
//      leaves the chunk leaves a partial sum: its tail piece (tpart[c]) if it
//      continues into the next chunk, its head piece (hpart[c]) if it began
//      in an earlier one.
//   4. k_bwd_cross: one wave per run that crosses chunk boundaries, started
//      at the chunk where the run ends.  It walks back 64 chunks at a time
//      (one key per chunk tells whether the run covers the chunk's first
//      position), sums the tail pieces in a fixed order, adds the head piece
//      and applies the step.
//
// Hot rows (a 3-row table read once per sample) therefore cost one partial
// per 16 reads and one walk, not a serial chain of thousands of reads.  No
// floating-point atomics are used; every sum has one order.
#include <string.h>

#include "rec_internal.h"

namespace rec {

namespace {

constexpr int kChunk = 16;       // sorted contributions per 16-lane group
constexpr int kWalk = 8;         // chunks per lane per round of the cross-chunk walk (512 a round)

struct BwdTabArr {
    BwdTab t[REC_MAX_TABLES];
};

// Table of a flat row: the last table whose base is <= key (bases ascend).
__device__ inline int table_of(const uint32_t* base, int T, uint32_t key) {
    int lo = 0, hi = T - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (base[mid] <= key) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Flat row key of raw id x in table tb: direct, base + floor_mod(x, rows);
// hash, base + the slot holding x, or `miss` (the total row count, which
// sorts after every row and is skipped) when no slot holds it -- a miss read
// the constant zero vector and takes no gradient.
__device__ inline uint32_t row_key(const BwdTab& tb, int64_t x, uint32_t miss) {
    if (tb.tab.kind == REC_HASH) {
        const int64_t slot = hash_probe(tb.tab, x);
        return slot < 0 ? miss : tb.base + (uint32_t)slot;
    }
    return tb.base + (uint32_t)floor_mod_magic(x, tb.tab.rows, tb.tab.magic, tb.tab.shift);
}

// ---------------------------------------------------------------------------
// 1. keys and sources.  Blocks of 256 threads; block x covers 4 x 64 bags of
// one table (x < T * bag_blocks) or 4 x 64 positions of one sub-feature.
__global__ __launch_bounds__(256) void k_bwd_keys(BwdArgs a, BwdTabArr tabs) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int64_t bag_blocks = (a.B + 255) / 256;
    const int64_t x = blockIdx.x;
    if (x < (int64_t)a.T * bag_blocks) {
        const int t = (int)(x / bag_blocks);
        const int64_t b = (x - (int64_t)t * bag_blocks) * 256 + wv * 64 + lane;
        if (b >= a.B) return;
        const BwdTab tb = tabs.t[t];
        const int64_t bag = (int64_t)t * a.B + b;
        const int64_t off = a.offsets[bag];
        const int32_t len = a.lengths[bag];
        const uint32_t src = (uint32_t)(b * a.T + t);
        for (int32_t i = 0; i < len && off + i < a.nnz; ++i) {
            a.keys_in[off + i] = row_key(tb, a.values[off + i], a.total_rows);
            a.src_in[off + i] = src;
        }
        return;
    }
    const int64_t y = x - (int64_t)a.T * bag_blocks;
    const int64_t pos_blocks = (a.P + 255) / 256;
    const int k = (int)(y / pos_blocks);
    if (k >= 3) return;
    const int64_t j = (y - (int64_t)k * pos_blocks) * 256 + wv * 64 + lane;
    if (j >= a.P) return;
    const BwdTab tb = tabs.t[a.seq_table[k]];
    const int64_t c = a.nnz + k * a.P + j;
    a.keys_in[c] = row_key(tb, a.seq_values[k * a.seq_stride + j], a.total_rows);
    a.src_in[c] = (uint32_t)(a.B * a.T + k * a.P + j);
}

__device__ inline void load_tables(const BwdTabArr& tabs, int T, BwdTab* lt, uint32_t* lbase) {
    if (threadIdx.x == 0) {
        for (int t = 0; t < T; ++t) {
            lt[t] = tabs.t[t];
            lbase[t] = tabs.t[t].base;
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// 2. radix sort passes.  A tile is 1024 pairs: round r (0..3), thread t holds
// pair tile*1024 + r*256 + t, so the pairs of a tile are visited in order
// (1024 rather than 2048: twice the workgroups for the scatter's serial
// rounds, 101 against 105 us per AdaGrad call; 512 gave 105 us again).
constexpr int kSortThreads = 256;
constexpr int kSortRounds = 4;
constexpr int kSortTile = kSortThreads * kSortRounds;

__global__ __launch_bounds__(256) void k_sort_hist(const uint32_t* keys, int64_t n, int shift,
                                                   int64_t ntiles, uint32_t* hist) {
    __shared__ uint32_t h[256];
    const int t = threadIdx.x;
    const int64_t tile = blockIdx.x;
    h[t] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t idx = tile * kSortTile + r * kSortThreads + t;
        if (idx < n) atomicAdd(&h[(keys[idx] >> shift) & 255u], 1u);   // counts: order-free
    }
    __syncthreads();
    hist[(int64_t)t * ntiles + tile] = h[t];
}

// Inclusive scan of one value over the 256 threads (4 waves); returns it and
// leaves the block total in *total.  Uses red[0..3].
__device__ inline uint32_t block_scan256(uint32_t v, uint32_t* red, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)v, k, 64);
        if (lane >= k) v += o;
    }
    if (lane == 63) red[w] = v;
    __syncthreads();
    uint32_t before = 0;
    for (int j = 0; j < w; ++j) before += red[j];
    *total = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return v + before;
}

// Block d: exclusive scan of digit d's counts over the tiles, in place; its
// total to tot[d].
__global__ __launch_bounds__(256) void k_sort_scan(uint32_t* hist, int64_t ntiles, uint32_t* tot) {
    __shared__ uint32_t red[4];
    const int t = threadIdx.x;
    uint32_t* row = hist + (int64_t)blockIdx.x * ntiles;
    uint32_t carry = 0;
    for (int64_t j0 = 0; j0 < ntiles; j0 += kSortThreads) {
        const int64_t j = j0 + t;
        const uint32_t v = j < ntiles ? row[j] : 0u;
        uint32_t sum;
        const uint32_t inc = block_scan256(v, red, &sum);
        if (j < ntiles) row[j] = carry + inc - v;
        carry += sum;
    }
    if (t == 0) tot[blockIdx.x] = carry;
}

__global__ __launch_bounds__(256) void k_sort_scatter(const uint32_t* keys, const uint32_t* vals,
                                                      int64_t n, int shift, int64_t ntiles,
                                                      const uint32_t* hist, const uint32_t* tot,
                                                      uint32_t* keys_out, uint32_t* vals_out) {
    __shared__ uint32_t base[256];        // where digit d's pairs of this tile start
    __shared__ uint32_t wcnt[4][256];     // this round: pairs of digit d in wave w
    __shared__ uint32_t red[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t tile = blockIdx.x;
    uint32_t sum;
    const uint32_t td = tot[t];
    const uint32_t dstart = block_scan256(td, red, &sum) - td;          // digits below t
    base[t] = dstart + hist[(int64_t)t * ntiles + tile];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // every round's pair is loaded before the first round runs: loaded per
    // round, the dependent loads between barriers bounded the launch
    uint32_t kr[kSortRounds], vr[kSortRounds];
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t idx = tile * kSortTile + r * kSortThreads + t;
        kr[r] = idx < n ? keys[idx] : 0u;
        vr[r] = idx < n ? vals[idx] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t idx = tile * kSortTile + r * kSortThreads + t;
        const bool valid = idx < n;
        const uint32_t k = kr[r];
        const uint32_t v = vr[r];
        const uint32_t d = (k >> shift) & 255u;
#pragma unroll
        for (int j = 0; j < 4; ++j) wcnt[j][t] = 0;
        __syncthreads();
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint64_t m = __ballot((d >> b) & 1u);
            peers &= ((d >> b) & 1u) ? m : ~m;
        }
        const uint32_t rank = (uint32_t)__popcll(peers & lt_mask);
        if (valid && rank == 0) wcnt[w][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pos = base[d] + rank;
            for (int j = 0; j < w; ++j) pos += wcnt[j][d];
            if ((int64_t)pos < n) {
                keys_out[pos] = k;
                vals_out[pos] = v;
            }
        }
        __syncthreads();
        base[t] += wcnt[0][t] + wcnt[1][t] + wcnt[2][t] + wcnt[3][t];
    }
}

// ---------------------------------------------------------------------------
// A 16-float row held by one lane.
struct Row16 {
    float v[16];
};

__device__ inline void load_row(Row16& r, const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float4 x = q[u];
        r.v[4 * u + 0] = x.x;
        r.v[4 * u + 1] = x.y;
        r.v[4 * u + 2] = x.z;
        r.v[4 * u + 3] = x.w;
    }
}

__device__ inline void store_row(float* p, const Row16& r) {
    float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = make_float4(r.v[4 * u], r.v[4 * u + 1], r.v[4 * u + 2], r.v[4 * u + 3]);
}

// Gradient row of a source index (a source past the end reads zeros).
__device__ inline void grad_row(Row16& r, const BwdArgs& a, uint32_t src) {
    const int64_t bt = a.B * a.T;
    const int64_t s = (int64_t)src - bt;
    if ((int64_t)src < bt) {
        load_row(r, a.grad_pooled + (int64_t)src * REC_DIM);
    } else if (s < 3 * a.P) {
        load_row(r, a.grad_seq + s * REC_DIM);
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) r.v[e] = 0.0f;
    }
}

// Weights and accumulator row of a flat row key (null past a table's end,
// which keys built above never are).
__device__ inline float* locate(const BwdTab* lt, const uint32_t* lbase, int T, uint32_t key,
                                float** accum) {
    const int t = table_of(lbase, T, key);
    const int64_t r = (int64_t)(key - lbase[t]);
    if (r >= lt[t].rows) return nullptr;
    *accum = lt[t].accum + r * REC_DIM;
    return lt[t].weights + r * REC_DIM;
}

// The AdaGrad step of one whole row by one lane, on rows loaded beforehand.
__device__ inline void adagrad_store(float* wp, float* Gp, Row16& w, Row16& G, const Row16& g,
                                     float lr, float eps) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        G.v[e] = G.v[e] + g.v[e] * g.v[e];
        w.v[e] = w.v[e] - lr * g.v[e] / (sqrtf(G.v[e]) + eps);
    }
    store_row(Gp, G);
    store_row(wp, w);
}

// Value of the lane k places lower in the same 16-lane row (DPP row_shr:k);
// lanes below k get 0 (never used by the callers).
template <int k>
__device__ inline float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + k, 0xf, 0xf, false));
}

template <int k>
__device__ inline void seg_step(Row16& x, bool take) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float t = row_shr<k>(x.v[e]);
        x.v[e] += take ? t : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// 3. chunk sums.  256 threads = 16 groups of 16 lanes, one chunk of 16 sorted
// contributions per group, lane i holding position i's whole gradient row.
// A segmented inclusive scan across the group (DPP row shifts, a fixed tree)
// leaves at each run's last lane the sum of the run's part in the chunk.
__global__ __launch_bounds__(256) void k_bwd_chunks(BwdArgs a, BwdTabArr tabs) {
    __shared__ BwdTab lt[REC_MAX_TABLES];
    __shared__ uint32_t lbase[REC_MAX_TABLES];
    load_tables(tabs, a.T, lt, lbase);
    const int i = threadIdx.x & 15;
    const int gl = (threadIdx.x & 63) & ~15;      // the group's first lane in its wave
    const int64_t c = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int64_t n = a.n;
    const int64_t p0 = c * kChunk;
    if (p0 >= n) return;
    const int cnt = (int)((n - p0) < kChunk ? (n - p0) : kChunk);
    const int64_t p = p0 + i;
    const bool in = i < cnt;
    const uint32_t key = in ? a.keys[p] : 0xffffffffu;
    const uint32_t src = in ? a.src[p] : 0xffffffffu;
    const bool head = in && (p == 0 || a.keys[p - 1] != key);
    const bool tail = in && (p + 1 >= n || a.keys[p + 1] != key);
    // the previous chunk (always whole) and the key before it, loaded beside
    // this chunk's: a run that crosses into this chunk from the previous one
    // and began there is summed here whole
    const uint32_t keyp = c > 0 ? a.keys[p - kChunk] : 0xffffffffu;
    const uint32_t srcp = c > 0 ? a.src[p - kChunk] : 0xffffffffu;
    const uint32_t kbb = c > 1 ? a.keys[p0 - kChunk - 1] : 0xffffffffu;
    const uint32_t hm = (uint32_t)(__ballot(head) >> gl) & 0xffffu;
    const uint32_t K0 = (uint32_t)__shfl((int)key, gl, 64);       // the chunk's first key
    const uint32_t prevm = (uint32_t)(__ballot(c > 0 && keyp == K0) >> gl) & 0xffffu;   // a suffix
    // the run of K0 crosses in (the previous chunk ends with K0), began in
    // the previous chunk (before it, another key) and ends in this one
    const bool cross_in = (prevm >> 15) & 1u;
    const bool began_prev = cross_in && (!(prevm & 1u) || kbb != K0);
    const bool k0_ends = (uint32_t)(__ballot(tail && (hm & ((2u << i) - 1u)) == 0u) >> gl) & 0xffffu;
    const bool pair_run = began_prev && k0_ends;
    Row16 x, xp;
    grad_row(x, a, src);
    if (pair_run && ((prevm >> i) & 1u)) {
        grad_row(xp, a, srcp);
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) xp.v[e] = 0.0f;
    }
    // start of lane i's run inside the chunk (0 when it began earlier)
    const uint32_t upto = hm & ((2u << i) - 1u);
    const int s0 = upto ? 31 - __builtin_clz(upto) : 0;
    // a run that ends here and began in this chunk (or, whole here, in the
    // previous one) is complete: its weights and accumulator are loaded now,
    // beside the gradients
    const bool whole = tail && (upto || pair_run);
    float* Gp = nullptr;
    float* wp = (whole && key < a.total_rows) ? locate(lt, lbase, a.T, key, &Gp) : nullptr;
    Row16 w, G;
    if (wp) {
        load_row(w, wp);
        load_row(G, Gp);
    }
    seg_step<1>(x, i - 1 >= s0);
    seg_step<2>(x, i - 2 >= s0);
    seg_step<4>(x, i - 4 >= s0);
    seg_step<8>(x, i - 8 >= s0);
    if (pair_run) {
        // the previous chunk's part of the run, summed over the group by a
        // fixed tree (every lane ends with the sum)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float v = xp.v[e];
            v += __shfl_xor(v, 8, 16);
            v += __shfl_xor(v, 4, 16);
            v += __shfl_xor(v, 2, 16);
            v += __shfl_xor(v, 1, 16);
            xp.v[e] = v;
        }
    }
    if (tail) {
        if (upto) {
            if (wp) adagrad_store(wp, Gp, w, G, x, a.lr, a.eps);
        } else if (pair_run) {
#pragma unroll
            for (int e = 0; e < 16; ++e) x.v[e] = xp.v[e] + x.v[e];
            if (wp) adagrad_store(wp, Gp, w, G, x, a.lr, a.eps);
        } else {
            store_row(a.hpart + c * REC_DIM, x);  // head piece of a run begun earlier
        }
    } else if (in && i == cnt - 1) {
        store_row(a.tpart + c * REC_DIM, x);      // tail piece: the run goes on
    }
}

// ---------------------------------------------------------------------------
// 4. runs that span three or more chunks.  One 16-lane group checks each
// chunk; the wave walks back from each chunk of its groups that is the END
// of such a run (its first position continues the previous chunk's run,
// which ends inside it), 64 kWalk chunks per round, each lane loading its
// chunks' last keys and tail pieces together, so a round is one memory round
// trip (a 16-lane group walking 64 chunks per round took 19 us for the hot
// rows of a three-row table, about 340 chunks long).
__global__ __launch_bounds__(256) void k_bwd_cross(BwdArgs a, BwdTabArr tabs) {
    __shared__ BwdTab lt[REC_MAX_TABLES];
    __shared__ uint32_t lbase[REC_MAX_TABLES];
    const int i = threadIdx.x & 15;
    const int64_t n = a.n;
    const int64_t nch = (n + kChunk - 1) / kChunk;
    const int64_t c1 = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int64_t p1 = c1 * kChunk;
    // Whether a run of at least three chunks ends in this chunk: it crosses
    // in, did not begin in the previous chunk (those runs are summed by
    // k_bwd_chunks) and does not go on past this chunk.  The five keys are
    // loaded at once (clamped into the array), and a block with no such run
    // returns before copying the table descriptors.
    const bool valid = c1 >= 2 && c1 < nch;
    auto kat = [&](int64_t q) { return a.keys[valid ? (q < n ? q : n - 1) : 0]; };
    const uint32_t K = kat(p1), kb = kat(p1 - 1), kbb = kat(p1 - kChunk - 1);
    const uint32_t ke = kat(p1 + kChunk - 1), kn = kat(p1 + kChunk);
    const bool ends = valid && kb == K && kbb == K && !(p1 + kChunk < n && ke == K && kn == K);
    if (!__syncthreads_or(ends)) return;          // (uniform: the whole block)
    load_tables(tabs, a.T, lt, lbase);
    // The wave's groups whose chunk ends such a run, one after another, each
    // run walked by all 64 lanes; lane 0 owns its step, whose rows and head
    // piece load beside the walk.  Chunk cb before the run's last chunk holds
    // a piece of it exactly when its last key is the run's (the run then goes
    // on from it, so its tail piece was written).  A round looks at kWalk
    // chunks per lane (lane l: chunks cc - l - 64 u), adds the pieces of the
    // run's chunks, and is the last round once one of its chunks is not the
    // run's.
    const int lane = threadIdx.x & 63;
    uint64_t todo = __ballot(ends && i == 0);
    while (todo) {
        const int g0 = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int64_t cq = __shfl(c1, g0, 64);
        const uint32_t Kq = (uint32_t)__shfl((int)K, g0, 64);
        float* Gp = nullptr;
        float* wp = (lane == 0 && Kq < a.total_rows) ? locate(lt, lbase, a.T, Kq, &Gp) : nullptr;
        Row16 w, G, h;
        if (wp) {
            load_row(w, wp);
            load_row(G, Gp);
            load_row(h, a.hpart + cq * REC_DIM);
        }
        Row16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc.v[e] = 0.0f;
        int64_t cc = cq - 1;                      // newest chunk not yet summed
        for (;;) {
            uint32_t lk[kWalk];
            Row16 part[kWalk];
#pragma unroll
            for (int u = 0; u < kWalk; ++u) {
                const int64_t cb = cc - lane - 64 * u;
                lk[u] = cb >= 0 ? a.keys[cb * kChunk + kChunk - 1] : ~Kq;
                if (cb >= 0) load_row(part[u], a.tpart + cb * REC_DIM);
            }
            bool out = false;
#pragma unroll
            for (int u = 0; u < kWalk; ++u) {
                const bool mine = lk[u] == Kq;
                out = out || !mine;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc.v[e] += mine ? part[u].v[e] : 0.0f;
            }
            if (__ballot(out)) break;
            cc -= 64 * kWalk;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float v = acc.v[e];
            v += __shfl_xor(v, 32, 64);
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 8, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 1, 64);
            acc.v[e] = v;
        }
        if (wp) {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc.v[e] += h.v[e];
            adagrad_store(wp, Gp, w, G, acc, a.lr, a.eps);
        }
    }
}

}  // namespace

int64_t bwd_sort_tiles(int64_t n) { return (n + kSortTile - 1) / kSortTile; }

hipError_t launch_radix_sort(uint32_t* kin, uint32_t* vin, uint32_t* kout, uint32_t* vout, int64_t n,
                             int key_bits, uint32_t* hist, uint32_t* tot,
                             hipStream_t s, const uint32_t** keys_sorted, const uint32_t** vals_sorted) {
    // ping-pong between (kin, vin) and (kout, vout)
    const int64_t nt = bwd_sort_tiles(n);
    for (int shift = 0; shift < key_bits; shift += 8) {
        hipLaunchKernelGGL(k_sort_hist, dim3((unsigned)nt), dim3(kSortThreads), 0, s, kin, n, shift, nt,
                           hist);
        hipLaunchKernelGGL(k_sort_scan, dim3(256), dim3(kSortThreads), 0, s, hist, nt, tot);
        hipLaunchKernelGGL(k_sort_scatter, dim3((unsigned)nt), dim3(kSortThreads), 0, s, kin, vin, n, shift,
                           nt, hist, tot, kout, vout);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        uint32_t* tk = kin; kin = kout; kout = tk;
        uint32_t* tv = vin; vin = vout; vout = tv;
    }
    *keys_sorted = kin;                           // the last pass's output
    *vals_sorted = vin;
    return hipSuccess;
}

hipError_t launch_embbag_adagrad(BwdArgs a, const BwdTab* tabs, uint32_t* keys_out, uint32_t* src_out,
                                 uint32_t* sort_hist, uint32_t* sort_tot, int key_bits, hipStream_t s) {
    BwdTabArr ta;
    memset(&ta, 0, sizeof(ta));
    for (int t = 0; t < a.T; ++t) ta.t[t] = tabs[t];
    const int64_t bag_blocks = (a.B + 255) / 256;
    const int64_t pos_blocks = (a.P + 255) / 256;
    const int64_t kb = (int64_t)a.T * bag_blocks + 3 * pos_blocks;
    if (kb > 0) hipLaunchKernelGGL(k_bwd_keys, dim3((unsigned)kb), dim3(256), 0, s, a, ta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t *ks, *vs;
    e = launch_radix_sort(a.keys_in, a.src_in, keys_out, src_out, a.n, key_bits, sort_hist, sort_tot,
                          s, &ks, &vs);
    if (e != hipSuccess) return e;
    a.keys = ks;
    a.src = vs;
    const int64_t nch = (a.n + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(k_bwd_chunks, dim3((unsigned)((nch + 15) / 16)), dim3(256), 0, s, a, ta);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_cross, dim3((unsigned)((nch + 15) / 16)), dim3(256), 0, s, a, ta);
    return hipGetLastError();
}

}  // namespace rec
