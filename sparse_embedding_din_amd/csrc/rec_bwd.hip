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
//   2. a stable radix sort of (key, source) pairs over the key's bits.
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
#include <rocprim/device/device_radix_sort.hpp>

#include "rec_internal.h"

namespace rec {

namespace {

constexpr int kChunk = 16;       // sorted contributions per 16-lane group

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
            const int64_t r = floor_mod_magic(a.values[off + i], tb.rows, tb.magic, tb.shift);
            a.keys_in[off + i] = tb.base + (uint32_t)r;
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
    const int64_t r = floor_mod_magic(a.seq_values[k * a.seq_stride + j], tb.rows, tb.magic, tb.shift);
    const int64_t c = a.nnz + k * a.P + j;
    a.keys_in[c] = tb.base + (uint32_t)r;
    a.src_in[c] = (uint32_t)(a.B * a.T + k * a.P + j);
}

// One element of the AdaGrad step: lane d of a group owns component d.
__device__ inline void adagrad_apply(const BwdTab* lt, const uint32_t* lbase, int T,
                                     uint32_t key, float g, int d, float lr, float eps) {
    const int t = table_of(lbase, T, key);
    const int64_t r = (int64_t)(key - lbase[t]);
    if (r >= lt[t].rows) return;                  // unreachable for keys built above
    float* w = lt[t].weights + r * REC_DIM + d;
    float* G = lt[t].accum + r * REC_DIM + d;
    const float gs = *G + g * g;
    *G = gs;
    *w = *w - lr * g / (sqrtf(gs) + eps);
}

// Gradient row of a source index; a source past the end reads nothing.
__device__ inline float grad_of(const BwdArgs& a, uint32_t src, int d) {
    const int64_t bt = a.B * a.T;
    if ((int64_t)src < bt) return a.grad_pooled[(int64_t)src * REC_DIM + d];
    const int64_t s = (int64_t)src - bt;
    if (s < 3 * a.P) return a.grad_seq[s * REC_DIM + d];
    return 0.0f;
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
// 3. chunk sums.  256 threads = 16 groups of 16 lanes, one chunk each.
__global__ __launch_bounds__(256) void k_bwd_chunks(BwdArgs a, BwdTabArr tabs) {
    __shared__ BwdTab lt[REC_MAX_TABLES];
    __shared__ uint32_t lbase[REC_MAX_TABLES];
    load_tables(tabs, a.T, lt, lbase);
    const int d = threadIdx.x & 15;
    const int grp = threadIdx.x >> 4;
    const int gl = (threadIdx.x & 63) & ~15;      // the group's first lane in its wave
    const int64_t c = (int64_t)blockIdx.x * 16 + grp;
    const int64_t n = a.n;
    const int64_t p0 = c * kChunk;
    if (p0 >= n) return;
    const int cnt = (int)((n - p0) < kChunk ? (n - p0) : kChunk);
    const uint32_t total = a.total_rows;

    // lane d: key and source of position p0 + d, and whether a run starts or
    // ends there
    const int64_t p = p0 + d;
    const bool in = d < cnt;
    const uint32_t key = in ? a.keys[p] : 0xffffffffu;
    const uint32_t src = in ? a.src[p] : 0xffffffffu;
    const bool head = in && (p == 0 || a.keys[p - 1] != key);
    const bool tail = in && (p + 1 >= n || a.keys[p + 1] != key);
    const uint64_t hm = (__ballot(head) >> gl) & 0xffffu;
    const uint64_t tm = (__ballot(tail) >> gl) & 0xffffu;

    float g[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const uint32_t si = (uint32_t)__shfl((int)src, gl + i, 64);
        g[i] = i < cnt ? grad_of(a, si, d) : 0.0f;
    }
    float acc = 0.0f;
    bool here = false;                            // the current run began in this chunk
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (i < cnt) {
            if ((hm >> i) & 1u) { acc = 0.0f; here = true; }
            acc += g[i];
            if ((tm >> i) & 1u) {
                const uint32_t ki = (uint32_t)__shfl((int)key, gl + i, 64);
                if (here) {
                    if (ki < total) adagrad_apply(lt, lbase, a.T, ki, acc, d, a.lr, a.eps);
                } else {
                    a.hpart[c * REC_DIM + d] = acc;
                }
            }
        }
    }
    if (!((tm >> (cnt - 1)) & 1u)) a.tpart[c * REC_DIM + d] = acc;
}

// ---------------------------------------------------------------------------
// 4. runs that cross chunks.  Each wave examines 64 chunks; a chunk is the
// END of a crossing run when its first position continues the previous
// chunk's run and that run ends inside it.
__global__ __launch_bounds__(256) void k_bwd_cross(BwdArgs a, BwdTabArr tabs) {
    __shared__ BwdTab lt[REC_MAX_TABLES];
    __shared__ uint32_t lbase[REC_MAX_TABLES];
    load_tables(tabs, a.T, lt, lbase);
    const int lane = threadIdx.x & 63;
    const int d = lane & 15;
    const int q = lane >> 4;
    const int64_t n = a.n;
    const int64_t nch = (n + kChunk - 1) / kChunk;
    const int64_t c0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;   // the wave's first chunk
    const int64_t c = c0 + lane;
    bool ends = false;
    if (c > 0 && c < nch) {
        const int64_t p0 = c * kChunk;
        const uint32_t k0 = a.keys[p0];
        if (a.keys[p0 - 1] == k0)
            ends = p0 + kChunk >= n || a.keys[p0 + kChunk - 1] != k0 || a.keys[p0 + kChunk] != k0;
    }
    uint64_t todo = __ballot(ends);
    while (todo) {
        const int m1 = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int64_t c1 = c0 + m1;
        const uint32_t K = a.keys[c1 * kChunk];
        float s = 0.0f;
        int64_t cc = c1 - 1;                      // newest chunk not yet summed
        for (;;) {
            // lane m: does the run also cover the position before chunk cc - m,
            // i.e. did it begin before that chunk?
            const int64_t cb = cc - lane;
            const bool before = cb > 0 && a.keys[cb * kChunk - 1] == K;
            const uint64_t bm = __ballot(before);
            const int nb = (~bm) ? __builtin_ctzll(~bm) + 1 : 64;   // chunks cc .. cc-nb+1
            for (int m = q; m < nb; m += 4) s += a.tpart[(cc - m) * REC_DIM + d];
            if (nb < 64 || bm != ~0ull) break;
            cc -= 64;
        }
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        const float gsum = s + a.hpart[c1 * REC_DIM + d];
        if (q == 0 && K < a.total_rows) adagrad_apply(lt, lbase, a.T, K, gsum, d, a.lr, a.eps);
    }
}

}  // namespace

size_t bwd_sort_bytes(int64_t n) {
    size_t bytes = 0;
    if (n <= 0) return 0;
    uint32_t* none = nullptr;                     // same iterator types as the launch
    if (rocprim::radix_sort_pairs(nullptr, bytes, none, none, none, none, (unsigned)n, 0u, 32u,
                                  (hipStream_t)nullptr) != hipSuccess)
        return 0;
    return bytes;
}

hipError_t launch_embbag_adagrad(BwdArgs a, const BwdTab* tabs, uint32_t* keys_out, uint32_t* src_out,
                                 void* sort_tmp, size_t sort_bytes, int key_bits, hipStream_t s) {
    BwdTabArr ta;
    memset(&ta, 0, sizeof(ta));
    for (int t = 0; t < a.T; ++t) ta.t[t] = tabs[t];
    const int64_t bag_blocks = (a.B + 255) / 256;
    const int64_t pos_blocks = (a.P + 255) / 256;
    const int64_t kb = (int64_t)a.T * bag_blocks + 3 * pos_blocks;
    if (kb > 0) hipLaunchKernelGGL(k_bwd_keys, dim3((unsigned)kb), dim3(256), 0, s, a, ta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    size_t bytes = sort_bytes;
    e = rocprim::radix_sort_pairs(sort_tmp, bytes, a.keys_in, keys_out, a.src_in, src_out,
                                  (unsigned)a.n, 0u, (unsigned)key_bits, s);
    if (e != hipSuccess) return e;
    a.keys = keys_out;
    a.src = src_out;
    const int64_t nch = (a.n + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(k_bwd_chunks, dim3((unsigned)((nch + 15) / 16)), dim3(256), 0, s, a, ta);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_cross, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, s, a, ta);
    return hipGetLastError();
}

}  // namespace rec
