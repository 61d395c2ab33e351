// Jagged bookkeeping on the GPU: lengths -> offsets (exclusive prefix sum),
// block sums from which the embedding bags derive their own offsets, and the
// DIN plan (packed sequence starts, per-position entries and rows).
//
// Pages: "MultiTowerDIN：当前现状分析" §2 (id features are jagged values +
// lengths) and §4.1 (click sequences are short, ~3-5 of a cap of 100, so the
// attention works on packed positions instead of a [B,100] padding).
//
// Two launches, no inter-block waiting: a reduce pass writes one sum per
// 1024-length block (and per smaller chunk where a consumer wants them); the
// consumer adds up the sums before its own piece and scans the piece itself.
// For plain offsets the consumer is an apply pass; for the KJT it is the
// embedding-bag kernel; for the DIN plan it is the pass that also writes the
// per-position entries.
#include "rec_internal.h"

namespace rec {
namespace {

__device__ inline int64_t wave_incl_scan(int64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

__device__ inline int64_t wave_sum(int64_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Sum of a value over the block (every thread gets it).
__device__ inline int64_t block_sum(int64_t v, int64_t* red /* [kScanThreads/64] */) {
    const int wave = threadIdx.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    int64_t s = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) s += red[w];
    return s;
}

// Exclusive prefix of v over the block's threads (thread order).
__device__ inline int64_t block_excl_scan(int64_t v, int64_t* red) {
    const int wave = threadIdx.x >> 6;
    const int64_t inc = wave_incl_scan(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 63) red[wave] = inc;
    __syncthreads();
    int64_t before = 0;
    for (int w = 0; w < wave; ++w) before += red[w];
    return before + inc - v;
}

// Load the block's lengths into LDS (coalesced), padded by one word per
// kScanItems so that each thread's consecutive values sit in distinct banks.
__device__ inline int sl_index(int e) { return e + e / kScanItems; }

__device__ inline void stage_chunk(const int32_t* len, int64_t n, int64_t base, int32_t* sl) {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int e = k * kScanThreads + (int)threadIdx.x;
        const int64_t idx = base + e;
        sl[sl_index(e)] = idx < n ? len[idx] : 0;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const int32_t* __restrict__ len,
                                                             int64_t n,
                                                             int64_t* __restrict__ sums) {
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanChunk;
    int64_t raw = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int64_t idx = base + k * kScanThreads + threadIdx.x;
        if (idx < n) raw += len[idx];
    }
    raw = block_sum(raw, red);
    if (threadIdx.x == 0) sums[blockIdx.x] = raw;
}

// KJT sums: block (t, K) covers samples [1024K, 1024K + 1024) of table t;
// thread i holds samples 4i..4i+3 of the block, so eight threads make one
// 32-sample chunk.
__global__ __launch_bounds__(kScanThreads) void k_kjt_sums(const int32_t* __restrict__ len,
                                                          int64_t B, int64_t nK,
                                                          int64_t* __restrict__ bs,
                                                          int64_t* __restrict__ cs) {
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t t = blockIdx.x / nK, K = blockIdx.x % nK;
    const int64_t b0 = K * kScanChunk + (int64_t)threadIdx.x * kScanItems;
    const int32_t* lt = len + t * B;
    int64_t v = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k)
        if (b0 + k < B) v += lt[b0 + k];
    int64_t c = v;
    c += __shfl_xor(c, 1, 64);
    c += __shfl_xor(c, 2, 64);
    c += __shfl_xor(c, 4, 64);
    if ((threadIdx.x & 7) == 0 && b0 < B)
        cs[t * nK * (kScanChunk / kKjtChunk) + b0 / kKjtChunk] = c;
    v = block_sum(v, red);
    if (threadIdx.x == 0) bs[blockIdx.x] = v;
}

// DIN plan sums over the sequence lengths, clamped to max_len and raw: per
// 1024-sample block the two block sums, then per 16-sample chunk (four
// threads) the two chunk sums.
__global__ __launch_bounds__(kScanThreads) void k_plan_sums(const int32_t* __restrict__ len,
                                                           int64_t B, int32_t max_len,
                                                           int64_t* __restrict__ sums,
                                                           int32_t* __restrict__ hdr_empty) {
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t b0 = (int64_t)blockIdx.x * kScanChunk + (int64_t)threadIdx.x * kScanItems;
    int64_t raw = 0, cl = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        if (b0 + k < B) {
            const int32_t v = len[b0 + k];
            raw += v;
            cl += v < 0 ? 0 : (v < max_len ? v : max_len);
        }
    }
    int64_t* out = sums + (int64_t)blockIdx.x * kPlanSumWords;
    int64_t cc = cl, cr = raw;
    cc += __shfl_xor(cc, 1, 64);
    cc += __shfl_xor(cc, 2, 64);
    cr += __shfl_xor(cr, 1, 64);
    cr += __shfl_xor(cr, 2, 64);
    if ((threadIdx.x & 3) == 0) {
        const int c = threadIdx.x >> 2;
        out[2 + 2 * c] = cc;
        out[3 + 2 * c] = cr;
    }
    cl = block_sum(cl, red);
    raw = block_sum(raw, red);
    if (threadIdx.x == 0) {
        out[0] = cl;
        out[1] = raw;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) hdr_empty[0] = 0;     // k_plan_build appends
}

__global__ __launch_bounds__(kScanThreads) void k_offsets_apply(const int32_t* __restrict__ len,
                                                               int64_t n,
                                                               const int64_t* __restrict__ sums,
                                                               int64_t* __restrict__ offsets) {
    __shared__ int32_t sl[kScanChunk + kScanChunk / kScanItems];
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanChunk;
    int64_t before = 0;
    for (int64_t j = threadIdx.x; j < (int64_t)blockIdx.x; j += kScanThreads) before += sums[j];
    before = block_sum(before, red);
    stage_chunk(len, n, base, sl);
    const int t = threadIdx.x;
    int64_t loc[kScanItems];
    int64_t run = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        run += sl[sl_index(t * kScanItems + k)];
        loc[k] = run;
    }
    const int64_t excl = block_excl_scan(run, red) + before;
    if (blockIdx.x == 0 && t == 0) offsets[0] = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int64_t idx = base + t * kScanItems + k;
        if (idx < n) offsets[idx + 1] = excl + loc[k];
    }
}

// The plan for 16 samples per block.  Wave 0 adds up the sums before the
// block, scans the 16 lengths and writes the per-sample arrays (and, in the
// block holding the last sample, the header); then every thread takes packed
// positions of the block, finds its sample among the 16 starts in LDS, and
// writes the position's sample, step and the rows of its three ids.
template <bool kHash>
__global__ __launch_bounds__(256) void k_plan_build(const PlanArgs a) {
    __shared__ int32_t s_start[kPlanChunk + 1];
    __shared__ int64_t s_base[kPlanChunk];
    const PlanLayout Lo = plan_layout(a.B, a.max_len);
    char* pb = (char*)a.plan;
    const int64_t* sums = (const int64_t*)(pb + Lo.off_sums);
    int32_t* hdr = (int32_t*)pb;
    int32_t* pos_start = (int32_t*)(pb + Lo.off_pos);
    int64_t* sbase = (int64_t*)(pb + Lo.off_sbase);
    int32_t* pos_b = (int32_t*)(pb + Lo.off_pb);
    int32_t* pos_jr = (int32_t*)(pb + Lo.off_pjr);
    int32_t* pos_rows = (int32_t*)(pb + Lo.off_prows);
    int32_t* empty = (int32_t*)(pb + Lo.off_empty);
    const int64_t B = a.B;
    const int32_t max_len = a.max_len;
    const int64_t b0 = (int64_t)blockIdx.x * kPlanChunk;
    const int nval = (int)min((int64_t)kPlanChunk, B - b0);
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int64_t K = b0 / kScanChunk;
        const int c = (int)((b0 % kScanChunk) / kPlanChunk);
        // sums of every sample before the block, clamped and raw
        int64_t pc = 0, pr = 0;
        for (int64_t i = lane; i < K; i += 64) {
            pc += sums[i * kPlanSumWords];
            pr += sums[i * kPlanSumWords + 1];
        }
        if (lane < c) {
            pc += sums[K * kPlanSumWords + 2 + 2 * lane];
            pr += sums[K * kPlanSumWords + 3 + 2 * lane];
        }
        const int64_t b = b0 + min(lane, nval - 1);
        const int32_t v = lane < nval ? a.seq_lengths[b] : 0;
        const int64_t sb_given = a.seq_offsets ? a.seq_offsets[b] : 0;
        pc = wave_sum(pc);
        pr = wave_sum(pr);
        const int64_t vc = v < 0 ? 0 : (v < max_len ? v : max_len);
        const int64_t ic = wave_incl_scan(vc), ir = wave_incl_scan((int64_t)v);
        const int64_t ps = pc + ic - vc, pr0 = pr + ir - v;
        // samples without positions join the empty list (one atomic per block)
        const uint64_t em = __ballot(lane < nval && vc == 0);
        if (em) {
            int32_t base = 0;
            if (lane == 0) base = atomicAdd(hdr + kHdrNEmpty, (int32_t)__popcll(em));
            base = __shfl(base, 0, 64);
            if (lane < nval && vc == 0)
                empty[base + __popcll(em & ((1ull << lane) - 1))] = (int32_t)b;
        }
        if (lane < nval) {
            pos_start[b] = (int32_t)ps;
            if (a.seq_offsets_out) a.seq_offsets_out[b] = pr0;
            const int64_t g = a.seq_offsets ? sb_given : pr0;
            sbase[b] = g;
            s_start[lane] = (int32_t)ps;
            s_base[lane] = g;
        }
        if (lane == nval - 1) {
            s_start[nval] = (int32_t)(ps + vc);
            if (b == B - 1) {
                pos_start[B] = (int32_t)(ps + vc);
                if (a.seq_offsets_out) a.seq_offsets_out[B] = pr0 + v;
                hdr[kHdrB] = (int32_t)B;
                hdr[kHdrMaxLen] = max_len;
                hdr[kHdrRReq] = a.range_positions;
                hdr[kHdrP] = (int32_t)(ps + vc);
                hdr[kHdrNBlocks] = (int32_t)Lo.nblocks;
            }
        }
    }
    __syncthreads();
    const int64_t P0 = s_start[0], P1 = s_start[nval];
    for (int64_t p = P0 + threadIdx.x; p < P1; p += 256) {
        int s = 0;
#pragma unroll
        for (int k = 1; k < kPlanChunk; ++k) s += (k < nval && s_start[k] <= p) ? 1 : 0;
        // a zero-length sample shares its start with the next one; the count
        // above lands on the last sample starting at or before p, which owns p
        const int32_t st = s_start[s];
        const int32_t L = s_start[s + 1] - st;
        const int32_t j = (int32_t)(p - st);
        const int64_t g = s_base[s] + j;
        pos_b[p] = (int32_t)(b0 + s);
        pos_jr[p] = j | ((L - 1 - j) << 16);
        int64_t raw[3];
#pragma unroll
        for (int f = 0; f < 3; ++f) raw[f] = a.seq_values[f * a.seq_stride + g];
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const TabDev& tb = a.tab[f];
            const int64_t row = kHash ? resolve_row(tb, raw[f]) : floor_mod_magic(raw[f], tb.rows, tb.magic, tb.shift);
            pos_rows[f * Lo.pmax + p] = (int32_t)row;
            if (a.rows_out) a.rows_out[f * a.seq_stride + g] = row;
        }
    }
}

}  // namespace

hipError_t launch_lengths_to_offsets(const int32_t* lengths, int64_t n, int64_t* offsets,
                                     int64_t* block_sums, hipStream_t s) {
    const int64_t nb = scan_blocks(n);
    if (nb > 0) {
        hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)nb), dim3(kScanThreads), 0, s, lengths, n,
                           block_sums);
    }
    hipLaunchKernelGGL(k_offsets_apply, dim3((unsigned)(nb > 0 ? nb : 1)), dim3(kScanThreads), 0,
                       s, lengths, n, block_sums, offsets);
    return hipGetLastError();
}

hipError_t launch_kjt_sums(const int32_t* lengths, int32_t T, int64_t B, void* sums, hipStream_t s) {
    const KjtLayout k = kjt_layout(T, B);
    int64_t* bs = (int64_t*)sums;
    int64_t* cs = (int64_t*)((char*)sums + k.off_cs);
    hipLaunchKernelGGL(k_kjt_sums, dim3((unsigned)(T * k.nK)), dim3(kScanThreads), 0, s, lengths, B,
                       k.nK, bs, cs);
    return hipGetLastError();
}

hipError_t launch_din_plan(const PlanArgs& a, hipStream_t s) {
    const PlanLayout L = plan_layout(a.B, a.max_len);
    char* p = (char*)a.plan;
    int64_t* sums = (int64_t*)(p + L.off_sums);
    hipLaunchKernelGGL(k_plan_sums, dim3((unsigned)L.nblocks), dim3(kScanThreads), 0, s,
                       a.seq_lengths, a.B, a.max_len, sums, (int32_t*)p + kHdrNEmpty);
    const bool hash = a.tab[0].kind == REC_HASH || a.tab[1].kind == REC_HASH || a.tab[2].kind == REC_HASH;
    const dim3 grid((unsigned)((a.B + kPlanChunk - 1) / kPlanChunk));
    if (hash) hipLaunchKernelGGL(k_plan_build<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_plan_build<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
