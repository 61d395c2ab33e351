// Jagged bookkeeping on the GPU: lengths -> offsets (exclusive prefix sum),
// and the DIN plan (packed sequence starts + whole-sample tasks).
//
// Pages: "MultiTowerDIN：当前现状分析" §2 (id features are jagged values +
// lengths) and §4.1 (click sequences are short, ~3-5 of a cap of 100, so the
// attention works on packed positions instead of a [B,100] padding).
//
// Two launches, no inter-block waiting: a reduce pass writes one sum per
// 1024-length block; an apply pass has every block add up the sums before
// it, scan its own block through LDS, and write the results.  The DIN plan
// adds a third pass over the packed positions.
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

template <bool kPlan>
__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const int32_t* __restrict__ len,
                                                             int64_t n, int32_t max_len,
                                                             int64_t* __restrict__ sums) {
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanChunk;
    int64_t raw = 0, clamped = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int64_t idx = base + k * kScanThreads + threadIdx.x;
        if (idx < n) {
            const int32_t v = len[idx];
            raw += v;
            if (kPlan) clamped += v < 0 ? 0 : (v < max_len ? v : max_len);
        }
    }
    raw = block_sum(raw, red);
    if (kPlan) clamped = block_sum(clamped, red);
    if (threadIdx.x == 0) {
        if (kPlan) {
            sums[2 * blockIdx.x] = clamped;
            sums[2 * blockIdx.x + 1] = raw;
        } else {
            sums[blockIdx.x] = raw;
        }
    }
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

__global__ __launch_bounds__(kScanThreads) void k_plan_apply(const PlanArgs a, int64_t nblocks) {
    __shared__ int32_t sl[kScanChunk + kScanChunk / kScanItems];
    __shared__ int64_t red[kScanThreads / 64];
    const PlanLayout Lo = plan_layout(a.B, a.max_len);
    char* pb = (char*)a.plan;
    const int64_t* sums = (const int64_t*)(pb + Lo.off_sums);
    int32_t* hdr = (int32_t*)pb;
    int32_t* pos_start = (int32_t*)(pb + Lo.off_pos);
    int64_t* sbase = (int64_t*)(pb + Lo.off_sbase);
    const int64_t B = a.B;
    const int32_t max_len = a.max_len;
    const int64_t base = (int64_t)blockIdx.x * kScanChunk;
    int64_t bc = 0, br = 0;
    for (int64_t j = threadIdx.x; j < (int64_t)blockIdx.x; j += kScanThreads) {
        bc += sums[2 * j];
        br += sums[2 * j + 1];
    }
    bc = block_sum(bc, red);
    br = block_sum(br, red);
    stage_chunk(a.seq_lengths, B, base, sl);
    const int t = threadIdx.x;
    int32_t v[kScanItems];
    int64_t rc = 0, rr = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        v[k] = sl[sl_index(t * kScanItems + k)];
        rr += v[k];
        rc += v[k] < 0 ? 0 : (v[k] < max_len ? v[k] : max_len);
    }
    int64_t pc = block_excl_scan(rc, red) + bc;     // clamped prefix before this thread
    int64_t pr = block_excl_scan(rr, red) + br;     // raw prefix before this thread
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int64_t b = base + t * kScanItems + k;
        if (b >= B) break;
        const int64_t c = v[k] < 0 ? 0 : (v[k] < max_len ? v[k] : max_len);
        const int64_t next = pc + c;
        pos_start[b] = (int32_t)pc;
        if (a.seq_offsets_out) a.seq_offsets_out[b] = pr;
        sbase[b] = a.seq_offsets ? a.seq_offsets[b] : pr;
        if (b == B - 1) {
            pos_start[B] = (int32_t)next;
            if (a.seq_offsets_out) a.seq_offsets_out[B] = pr + v[k];
            hdr[kHdrB] = (int32_t)B;
            hdr[kHdrMaxLen] = max_len;
            hdr[kHdrRReq] = a.range_positions;
            hdr[kHdrP] = (int32_t)next;
            hdr[kHdrNBlocks] = (int32_t)nblocks;
        }
        pc = next;
        pr += v[k];
    }
}

// Per packed position: its sample and step, and the rows of its three ids.
// A 64-lane group serves one sample (positions j = lane, lane + 64, ...), so
// the id reads and the entry writes of a group are contiguous.
template <bool kHash>
__global__ __launch_bounds__(256) void k_plan_positions(const PlanArgs a) {
    const PlanLayout Lo = plan_layout(a.B, a.max_len);
    char* pb = (char*)a.plan;
    const int32_t* pos_start = (const int32_t*)(pb + Lo.off_pos);
    const int64_t* sbase = (const int64_t*)(pb + Lo.off_sbase);
    int32_t* pos_b = (int32_t*)(pb + Lo.off_pb);
    int32_t* pos_jr = (int32_t*)(pb + Lo.off_pjr);
    int32_t* pos_rows = (int32_t*)(pb + Lo.off_prows);
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int32_t ps = pos_start[b];
    const int32_t L = pos_start[b + 1] - ps;
    const int64_t g0 = sbase[b];
    for (int j = lane; j < L; j += 64) {
        const int64_t p = ps + j;
        const int64_t g = g0 + j;
        pos_b[p] = (int32_t)b;
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
        hipLaunchKernelGGL(k_scan_reduce<false>, dim3((unsigned)nb), dim3(kScanThreads), 0, s,
                           lengths, n, 0, block_sums);
    }
    hipLaunchKernelGGL(k_offsets_apply, dim3((unsigned)(nb > 0 ? nb : 1)), dim3(kScanThreads), 0,
                       s, lengths, n, block_sums, offsets);
    return hipGetLastError();
}

hipError_t launch_din_plan(const PlanArgs& a, hipStream_t s) {
    const PlanLayout L = plan_layout(a.B, a.max_len);
    char* p = (char*)a.plan;
    int64_t* sums = (int64_t*)(p + L.off_sums);
    hipLaunchKernelGGL(k_scan_reduce<true>, dim3((unsigned)L.nblocks), dim3(kScanThreads), 0, s,
                       a.seq_lengths, a.B, a.max_len, sums);
    hipLaunchKernelGGL(k_plan_apply, dim3((unsigned)L.nblocks), dim3(kScanThreads), 0, s, a, L.nblocks);
    const bool hash = a.tab[0].kind == REC_HASH || a.tab[1].kind == REC_HASH || a.tab[2].kind == REC_HASH;
    const dim3 grid((unsigned)((a.B + 3) / 4));
    if (hash) hipLaunchKernelGGL(k_plan_positions<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_plan_positions<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
