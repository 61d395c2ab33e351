// Device bodies of the jagged-bookkeeping kernels (one block each), shared by
// their own launches and by the fused forward's launches.  See rec_scan.hip.
#pragma once
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

// KJT sums: block (t, K) covers segments g = 0..G-1 of 1024 samples of table
// t, one after another; thread i holds samples 4i..4i+3 of a segment, so
// eight threads make one 32-sample chunk.  Per segment the 32 chunk sums go
// through LDS into an exclusive scan; a running total gives the segments'
// exclusive prefix and, at the end, the block sum.
__device__ inline void k_kjt_sums_body(const int32_t* __restrict__ len, int64_t B, int64_t nK,
                                       int64_t G, int64_t* __restrict__ bs,
                                       int64_t* __restrict__ segp, int64_t* __restrict__ chp,
                                       int64_t bid) {
    __shared__ int64_t s_ch[kKjtSegChunks];
    const int64_t t = bid / nK, K = bid % nK;
    const int32_t* lt = len + t * B;
    int64_t run = 0;
    for (int64_t g = 0; g < G; ++g) {
        const int64_t seg = K * G + g;                   // segment index inside the table
        const int64_t b0 = seg * kScanChunk + (int64_t)threadIdx.x * kScanItems;
        int64_t v = 0;
#pragma unroll
        for (int k = 0; k < kScanItems; ++k)
            if (b0 + k < B) v += lt[b0 + k];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        if ((threadIdx.x & 7) == 0) s_ch[threadIdx.x >> 3] = v;
        __syncthreads();
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            const int64_t c = lane < kKjtSegChunks ? s_ch[lane] : 0;
            const int64_t inc = wave_incl_scan(c);
            const int64_t tot = __shfl(inc, kKjtSegChunks - 1, 64);
            const int64_t base = (t * nK + K) * G + g;
            if (lane < kKjtSegChunks) chp[base * kKjtSegChunks + lane] = inc - c;
            if (lane == 0) segp[base] = run;
            run += tot;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) bs[bid] = run;
}

// DIN plan sums over the sequence lengths, clamped to max_len and raw: per
// 1024-sample block the two block sums, then per 16-sample chunk (four
// threads) the two chunk sums.
__device__ inline void k_plan_sums_body(const int32_t* __restrict__ len,
                                                           int64_t B, int32_t max_len,
                                                           int64_t* __restrict__ sums,
                                                           int32_t* __restrict__ hdr,
                                                           int64_t bid) {
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t b0 = (int64_t)bid * kScanChunk + (int64_t)threadIdx.x * kScanItems;
    int64_t raw = 0, cl = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        if (b0 + k < B) {
            const int32_t v = len[b0 + k];
            raw += v;
            cl += v < 0 ? 0 : (v < max_len ? v : max_len);
        }
    }
    int64_t* out = sums + (int64_t)bid * kPlanSumWords;
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
    if (bid == 0 && threadIdx.x == 0) hdr[kHdrNEmpty] = 0;   // k_plan_build appends
}

// The plan for 16 samples per block.  Wave 0 adds up the sums before the
// block (and all of them: P, hence the attention's group span), scans the 16 lengths
// and writes the per-sample arrays (and, in the block holding the last
// sample, the header); then every thread takes packed positions of the block,
// finds its sample among the 16 starts in LDS, and writes the position's
// sample, step and the rows of its three ids.  The position g * span of a
// group boundary also writes where group g starts: at the start of the sample
// holding that position or of the next one, whichever is nearer (a group's
// ends then move by at most half a sample).
template <bool kHash>
__device__ inline void k_plan_build_body(const PlanArgs a, int64_t bid, int64_t nblk) {
    __shared__ int32_t s_start[kPlanChunk + 1];
    __shared__ int64_t s_base[kPlanChunk];
    __shared__ int64_t s_span;
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
    int32_t* group_start = (int32_t*)(pb + Lo.off_group);
    const int64_t B = a.B;
    const int32_t max_len = a.max_len;
    const int64_t b0 = (int64_t)bid * kPlanChunk;
    const int nval = (int)min((int64_t)kPlanChunk, B - b0);
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int64_t K = b0 / kScanChunk;
        const int c = (int)((b0 % kScanChunk) / kPlanChunk);
        // sums of every sample before the block, clamped and raw, and the
        // clamped total P.  The chunk sums and the block's lengths are loaded
        // ahead of the block sums, so all of them are in flight at once.
        const int64_t b = b0 + min(lane, nval - 1);
        const int32_t v = lane < nval ? a.seq_lengths[b] : 0;
        int64_t pc = lane < c ? sums[K * kPlanSumWords + 2 + 2 * lane] : 0;
        int64_t pr = lane < c ? sums[K * kPlanSumWords + 3 + 2 * lane] : 0;
        int64_t ptot = 0;
        for (int64_t i = lane; i < Lo.nblocks; i += 64) {
            const int64_t cs = sums[i * kPlanSumWords];
            const int64_t rs = sums[i * kPlanSumWords + 1];
            ptot += cs;
            pc += i < K ? cs : 0;
            pr += i < K ? rs : 0;
        }
        const int64_t sb_given = a.seq_offsets ? a.seq_offsets[b] : 0;
        pc = wave_sum(pc);
        pr = wave_sum(pr);
        ptot = wave_sum(ptot);
        const int64_t span = din_span(ptot, a.range_positions, a.waves);
        if (lane == 0) s_span = span;
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
                hdr[kHdrNGroups] = (int32_t)((ptot + span - 1) / span);
                group_start[0] = 0;
                group_start[(ptot + span - 1) / span] = (int32_t)ptot;   // ps + vc == ptot
            }
        }
    }
    __syncthreads();
    const int64_t P0 = s_start[0], P1 = s_start[nval], span = s_span;
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
        if (p > 0 && p % span == 0) group_start[p / span] = 2 * j <= L ? st : st + L;
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
}  // namespace rec
