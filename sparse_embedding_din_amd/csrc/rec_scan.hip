// Jagged bookkeeping on the GPU: lengths -> offsets (exclusive prefix sum),
// and the DIN plan (packed sequence starts + whole-sample tasks).
//
// Pages: "MultiTowerDIN：当前现状分析" §2 (id features are jagged values +
// lengths) and §4.1 (click sequences are short, ~3-5 of a cap of 100, so the
// attention works on packed positions instead of a [B,100] padding).
//
// Two launches, no inter-block waiting: a reduce pass writes one sum per
// 4096-length block; an apply pass has every block add up the sums before
// it, scan its own block through LDS, and write the results.
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

// Load the block's 4096 lengths into LDS (coalesced), padded so that each
// thread's 16 consecutive values sit in distinct banks.
__device__ inline void stage_chunk(const int32_t* len, int64_t n, int64_t base, int32_t* sl) {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int e = k * kScanThreads + (int)threadIdx.x;
        const int64_t idx = base + e;
        sl[e + (e >> 4)] = idx < n ? len[idx] : 0;
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
    __shared__ int32_t sl[kScanChunk + kScanChunk / 16];
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
        run += sl[t * 17 + k];
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

__global__ __launch_bounds__(kScanThreads) void k_plan_apply(const int32_t* __restrict__ len,
                                                            int64_t B, int32_t max_len,
                                                            int32_t task_positions,
                                                            int32_t total_waves, int64_t nblocks,
                                                            const int64_t* __restrict__ sums,
                                                            int64_t* __restrict__ seq_off,
                                                            int32_t* __restrict__ hdr,
                                                            int32_t* __restrict__ pos_start,
                                                            int2* __restrict__ task_info) {
    __shared__ int32_t sl[kScanChunk + kScanChunk / 16];
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanChunk;
    int64_t bc = 0, br = 0, tot = 0;
    for (int64_t j = threadIdx.x; j < nblocks; j += kScanThreads) {
        const int64_t c = sums[2 * j];
        if (j < (int64_t)blockIdx.x) { bc += c; br += sums[2 * j + 1]; }
        tot += c;
    }
    bc = block_sum(bc, red);
    br = block_sum(br, red);
    const int64_t P = block_sum(tot, red);
    // Positions per task: the requested value, or an even split of P over
    // every wave the attention kernel runs, rounded to the 16-row tile.
    int64_t C = task_positions;
    if (C == 0) {
        C = (P + total_waves - 1) / total_waves;
        C = (C + kMinTaskPositions - 1) / kMinTaskPositions * kMinTaskPositions;
        C = C < kMinTaskPositions ? kMinTaskPositions : (C > kMaxTaskPositions ? kMaxTaskPositions : C);
    }
    stage_chunk(len, B, base, sl);
    const int t = threadIdx.x;
    int32_t v[kScanItems];
    int64_t rc = 0, rr = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        v[k] = sl[t * 17 + k];
        rr += v[k];
        rc += v[k] < 0 ? 0 : (v[k] < max_len ? v[k] : max_len);
    }
    int64_t pc = block_excl_scan(rc, red) + bc;     // clamped prefix before this thread
    int64_t pr = block_excl_scan(rr, red) + br;     // raw prefix before this thread
    if (blockIdx.x == 0 && t == 0) task_info[0] = make_int2(0, 0);
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int64_t b = base + t * kScanItems + k;
        if (b >= B) break;
        const int64_t c = v[k] < 0 ? 0 : (v[k] < max_len ? v[k] : max_len);
        const int64_t next = pc + c;
        pos_start[b] = (int32_t)pc;
        if (seq_off) seq_off[b] = pr;
        // sample b+1 is the first sample of every task t with
        // pc < t*C <= next; the last sample also closes the task list.
        int64_t t_hi = next / C;
        if (b == B - 1) t_hi += 1;
        for (int64_t tt = pc / C + 1; tt <= t_hi; ++tt) task_info[tt] = make_int2((int32_t)(b + 1), (int32_t)next);
        if (b == B - 1) {
            pos_start[B] = (int32_t)next;
            if (seq_off) seq_off[B] = pr + v[k];
            hdr[kHdrB] = (int32_t)B;
            hdr[kHdrMaxLen] = max_len;
            hdr[kHdrC] = (int32_t)C;
            hdr[kHdrNumTasks] = (int32_t)(next / C + 1);
            hdr[kHdrP] = (int32_t)next;
            hdr[kHdrNBlocks] = (int32_t)nblocks;
        }
        pc = next;
        pr += v[k];
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

hipError_t launch_din_plan(const int32_t* seq_lengths, int64_t B, int32_t max_len,
                           int32_t task_positions, int32_t total_waves,
                           int64_t* seq_offsets_out, void* plan, hipStream_t s) {
    const PlanLayout L = plan_layout(B, max_len);
    char* p = (char*)plan;
    int64_t* sums = (int64_t*)(p + L.off_sums);
    hipLaunchKernelGGL(k_scan_reduce<true>, dim3((unsigned)L.nblocks), dim3(kScanThreads), 0, s,
                       seq_lengths, B, max_len, sums);
    hipLaunchKernelGGL(k_plan_apply, dim3((unsigned)L.nblocks), dim3(kScanThreads), 0, s,
                       seq_lengths, B, max_len, task_positions, total_waves, L.nblocks, sums,
                       seq_offsets_out, (int32_t*)p, (int32_t*)(p + L.off_pos),
                       (int2*)(p + L.off_task));
    return hipGetLastError();
}

}  // namespace rec
