// Jagged bookkeeping on the GPU: lengths -> offsets (exclusive prefix sum),
// block sums from which the embedding bags derive their own offsets, and the
// DIN plan (packed sequence starts, per-position entries and rows).
//
// Pages: "MultiTowerDIN：当前现状分析" §2 (id features are jagged values +
// lengths) and §4.1 (click sequences are short, ~3-5 of a cap of 100, so the
// attention works on packed positions instead of a [B,100] padding).
//
// Plain offsets take three launches and no workspace: a reduce pass writes
// each 1024-length block's sum into the offsets array itself, at the first
// slot the block will later own (offsets[1024 k + 1]); one workgroup turns
// those sums into exclusive block prefixes in place; the apply pass then
// reads its block's prefix from that slot before writing its offsets over
// it (no other block reads or writes the slot).  The KJT and the DIN plan
// use two launches: a reduce pass writes one sum per block (and per smaller
// chunk where a consumer wants them) into their own buffers, and the
// consumer adds up the sums before its own piece and scans the piece itself
// (for the KJT the consumer is the embedding-bag kernel; for the plan, the
// pass that also writes the per-position entries).
#include "rec_scan_dev.h"

namespace rec {
namespace {

__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const int32_t* __restrict__ len,
                                                             int64_t n,
                                                             int64_t* __restrict__ offsets) {
    __shared__ int64_t red[kScanThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * kScanChunk;
    int64_t raw = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int64_t idx = base + k * kScanThreads + threadIdx.x;
        if (idx < n) raw += len[idx];
    }
    raw = block_sum(raw, red);
    if (threadIdx.x == 0) offsets[base + 1] = raw;
}

// One workgroup: the block sums at offsets[1024 k + 1] become the sums of
// the blocks before k, in block order.
__global__ __launch_bounds__(kScanThreads) void k_scan_blocks(int64_t nb,
                                                             int64_t* __restrict__ offsets) {
    __shared__ int64_t red[kScanThreads / 64];
    int64_t run = 0;
    for (int64_t c = 0; c < nb; c += kScanThreads) {
        const int64_t k = c + threadIdx.x;
        const int64_t v = k < nb ? offsets[k * kScanChunk + 1] : 0;
        const int64_t ex = block_excl_scan(v, red);
        const int64_t tot = block_sum(v, red);
        if (k < nb) offsets[k * kScanChunk + 1] = run + ex;
        run += tot;
    }
}

__global__ __launch_bounds__(kScanThreads) void k_offsets_apply(const int32_t* __restrict__ len,
                                                               int64_t n,
                                                               int64_t* __restrict__ offsets) {
    __shared__ int32_t sl[kScanChunk + kScanChunk / kScanItems];
    __shared__ int64_t red[kScanThreads / 64];
    __shared__ int64_t s_before;
    const int64_t base = (int64_t)blockIdx.x * kScanChunk;
    if (threadIdx.x == 0) s_before = n > 0 ? offsets[base + 1] : 0;
    stage_chunk(len, n, base, sl);          // its barrier also publishes s_before
    const int64_t before = s_before;
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

__global__ __launch_bounds__(kScanThreads) void k_kjt_sums(const int32_t* __restrict__ len,
                                                          int64_t B, int64_t nK, int64_t G,
                                                          int64_t* __restrict__ bs,
                                                          int64_t* __restrict__ segp,
                                                          int64_t* __restrict__ chp) {
    k_kjt_sums_body(len, B, nK, G, bs, segp, chp, blockIdx.x);
}

__global__ __launch_bounds__(kScanThreads) void k_plan_sums(const int32_t* __restrict__ len,
                                                           int64_t B, int32_t max_len,
                                                           int64_t* __restrict__ sums,
                                                           int32_t* __restrict__ hdr) {
    k_plan_sums_body(len, B, max_len, sums, hdr, blockIdx.x);
}

template <bool kHash>
__global__ __launch_bounds__(256) void k_plan_build(const PlanArgs a) {
    k_plan_build_body<kHash>(a, blockIdx.x, gridDim.x);
}

}  // namespace

hipError_t launch_lengths_to_offsets(const int32_t* lengths, int64_t n, int64_t* offsets,
                                     hipStream_t s) {
    const int64_t nb = scan_blocks(n);
    if (nb > 0) {
        hipLaunchKernelGGL(k_scan_reduce, dim3((unsigned)nb), dim3(kScanThreads), 0, s, lengths, n,
                           offsets);
        hipLaunchKernelGGL(k_scan_blocks, dim3(1), dim3(kScanThreads), 0, s, nb, offsets);
    }
    hipLaunchKernelGGL(k_offsets_apply, dim3((unsigned)(nb > 0 ? nb : 1)), dim3(kScanThreads), 0,
                       s, lengths, n, offsets);
    return hipGetLastError();
}

hipError_t launch_kjt_sums(const int32_t* lengths, int32_t T, int64_t B, void* sums, hipStream_t s) {
    const KjtLayout k = kjt_layout(T, B);
    char* p = (char*)sums;
    REC_LAUNCH(REC_TIME_SUMS, k_kjt_sums, dim3((unsigned)(T * k.nK)), dim3(kScanThreads), 0, s, lengths, B,
                       k.nK, k.G, (int64_t*)p, (int64_t*)(p + k.off_segp), (int64_t*)(p + k.off_chp));
    return hipGetLastError();
}

hipError_t launch_din_plan(const PlanArgs& a, hipStream_t s) {
    const PlanLayout L = plan_layout(a.B, a.max_len);
    char* p = (char*)a.plan;
    int64_t* sums = (int64_t*)(p + L.off_sums);
    hipLaunchKernelGGL(k_plan_sums, dim3((unsigned)L.nblocks), dim3(kScanThreads), 0, s,
                       a.seq_lengths, a.B, a.max_len, sums, (int32_t*)p);
    const bool hash = a.tab[0].kind == REC_HASH || a.tab[1].kind == REC_HASH || a.tab[2].kind == REC_HASH;
    const dim3 grid((unsigned)((a.B + kPlanChunk - 1) / kPlanChunk));
    if (hash) hipLaunchKernelGGL(k_plan_build<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_plan_build<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
