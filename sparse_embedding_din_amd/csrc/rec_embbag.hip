// Sum-pooled embedding bags and lookup-only hash probes.
//
// Pages: "MultiTowerDIN：当前现状分析" §3 (one dense [N,16] fp32 table per id
// feature, row = raw_id % num_buckets) and §4.4 (the pooled deep input);
// "MultiTowerDIN：集成 DynamicEmb" §3.2 (open-addressing lookup, an unseen id
// gives the zero vector); DLRM essay (wmrh.cn/news/12459) §3.2 (EmbeddingBag
// sum pooling).
//
// Layout on the GPU: a wave pools two tables (2p, 2p+1) for 32 consecutive
// samples: lanes 0-31 take table 2p, lanes 32-63 table 2p+1, one bag per lane.
// Both descriptors are wave-uniform, the lengths/offsets of a wave are two
// 128-byte runs of the key-major KJT, and each sample's two 64-byte outputs
// form one full 128-byte line.  A round's id loads and then its row loads are
// issued together under the execution mask, only for the ids each bag still
// holds (misses load no row), so a lane has all of a round's loads of one kind
// in flight at once and short bags issue no duplicate loads.
//
// Given only the lengths (offsets == NULL), a wave derives its 64 bag offsets
// itself from the KJT sums: the sum of the block sums before its block and of
// the 32-sample chunk sums before its chunk, then a scan of its own 32
// lengths per table.  Those loads are independent of the lengths, so the
// offsets cost no extra round trip to memory.
#include "rec_embbag_dev.h"

namespace rec {
namespace {

template <bool kHash, bool kFused>
__global__ __launch_bounds__(64 * kWaves) void k_embbag_fwd(const EmbArgs a) {
    k_embbag_fwd_body<kHash, kFused>(a, blockIdx.x);
}

__global__ __launch_bounds__(64 * kWaves) void k_hash_lookup(const HashArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t i = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * 16 + (lane >> 2);
    const int q = lane & 3;
    if (i >= a.n) return;
    const int64_t slot = hash_probe(a.tab, a.keys[i]);
    if (a.slot_out && q == 0) a.slot_out[i] = slot;
    if (a.rows_out) {
        const float4 v = slot >= 0 ? *(const float4*)(a.tab.values + slot * 16 + 4 * q)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        *(float4*)(a.rows_out + i * 16 + 4 * q) = v;
    }
}

}  // namespace

hipError_t launch_embbag(const EmbArgs& a, hipStream_t s) {
    const int64_t waves = (int64_t)((a.T + 1) / 2) * ((a.B + 31) / 32);
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    bool hash = false;
    for (int t = 0; t < a.T; ++t) hash = hash || a.tab[t].kind == REC_HASH;
    const dim3 grid((unsigned)blocks), block(64 * kWaves);
    if (a.offsets) {
        if (hash) REC_LAUNCH(REC_TIME_GATHER, (k_embbag_fwd<true, false>), grid, block, 0, s, a);
        else REC_LAUNCH(REC_TIME_GATHER, (k_embbag_fwd<false, false>), grid, block, 0, s, a);
    } else {
        if (hash) REC_LAUNCH(REC_TIME_GATHER, (k_embbag_fwd<true, true>), grid, block, 0, s, a);
        else REC_LAUNCH(REC_TIME_GATHER, (k_embbag_fwd<false, true>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_hash_lookup(const HashArgs& a, hipStream_t s) {
    const int64_t waves = (a.n + 15) / 16;
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_hash_lookup, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
