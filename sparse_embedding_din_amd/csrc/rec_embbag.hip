// Sum-pooled embedding bags and lookup-only hash probes.
//
// Pages: "MultiTowerDIN：当前现状分析" §3 (one dense [N,16] fp32 table per id
// feature, row = raw_id % num_buckets) and §4.4 (the pooled deep input);
// "MultiTowerDIN：集成 DynamicEmb" §3.2 (open-addressing lookup, an unseen id
// gives the zero vector); DLRM essay (wmrh.cn/news/12459) §3.2 (EmbeddingBag
// sum pooling).
//
// Layout on the GPU: one wave pools one sample's 16 bags.  Lane l serves
// bag t = l/4 and the 16-byte quarter q = l%4 of each 64-byte row, so a
// wave's row loads are 16 rows x 64 B and its output store is the sample's
// whole 1 KiB KeyedTensor row in one coalesced write.  Ids are taken four at a
// time so that four independent row loads per lane are in flight.
#include "rec_internal.h"

namespace rec {
namespace {

constexpr int kWaves = 4;            // waves (samples) per workgroup
constexpr int kUnroll = 4;           // ids resolved per round

__global__ __launch_bounds__(64 * kWaves) void k_embbag_fwd(const EmbArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t b = item / a.chunks;
    const int t = (int)(item % a.chunks) * 16 + (lane >> 2);
    const int q = lane & 3;
    if (b >= a.B || t >= a.T) return;
    const TabDev& tab = a.tab[t];
    const int64_t bag = (int64_t)t * a.B + b;
    const int32_t len = a.lengths[bag];
    const int64_t off = a.offsets[bag];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < len; j0 += kUnroll) {
        int64_t row[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            row[u] = (j0 + u < len) ? resolve_row(tab, a.values[off + j0 + u]) : -1;
        float4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = row[u] >= 0 ? *(const float4*)(tab.values + row[u] * 16 + 4 * q)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (j0 + u < len) {
                acc.x += v[u].x;
                acc.y += v[u].y;
                acc.z += v[u].z;
                acc.w += v[u].w;
            }
        }
        if (a.rows_out && q == 0) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (j0 + u < len) a.rows_out[off + j0 + u] = row[u];
        }
    }
    *(float4*)(a.out + b * (int64_t)a.T * 16 + t * 16 + 4 * q) = acc;
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
    const int64_t items = a.B * a.chunks;
    const int64_t blocks = (items + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_embbag_fwd, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_hash_lookup(const HashArgs& a, hipStream_t s) {
    const int64_t waves = (a.n + 15) / 16;
    const int64_t blocks = (waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(k_hash_lookup, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
