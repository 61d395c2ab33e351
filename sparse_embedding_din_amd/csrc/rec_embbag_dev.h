// Device body of the embedding-bag kernel (one 4-wave block), shared by its
// own launch and the fused forward's.  Sum-pooled embedding bags:
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
// form one full 128-byte line.  A round resolves up to three ids per bag: a
// lane loads the ids its bag still holds, then their rows, each under the
// execution mask with no branch between the loads, so a lane has all of a
// round's id loads and then all of its row loads in flight at once.  Lanes past
// their bag's end (and misses) load nothing and add zeros: a bag of one id
// issues one id load and one row instead of three of each.
//
// Given only the lengths (offsets == NULL), a wave derives its 64 bag offsets
// itself from the KJT sums: the block sums before its block, the prefix of its
// segment inside the block and of its 32-sample chunk inside the segment,
// then a scan of its own 32 lengths per table.  Those loads are independent
// of the lengths, so the offsets cost no extra round trip to memory.
#pragma once
#include "rec_internal.h"

namespace rec {
namespace {

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kUnroll = 3;           // ids per bag resolved per round

// A table descriptor whose fields are pinned to scalar registers.  Choosing
// between two of them per lane is then a register select; choosing between
// two descriptors in the kernel arguments would compile into per-lane loads
// of the chosen descriptor's fields, a dependent round trip before any id.
__device__ inline uint64_t uniform64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ inline TabDev uniform_tab(const TabDev& t) {
    TabDev u;
    u.values = (const float*)(const float __attribute__((address_space(1)))*)uniform64((uint64_t)t.values);
    u.keys = (const int64_t*)(const int64_t __attribute__((address_space(1)))*)uniform64((uint64_t)t.keys);
    u.digests = (const uint8_t*)(const uint8_t __attribute__((address_space(1)))*)uniform64((uint64_t)t.digests);
    u.rows = (int64_t)uniform64((uint64_t)t.rows);
    u.magic = uniform64(t.magic);
    u.shift = __builtin_amdgcn_readfirstlane(t.shift);
    u.kind = __builtin_amdgcn_readfirstlane(t.kind);
    return u;
}

__device__ inline TabDev pick_tab(bool hi, const TabDev& t1, const TabDev& t0) {
    TabDev r;
    r.values = hi ? t1.values : t0.values;
    r.keys = hi ? t1.keys : t0.keys;
    r.digests = hi ? t1.digests : t0.digests;
    r.rows = hi ? t1.rows : t0.rows;
    r.magic = hi ? t1.magic : t0.magic;
    r.shift = hi ? t1.shift : t0.shift;
    r.kind = hi ? t1.kind : t0.kind;
    return r;
}

template <bool kHash, bool kFused>
__device__ inline void k_embbag_fwd_body(const EmbArgs& a, int64_t bid) {
    const int lane = threadIdx.x & 63;
    // the wave index is uniform: pinning it lets the table descriptors be read
    // with scalar loads and chosen per lane by a register select
    const int64_t w = (int64_t)bid * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nbw = (a.B + 31) / 32;
    const int tp = (int)(w / nbw);
    if (2 * tp >= a.T) return;                               // wave-uniform
    const int64_t b = (w % nbw) * 32 + (lane & 31);
    const int t = 2 * tp + (lane >> 5);
    const bool live = b < a.B && t < a.T;
    const TabDev t0 = uniform_tab(a.tab[2 * tp]);
    const TabDev t1 = uniform_tab(a.tab[2 * tp + 1]);        // zeroed past T
    // lanes of a missing odd table read table 2p's rows (masked out below)
    const bool hi = lane >= 32 && 2 * tp + 1 < a.T;
    const TabDev tl = pick_tab(hi, t1, t0);
    const float* vals = tl.values;
    const int64_t rows = tl.rows;
    const uint64_t magic = tl.magic;
    const int32_t shift = tl.shift;
    const int tc = min(t, a.T - 1);
    const int64_t bag = (int64_t)tc * a.B + min(b, a.B - 1);
    int32_t len = a.lengths[bag];
    int64_t off;
    if (kFused) {
        const int64_t kc = w % nbw;                              // 32-sample chunk of table tc
        const int64_t seg = kc / kKjtSegChunks;                 // 1024-sample segment
        const int64_t blk = seg / a.G, g = seg % a.G;           // block, segment inside it
        const int c = (int)(kc % kKjtSegChunks);                // chunk inside the segment
        const int l = lane & 31;
        const int64_t nflat = (int64_t)tc * a.nK + blk;
        const int64_t sidx = nflat * a.G + g;
        // Every load of the prefix is issued before any sum waits on one: the
        // segment and chunk prefixes, then the block sums of everything before
        // this block (T * nK < 160, so at most five per lane) -- a loop that
        // added each block sum as it arrived paid one round trip per five
        // tables.
        const int64_t sp = a.kjt_segp[sidx], cp = a.kjt_chp[sidx * kKjtSegChunks + c];
        int64_t s = 0;
        for (int64_t i0 = l; i0 < nflat; i0 += 5 * 32) {
            int64_t v[5];
#pragma unroll
            for (int u = 0; u < 5; ++u) v[u] = a.kjt_bs[i0 + 32 * u < nflat ? i0 + 32 * u : 0];
#pragma unroll
            for (int u = 0; u < 5; ++u) s += i0 + 32 * u < nflat ? v[u] : 0;
        }
        if (l == 0) s += sp + cp;
        if (!live) len = 0;
        int64_t inc = len;
#pragma unroll
        for (int d = 1; d < 32; d <<= 1) {
            const int64_t u = __shfl_up(inc, d, 32);
            if (l >= d) inc += u;
        }
#pragma unroll
        for (int d = 16; d >= 1; d >>= 1) s += __shfl_xor(s, d, 32);
        off = s + inc - len;
        if (a.offsets_out) {
            if (live) a.offsets_out[bag] = off;
            if (live && t == a.T - 1 && b == a.B - 1) a.offsets_out[(int64_t)a.T * a.B] = off + len;
        }
    } else {
        off = a.offsets[bag];
        if (!live) len = 0;
    }
    float4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; __ballot(j0 < len) != 0; j0 += kUnroll) {
        int64_t raw[kUnroll], row[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            raw[u] = 0;
            if (j0 + u < len) raw[u] = a.values[off + j0 + u];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            row[u] = -1;
            if (j0 + u < len) {
                if (kHash) {
                    row[u] = tl.kind == REC_HASH ? hash_probe(tl, raw[u]) : floor_mod_magic(raw[u], rows, magic, shift);
                } else {
                    row[u] = floor_mod_magic(raw[u], rows, magic, shift);
                }
            }
        }
        float4 v[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool use = j0 + u < len && row[u] >= 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[u][r] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (use) {
                const float4* src = (const float4*)(vals + row[u] * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) v[u][r] = src[r];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[r].x += v[u][r].x;
                acc[r].y += v[u][r].y;
                acc[r].z += v[u][r].z;
                acc[r].w += v[u][r].w;
            }
        }
        if (a.rows_out) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (j0 + u < len) a.rows_out[off + j0 + u] = row[u];
        }
    }
    if (live) {
        float4* o = (float4*)(a.out + b * (int64_t)a.T * 16 + t * 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = acc[r];
    }
}

}  // namespace
}  // namespace rec
