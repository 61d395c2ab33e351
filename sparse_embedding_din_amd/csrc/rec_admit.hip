// Frequency admission and score-driven eviction for a lookup-only hash table,
// one batch of ids per call.
//
// Pages: "MultiTowerDIN：集成 DynamicEmb" §4.1 (an id enters its table only
// once it has been seen `threshold` times, and reads the constant 0 vector
// until then), §4.2 (the score strategy decides what leaves a full table:
// STEP the entry inserted earliest, LFU the least used; NO_EVICTION stops
// inserting), §2 and §7 (an initializer gives a new row its values), §1 (the
// slot layout).
//
// The ids of a call are taken together (include/rec.h states the rules).  On
// the device, one lane per batch position, in eight steps:
//   1. k_admit_clear: empties the batch's distinct-id set (workspace) and
//      counts, per block of slots, the keys the table holds;
//   2. k_admit_count: each id joins the set: its occurrences (atomic add)
//      and its first position (atomic min), so both end the same whatever
//      the order of the lanes;
//   3. k_admit_classify: the lane at an id's first position looks the id up:
//      a stored id is used (STEP writes the step, LFU adds the occurrences);
//      an absent one adds its occurrences to its count in the counter table
//      and becomes a candidate when the count reaches the threshold;
//   4. k_admit_blocks, k_admit_ranks: each candidate's rank in position
//      order (counts per 1024 positions, then an exclusive scan), and the
//      header: ids stored, candidates, room, entries to evict, ids admitted;
//   5. a stable LSD radix sort of the slots (only when something must be
//      evicted; the launches read the header and return otherwise) by the
//      stored id's low word, then its high word (sign flipped, so signed
//      order), then the saturated score, empty and tombstone slots last; so
//      the sorted order is by (score, id), whatever slots the ids hold;
//      k_admit_sortkeys writes each round's 32-bit keys;
//   6. k_admit_evict: the first entries of that order become tombstones;
//   7. k_admit_insert: candidates ranked below the admitted count claim the
//      first empty or tombstone slot of their probe sequence with a 64-bit
//      compare-and-swap (slots only fill in this phase, so every key keeps
//      an unbroken path from its home); the others keep their counts;
//   8. k_admit_lookup: the slot of every batch position after the call.
// Integer atomics only: every value stored, every count, the set of victims
// and of admitted ids are the same run to run; which free slot a new id
// takes may depend on the order of concurrent claims (lookups do not).
// Probes read slots with cached (workgroup-scope) loads: within a launch a
// slot only goes from free to a key, and a key that was stored before the
// launch never moves, so a stale read can only show a now-taken slot as
// free; the compare-and-swap that follows then fails and reports the key
// that is there.  A device-scope load per probe went to memory every time.
#include <limits.h>

#include "rec_internal.h"

namespace rec {
namespace {

constexpr uint32_t kScoreSat = 0xfffffffeu;     // scores compare saturated here
constexpr uint32_t kFreeKey = 0xffffffffu;      // sort key of empty and tombstone slots
enum { kHdrStored = 0, kHdrCand, kHdrRoom, kHdrEvict, kHdrAdmit };

__device__ inline bool reserved_key(int64_t k) { return k == REC_EMPTY_KEY || k == REC_TOMBSTONE_KEY; }
__device__ inline bool holds_key(int64_t k) { return !reserved_key(k); }

// The set entry of `key` (linear probing over nset, a power of two at least
// twice the batch, so never full); with insert, claims an empty entry.
__device__ inline int64_t set_entry(const AdmitArgs& a, int64_t key, bool insert) {
    int64_t e = (int64_t)(mix64((uint64_t)key) & (uint64_t)(a.nset - 1));
    for (int64_t probes = 0; probes < a.nset; ++probes) {
        int64_t cur = __hip_atomic_load(a.set_key + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (cur == key) return e;
        if (cur == REC_EMPTY_KEY) {
            if (!insert) return -1;
            int64_t seen = REC_EMPTY_KEY;
            if (__hip_atomic_compare_exchange_strong(a.set_key + e, &seen, key, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                return e;
            if (seen == key) return e;
        }
        e = (e + 1) & (a.nset - 1);
    }
    return -1;
}

// Counter table: the slot of `key`, or -1; with claim, an empty slot is
// taken (compare-and-swap) when the key is absent; -1 when it is full.
__device__ inline int64_t counter_slot(const AdmitArgs& a, int64_t key, bool claim) {
    int64_t at = hash_home(mix64((uint64_t)key), a.ccap);
    for (int64_t probes = 0; probes < a.ccap; ++probes) {
        const int64_t cur = __hip_atomic_load(a.ckeys + at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (cur == key) return at;
        if (cur == REC_EMPTY_KEY) {
            if (!claim) return -1;
            int64_t seen = REC_EMPTY_KEY;
            if (__hip_atomic_compare_exchange_strong(a.ckeys + at, &seen, key, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                return at;
            if (seen == key) return at;
        }
        at = at + 1 == a.ccap ? 0 : at + 1;
    }
    return -1;
}

__device__ inline int32_t block_sum_i32(int32_t v, int32_t* red) {
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__device__ inline int64_t block_sum_i64(int64_t v, int64_t* red) {
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void k_admit_clear(const AdmitArgs a) {
    __shared__ int32_t red[4];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < a.nset) {
        a.set_key[i] = REC_EMPTY_KEY;
        a.set_cnt[i] = 0;
        a.set_first[i] = INT_MAX;
    }
    const int32_t held = i < a.capacity && holds_key(a.keys[i]) ? 1 : 0;
    const int32_t s = block_sum_i32(held, red);
    if (threadIdx.x == 0) a.blk_stored[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_admit_count(const AdmitArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    const int64_t key = a.in_keys[i];
    if (reserved_key(key)) return;
    const int64_t e = set_entry(a, key, true);
    if (e < 0) return;                            // cannot happen: the set has room for 2n
    atomicAdd(a.set_cnt + e, 1u);
    atomicMin(a.set_first + e, (int32_t)i);
}

__global__ __launch_bounds__(256) void k_admit_classify(const AdmitArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    a.flag[i] = 0;
    const int64_t key = a.in_keys[i];
    if (reserved_key(key)) return;
    const int64_t e = set_entry(a, key, false);
    if (e < 0 || a.set_first[e] != (int32_t)i) return;
    const uint64_t c = a.set_cnt[e];
    const int64_t s = hash_probe(a.tab, key);
    if (s >= 0) {                                  // stored: used
        if (a.mode == REC_SCORE_STEP) a.scores[s] = a.step;
        if (a.mode == REC_SCORE_LFU) a.scores[s] += c;
        return;
    }
    const int64_t cs = counter_slot(a, key, false);
    const uint64_t total = (cs >= 0 ? a.ccounts[cs] : 0) + c;
    if (total < a.threshold) {
        const int64_t w = cs >= 0 ? cs : counter_slot(a, key, true);
        if (w >= 0) a.ccounts[w] = total;         // a full counter table counts no new id
        return;
    }
    a.flag[i] = 1;
    a.total[i] = total;
    a.cslot[i] = cs;
}

// Candidates per 1024 positions.
__global__ __launch_bounds__(256) void k_admit_blocks(const AdmitArgs a) {
    __shared__ int32_t red[4];
    int32_t c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t i = (int64_t)blockIdx.x * 1024 + k * 256 + threadIdx.x;
        c += i < a.n ? a.flag[i] : 0;
    }
    c = block_sum_i32(c, red);
    if (threadIdx.x == 0) a.blk_cnt[blockIdx.x] = c;
}

// Each candidate's rank among the candidates, in position order; block 0
// also writes the header.
__global__ __launch_bounds__(256) void k_admit_ranks(const AdmitArgs a) {
    __shared__ int32_t red[4];
    __shared__ int64_t red64[4];
    __shared__ int32_t wsum[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int32_t before = 0;
    for (int64_t j = t; j < (int64_t)blockIdx.x; j += 256) before += a.blk_cnt[j];
    before = block_sum_i32(before, red);
    // thread t holds positions 4t .. 4t+3 of the block
    const int64_t i0 = (int64_t)blockIdx.x * 1024 + 4 * t;
    int32_t f[4], run = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[k] = i0 + k < a.n ? a.flag[i0 + k] : 0;
        run += f[k];
    }
    int32_t inc = run;
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t u = __shfl_up(inc, d, 64);
        if (lane >= d) inc += u;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int32_t ex = before + inc - run;
    for (int k = 0; k < w; ++k) ex += wsum[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (f[k]) a.rank[i0 + k] = ex;
        ex += f[k];
    }
    if (blockIdx.x == 0) {
        int64_t stored = 0, cand = 0;
        for (int64_t j = t; j < a.nbs; j += 256) stored += a.blk_stored[j];
        for (int64_t j = t; j < a.nbn; j += 256) cand += a.blk_cnt[j];
        stored = block_sum_i64(stored, red64);
        cand = block_sum_i64(cand, red64);
        if (t == 0) {
            int64_t room = a.max_keys - stored;
            if (room < 0) room = 0;
            int64_t ev = 0;
            if (a.mode != REC_SCORE_NONE && cand > room) ev = min(cand - room, stored);
            a.hdr[kHdrStored] = stored;
            a.hdr[kHdrCand] = cand;
            a.hdr[kHdrRoom] = room;
            a.hdr[kHdrEvict] = ev;
            a.hdr[kHdrAdmit] = min(cand, room + ev);
        }
    }
}

// Round 0: position i is slot i, keyed by the low word of its id.  Rounds 1
// and 2 key position i by its slot's high id word (sign flipped) and then by
// its saturated score (free slots last).
__global__ __launch_bounds__(256) void k_admit_sortkeys(const AdmitArgs a, int round) {
    if (a.hdr[kHdrEvict] == 0) return;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.capacity) return;
    const uint32_t s = round == 0 ? (uint32_t)i : a.sort_v[i];
    const int64_t k = a.keys[s];
    if (round == 0) {
        a.sort_k[i] = (uint32_t)(uint64_t)k;
        a.sort_v[i] = s;
    } else if (round == 1) {
        a.sort_k[i] = (uint32_t)((uint64_t)k >> 32) ^ 0x80000000u;
    } else {
        const uint64_t sc = a.scores[s];
        a.sort_k[i] = holds_key(k) ? (sc < kScoreSat ? (uint32_t)sc : kScoreSat) : kFreeKey;
    }
}

__global__ __launch_bounds__(256) void k_admit_evict(const AdmitArgs a, const uint32_t* order) {
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= a.hdr[kHdrEvict]) return;
    const uint32_t s = order[v];
    a.keys[s] = REC_TOMBSTONE_KEY;                 // the digest stays: probes pass the slot
    a.scores[s] = 0;
}

__global__ __launch_bounds__(256) void k_admit_insert(const AdmitArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n || !a.flag[i]) return;
    const int64_t key = a.in_keys[i];
    const int64_t cs = a.cslot[i];
    if ((int64_t)a.rank[i] >= a.hdr[kHdrAdmit]) {  // left out: the count is kept
        const int64_t w = cs >= 0 ? cs : counter_slot(a, key, true);
        if (w >= 0) a.ccounts[w] = a.total[i];
        return;
    }
    const uint64_t h = mix64((uint64_t)key);
    int64_t at = hash_home(h, a.capacity), slot = -1;
    for (int64_t probes = 0; probes < a.capacity; ++probes) {
        int64_t cur = __hip_atomic_load(a.keys + at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (cur == REC_EMPTY_KEY || cur == REC_TOMBSTONE_KEY) {
            if (__hip_atomic_compare_exchange_strong(a.keys + at, &cur, key, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                slot = at;
                break;
            }
        }
        at = at + 1 == a.capacity ? 0 : at + 1;
    }
    if (slot < 0) return;                          // cannot happen: the room was counted
    a.digests[slot] = (uint8_t)hash_digest(h);
    const float4* src = (const float4*)(a.init_values + i * 16);
    float4* dst = (float4*)(a.values + slot * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r] = src[r];
    if (a.mode == REC_SCORE_STEP) a.scores[slot] = a.step;
    if (a.mode == REC_SCORE_LFU) a.scores[slot] = a.total[i];
    if (cs >= 0) a.ccounts[cs] = 0;
}

__global__ __launch_bounds__(256) void k_admit_lookup(const AdmitArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i == 0 && a.counts_out) {
        a.counts_out[0] = a.hdr[kHdrAdmit];
        a.counts_out[1] = a.hdr[kHdrEvict];
        a.counts_out[2] = a.hdr[kHdrCand] - a.hdr[kHdrAdmit];
    }
    if (i >= a.n || !a.slot_out) return;
    const int64_t key = a.in_keys[i];
    a.slot_out[i] = reserved_key(key) ? -2 : hash_probe(a.tab, key);
}

}  // namespace

AdmitLayout admit_layout(int64_t n, int64_t capacity, bool evict) {
    AdmitLayout L;
    L.nset = 64;
    while (L.nset < 2 * n) L.nset <<= 1;
    L.nbn = (n + 1023) / 1024;
    L.nbs = (max(L.nset, capacity) + 255) / 256;
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o += (bytes + 255) & ~(size_t)255; return at; };
    L.set_key = take(8 * (size_t)L.nset);
    L.set_cnt = take(4 * (size_t)L.nset);
    L.set_first = take(4 * (size_t)L.nset);
    L.flag = take(4 * (size_t)n);
    L.rank = take(4 * (size_t)n);
    L.total = take(8 * (size_t)n);
    L.cslot = take(8 * (size_t)n);
    L.blk_cnt = take(4 * (size_t)L.nbn);
    L.blk_stored = take(4 * (size_t)L.nbs);
    L.hdr = take(8 * 8);
    L.sort_k0 = L.sort_v0 = L.sort_k1 = L.sort_v1 = L.hist = L.tot = 0;
    if (evict) {
        L.sort_k0 = take(4 * (size_t)capacity);
        L.sort_v0 = take(4 * (size_t)capacity);
        L.sort_k1 = take(4 * (size_t)capacity);
        L.sort_v1 = take(4 * (size_t)capacity);
        L.hist = take(4 * 256 * (size_t)bwd_sort_tiles(capacity));
        L.tot = take(4 * 256);
    }
    L.bytes = o;
    return L;
}

hipError_t launch_hash_admit(AdmitArgs a, uint32_t* k1, uint32_t* v1, uint32_t* hist, uint32_t* tot,
                             hipStream_t s) {
    const dim3 blk(256);
    const unsigned gn = (unsigned)((a.n + 255) / 256);
    hipLaunchKernelGGL(k_admit_clear, dim3((unsigned)a.nbs), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_count, dim3(gn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_classify, dim3(gn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_blocks, dim3((unsigned)a.nbn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_ranks, dim3((unsigned)a.nbn), blk, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint32_t* order = nullptr;
    if (a.mode != REC_SCORE_NONE) {
        const dim3 gc((unsigned)((a.capacity + 255) / 256));
        for (int round = 0; round < 3; ++round) {
            // four 8-bit passes per round leave the result in (sort_k, sort_v)
            hipLaunchKernelGGL(k_admit_sortkeys, gc, blk, 0, s, a, round);
            const uint32_t* ks;
            e = launch_radix_sort(a.sort_k, a.sort_v, k1, v1, a.capacity, 32, hist, tot, a.hdr + kHdrEvict,
                                  s, &ks, &order);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_admit_evict, dim3(gn), blk, 0, s, a, order);
    }
    hipLaunchKernelGGL(k_admit_insert, dim3(gn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_lookup, dim3(gn), blk, 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
