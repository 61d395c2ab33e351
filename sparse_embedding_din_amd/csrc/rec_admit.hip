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
//   5. k_admit_select, 13 passes (only when something must be evicted; the
//      launches read the header and return otherwise): a radix selection of
//      the E-th smallest stored entry by (saturated score, id as a signed
//      integer), a 96-bit key taken 8 bits at a time from the top: pass p
//      counts digit p of the keys that share the digits chosen so far and
//      picks the digit where the E-th smallest lies; every block of the next
//      pass redoes that pick from the counts (so no extra launch), block 0
//      writes it down; ids are unique, so exactly E keys are at most the
//      selected one;
//   6. the pass whose chosen bin holds exactly the keys still sought (at the
//      latest the thirteenth) turns every stored key at most the bound into a
//      tombstone, and the passes after it return at once;
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
// The insert's claiming probe reads 32 slots per round trip.
#include <limits.h>

#include "rec_internal.h"

namespace rec {
namespace {

constexpr uint32_t kScoreSat = 0xfffffffeu;     // scores compare saturated here
constexpr uint32_t kFreeKey = 0xffffffffu;      // score word of empty and tombstone slots
constexpr int kSelPasses = 12;                  // 8-bit digits of the 96-bit eviction key
constexpr int kSelDone = 4 * (kSelPasses + 1);  // sel_state word: the selection is complete
constexpr int kSelBlocks = 512;
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
    if (a.sel_hist)                                // the selection's counts start at zero
        for (int64_t j = i; j < kSelPasses * 256; j += (int64_t)gridDim.x * 256) a.sel_hist[j] = 0;
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
            if (a.sel_state) {
                a.sel_state[0] = a.sel_state[1] = a.sel_state[2] = 0;
                a.sel_state[3] = ev;
                a.sel_state[kSelDone] = 0;
            }
        }
    }
}

// The 96-bit eviction key of slot s as three words, most significant first:
// the saturated score (free slots above every stored entry), the id's high
// word with the sign flipped and its low word, so unsigned word order is the
// order by (score, signed id).
__device__ inline void slot_key(const AdmitArgs& a, int64_t s, uint32_t (&w)[3]) {
    const int64_t k = a.keys[s];
    const uint64_t sc = a.scores[s];
    w[0] = holds_key(k) ? (sc < kScoreSat ? (uint32_t)sc : kScoreSat) : kFreeKey;
    w[1] = (uint32_t)((uint64_t)k >> 32) ^ 0x80000000u;
    w[2] = (uint32_t)(uint64_t)k;
}

// Digit p (0 .. 11, 8 bits each, most significant first) of a key.
__device__ inline uint32_t key_digit(const uint32_t (&w)[3], int p) {
    return (w[p >> 2] >> (24 - 8 * (p & 3))) & 255u;
}

// Whether a key's digits 0 .. p-1 are those of `pre`.
__device__ inline bool key_prefix_eq(const uint32_t (&w)[3], const uint32_t (&pre)[3], int p) {
    bool eq = true;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        const int nb = min(max(8 * p - 32 * q, 0), 32);        // bits of word q fixed so far
        const uint32_t mask = nb == 0 ? 0u : (nb == 32 ? ~0u : ~0u << (32 - nb));
        eq = eq && ((w[q] ^ pre[q]) & mask) == 0;
    }
    return eq;
}

// Pass p of the eviction's selection (at most kSelBlocks blocks of 256
// threads striding over the slots: fewer blocks redo the pick, and a pass
// after completion costs little more than its dispatch).
// State p (sel_state[4p .. 4p+3]): the key words of the digits chosen so far
// (the rest zero) and the rank still sought among the keys with that prefix;
// state 0 is (0, 0, 0, entries to evict), written by k_admit_ranks.  The
// selection is complete once the chosen bin holds exactly the keys still
// sought (at the latest when all twelve digits are chosen): the key bound is
// then the prefix with every later bit set, the pass evicts every stored key
// at most that bound and sets the done word, and the later passes return.
__global__ __launch_bounds__(256) void k_admit_select(const AdmitArgs a, int p) {
    if (a.hdr[kHdrEvict] == 0) return;
    if (p > 0 && a.sel_state[kSelDone] != 0) return;       // complete in an earlier pass
    __shared__ uint32_t h[256];
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t pick, pick_cnt;
    __shared__ int64_t need_s;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t s0 = (int64_t)blockIdx.x * 256 + t, stride = (int64_t)gridDim.x * 256;
    uint32_t pre[3] = {0u, 0u, 0u};
    if (p > 0) {
        // redo pass p-1's pick: the bin holding the sought rank
        const int64_t* st = a.sel_state + 4 * (p - 1);
        const int64_t need = st[3];
        const uint32_t c = a.sel_hist[(p - 1) * 256 + t];
        uint32_t inc = c;
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t u = __shfl_up(inc, d, 64);
            if (lane >= d) inc += u;
        }
        if (lane == 63) wsum[wv] = inc;
        if (t == 0) {                                      // (always overwritten below)
            pick = 0;
            pick_cnt = 0;
            need_s = need;
        }
        __syncthreads();
        uint32_t ex = inc - c;
        for (int k = 0; k < wv; ++k) ex += wsum[k];
        if ((int64_t)ex < need && need <= (int64_t)ex + c) {   // exactly one bin
            pick = (uint32_t)t;
            pick_cnt = c;
            need_s = need - ex;
        }
        __syncthreads();
        const int q = (p - 1) >> 2, sh = 24 - 8 * ((p - 1) & 3);
#pragma unroll
        for (int k = 0; k < 3; ++k) pre[k] = (uint32_t)st[k] | (k == q ? pick << sh : 0u);
        const bool complete = need_s == (int64_t)pick_cnt;
        if (complete) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {                  // every bit after digit p-1 set
                const int nb = min(max(8 * p - 32 * k, 0), 32);
                pre[k] |= nb == 32 ? 0u : (~0u >> nb);
            }
        }
        if (blockIdx.x == 0 && t == 0) {
            int64_t* nx = a.sel_state + 4 * p;
            nx[0] = pre[0];
            nx[1] = pre[1];
            nx[2] = pre[2];
            nx[3] = need_s;
            if (complete) a.sel_state[kSelDone] = 1;
        }
        if (complete) {
            for (int64_t s = s0; s < a.capacity; s += stride) {
                if (!holds_key(a.keys[s])) continue;
                uint32_t w[3];
                slot_key(a, s, w);
                const bool le =
                    w[0] != pre[0] ? w[0] < pre[0] : (w[1] != pre[1] ? w[1] < pre[1] : w[2] <= pre[2]);
                if (le) {
                    a.keys[s] = REC_TOMBSTONE_KEY;         // the digest stays: probes pass the slot
                    a.scores[s] = 0;
                }
            }
            return;
        }
    }
    h[t] = 0;
    __syncthreads();
    for (int64_t s = s0; s < a.capacity; s += stride) {
        uint32_t w[3];
        slot_key(a, s, w);
        if (key_prefix_eq(w, pre, p)) atomicAdd(&h[key_digit(w, p)], 1u);
    }
    __syncthreads();
    if (h[t]) atomicAdd(a.sel_hist + p * 256 + t, h[t]);
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
    for (int64_t seen_n = 0; seen_n < a.capacity && slot < 0; seen_n += kAdmitKeyWin) {
        int64_t w[kAdmitKeyWin];
        key_window(a.keys, at, a.capacity, w);
#pragma unroll
        for (int j = 0; j < kAdmitKeyWin; ++j) {
            if (slot >= 0 || seen_n + j >= a.capacity) continue;
            int64_t cur = w[j];
            if (cur == REC_EMPTY_KEY || cur == REC_TOMBSTONE_KEY) {
                int64_t sj = at + j;
                while (sj >= a.capacity) sj -= a.capacity;
                if (__hip_atomic_compare_exchange_strong(a.keys + sj, &cur, key, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                    slot = sj;
            }
        }
        at += kAdmitKeyWin;
        while (at >= a.capacity) at -= a.capacity;
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
    L.sel_hist = L.sel_state = 0;
    if (evict) {
        L.sel_hist = take(4 * 256 * (size_t)kSelPasses);
        L.sel_state = take(8 * ((size_t)kSelDone + 1));
    }
    L.bytes = o;
    return L;
}

hipError_t launch_hash_admit(AdmitArgs a, hipStream_t s) {
    const dim3 blk(256);
    const unsigned gn = (unsigned)((a.n + 255) / 256);
    hipLaunchKernelGGL(k_admit_clear, dim3((unsigned)a.nbs), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_count, dim3(gn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_classify, dim3(gn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_blocks, dim3((unsigned)a.nbn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_ranks, dim3((unsigned)a.nbn), blk, 0, s, a);
    if (a.mode != REC_SCORE_NONE) {
        const dim3 gc((unsigned)min((a.capacity + 255) / 256, (int64_t)kSelBlocks));
        for (int p = 0; p <= kSelPasses; ++p) hipLaunchKernelGGL(k_admit_select, gc, blk, 0, s, a, p);
    }
    hipLaunchKernelGGL(k_admit_insert, dim3(gn), blk, 0, s, a);
    hipLaunchKernelGGL(k_admit_lookup, dim3(gn), blk, 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
