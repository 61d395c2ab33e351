// Hash-table write side: insert-or-assign of (key, values) pairs and clearing.
//
// Pages: "MultiTowerDIN：集成 DynamicEmb" §6.4 (at start-up a service rebuilds
// each table by inserting its stored key/value pairs), §4.2 (score strategies
// STEP / LFU / NO_EVICTION), §1 (a slot: key, score, digest, 16 values).
//
// Three launches, one lane per pair in each:
//   1. claim: the lane walks the key's probe sequence (the table convention of
//      rec_internal.h: SplitMix64 mix, multiply-high home slot, linear
//      wrapping probes).  A slot holding the key is found; an empty slot is
//      claimed with a 64-bit compare-and-swap of its key, so two lanes never
//      take the same slot, and a lane that loses the swap to its own key (a
//      duplicate in the batch) has found it.  Keys only ever go from empty to
//      a key, so a stale read can only show a slot as empty; the swap then
//      fails and reports the key that is there (so the probe reads are plain
//      cached loads, eight slots per round trip).  The winner writes the
//      digest; scores are updated (STEP: every lane writes the same step;
//      LFU: one atomic add per pair).  With no empty slot on the whole
//      sequence the pair is not stored (no eviction).  The same launch
//      clears the workspace's winner words (one per slot).
//   2. winner: every pair that placed its key records its index in the
//      workspace's winner word of its slot with an atomic max, so each slot
//      ends with its last pair.
//   3. values: the pair whose index won copies its 16 values into the slot;
//      so a key given several times gets the values of its last occurrence,
//      as inserting the pairs one after another would leave them.
#include "rec_internal.h"

namespace rec {
namespace {

__global__ __launch_bounds__(256) void k_hash_insert(const HashInsArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < a.capacity) a.winner[i] = -1;
    if (i >= a.n) return;
    const int64_t key = a.in_keys[i];
    int64_t slot = -2;                        // the reserved markers are never stored
    if (key != REC_EMPTY_KEY && key != REC_TOMBSTONE_KEY) {
        const uint64_t h = mix64((uint64_t)key);
        int64_t at = hash_home(h, a.capacity);
        bool claimed = false, done = false;
        slot = -1;
        for (int64_t seen_n = 0; seen_n < a.capacity && !done; seen_n += kKeyWin) {
            int64_t w[kKeyWin];
            key_window(a.keys, at, a.capacity, w);
#pragma unroll
            for (int j = 0; j < kKeyWin; ++j) {
                if (done || seen_n + j >= a.capacity) continue;
                int64_t sj = at + j;
                while (sj >= a.capacity) sj -= a.capacity;
                if (w[j] == key) {
                    slot = sj;
                    done = true;
                } else if (w[j] == REC_EMPTY_KEY) {
                    int64_t seen = REC_EMPTY_KEY;
                    if (__hip_atomic_compare_exchange_strong(a.keys + sj, &seen, key, __ATOMIC_RELAXED,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                        slot = sj;
                        claimed = true;
                        done = true;
                    } else if (seen == key) {
                        slot = sj;
                        done = true;
                    }
                }
            }
            at += kKeyWin;
            while (at >= a.capacity) at -= a.capacity;
        }
        if (slot >= 0) {
            if (claimed) a.digests[slot] = (uint8_t)hash_digest(h);
            if (a.mode == REC_SCORE_STEP) a.scores[slot] = a.step;
            if (a.mode == REC_SCORE_LFU)
                __hip_atomic_fetch_add(a.scores + slot, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    a.pair_slot[i] = (int32_t)slot;
}

__global__ __launch_bounds__(256) void k_hash_insert_winner(const HashInsArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    const int32_t s = a.pair_slot[i];
    if (s >= 0) atomicMax(a.winner + s, (int32_t)i);
}

__global__ __launch_bounds__(256) void k_hash_insert_values(const HashInsArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    const int32_t s = a.pair_slot[i];
    if (a.slot_out) a.slot_out[i] = s;
    if (s < 0 || a.winner[s] != (int32_t)i) return;
    const float4* src = (const float4*)(a.in_values + i * 16);
    float4* dst = (float4*)(a.values + (int64_t)s * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r] = src[r];
}

__global__ __launch_bounds__(256) void k_hash_clear(int64_t* keys, uint8_t* digests, uint64_t* scores,
                                                    int64_t capacity) {
    for (int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x; s < capacity; s += (int64_t)gridDim.x * 256) {
        keys[s] = REC_EMPTY_KEY;
        digests[s] = 0;
        if (scores) scores[s] = 0;
    }
}

}  // namespace

hipError_t launch_hash_insert(const HashInsArgs& a, hipStream_t s) {
    const int64_t blocks = (a.n + 255) / 256;
    const int64_t blocks0 = (max(a.n, a.capacity) + 255) / 256;
    hipLaunchKernelGGL(k_hash_insert, dim3((unsigned)blocks0), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_hash_insert_winner, dim3((unsigned)blocks), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_hash_insert_values, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_hash_clear(int64_t* keys, uint8_t* digests, uint64_t* scores, int64_t capacity,
                             hipStream_t s) {
    const int64_t blocks = min((capacity + 255) / 256, (int64_t)4096);
    hipLaunchKernelGGL(k_hash_clear, dim3((unsigned)blocks), dim3(256), 0, s, keys, digests, scores, capacity);
    return hipGetLastError();
}

}  // namespace rec
