// Internal declarations shared by librec's translation units: table
// descriptors as the kernels see them, the index arithmetic (host and
// device), and the kernel launchers each .hip file provides.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rec.h"

namespace rec {

// Kernel timing (rec_time_next_launch): takes, and clears, the events this
// thread set for the next launch of kernel class `which`.
bool take_timing(int which, hipEvent_t* start, hipEvent_t* stop);

// A launch that records the caller's timing events, when set, at the
// kernel's own start and end (hipExtLaunchKernelGGL), else a plain launch.
#define REC_LAUNCH(which, kernel, grid, block, shmem, stream, ...)                              \
    do {                                                                                         \
        hipEvent_t ev0_, ev1_;                                                                   \
        if (take_timing(which, &ev0_, &ev1_))                                                    \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ev0_, ev1_, 0, __VA_ARGS__); \
        else                                                                                     \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                   \
    } while (0)

// ---------------------------------------------------------------------------
// A table as the kernels see it (48 bytes, passed in kernel arguments).
struct TabDev {
    const float* values;      // [rows][16]
    const int64_t* keys;      // hash: [rows]
    const uint8_t* digests;   // hash: [rows], 0 = empty slot
    int64_t rows;             // direct: num_buckets; hash: capacity
    uint64_t magic;           // direct: multiplier for the floor modulo (0 when rows == 1)
    int32_t shift;            // direct: post-shift of the multiply-high
    int32_t kind;             // REC_DIRECT / REC_HASH
};

__host__ __device__ inline uint64_t mulhi64(uint64_t a, uint64_t b) {
    return (uint64_t)(((unsigned __int128)a * (unsigned __int128)b) >> 64);
}

// Floor modulo by an invariant divisor n >= 2 through one multiply-high
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, Thm 4.2, specialised to 63-bit dividends):
// with l = ceil(log2 n) and m = ceil(2^(63+l) / n) (< 2^64), every
// v < 2^63 has floor(v / n) = mulhi(v, m) >> (l - 1).
inline void floor_mod_prepare(int64_t n, uint64_t* magic, int32_t* shift) {
    if (n <= 1) { *magic = 0; *shift = 0; return; }
    int l = 0;
    while (l < 63 && ((int64_t)1 << l) < n) ++l;           // 2^(l-1) < n <= 2^l
    unsigned __int128 num = (unsigned __int128)1 << (63 + l);
    *magic = (uint64_t)((num + (unsigned __int128)(n - 1)) / (unsigned __int128)n);
    *shift = l - 1;
}

// Row of raw id x in a table of n rows: x mod n in [0, n).  A negative x is
// handled through its one's complement v = -x - 1 (< 2^63): x mod n =
// n - 1 - (v mod n).
__host__ __device__ inline int64_t floor_mod_magic(int64_t x, int64_t n, uint64_t magic,
                                                   int32_t shift) {
    if (magic == 0) return 0;                                // n == 1
    const bool neg = x < 0;
    const uint64_t v = neg ? ~(uint64_t)x : (uint64_t)x;
    const uint64_t q = mulhi64(v, magic) >> shift;
    const int64_t r = (int64_t)(v - q * (uint64_t)n);
    return neg ? (n - 1 - r) : r;
}

// SplitMix64's output mixing function (Steele, Lea & Flood, OOPSLA 2014, with
// Stafford's Mix13 constants): a bijection on 64-bit words.
__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xbf58476d1ce4e5b9ULL;
    z ^= z >> 27;
    z *= 0x94d049bb133111ebULL;
    z ^= z >> 31;
    return z;
}

// Home slot: floor(h * capacity / 2^64) (Lemire's multiply-high range map).
__host__ __device__ inline int64_t hash_home(uint64_t h, int64_t capacity) {
    return (int64_t)mulhi64(h, (uint64_t)capacity);
}

__host__ __device__ inline uint32_t hash_digest(uint64_t h) {
    const uint32_t d = (uint32_t)(h & 0xffu);
    return d ? d : 1u;
}

// Linear probe from the home slot: the slot holding `key`, or -1 on reaching
// an empty slot (digest 0) or after `rows` probes.  Digests are read 32 at a
// time (two aligned 16-byte loads covering the probe position) and scanned in
// registers; a key is read only where the digest matches.  Near the end of
// the table, where 32 bytes would run past it, the window is read byte by
// byte with the probe's wrap-around.
__host__ __device__ inline int64_t hash_probe(const TabDev& t, int64_t key) {
    if (key == REC_TOMBSTONE_KEY) return -1;          // reserved: marks evicted slots
    const uint64_t h = mix64((uint64_t)key);
    const uint32_t d = hash_digest(h);
    const int64_t n = t.rows;
    int64_t s = hash_home(h, n);                 // next slot to examine
    int64_t left = n;                            // slots not yet examined
    while (left > 0) {
        const int64_t w = s & ~(int64_t)15;      // window [w, w + 32)
        uint32_t dw[8];
        if (w + 32 <= n) {
            const uint4 a = *(const uint4*)(t.digests + w);
            const uint4 b = *(const uint4*)(t.digests + w + 16);
            dw[0] = a.x; dw[1] = a.y; dw[2] = a.z; dw[3] = a.w;
            dw[4] = b.x; dw[5] = b.y; dw[6] = b.z; dw[7] = b.w;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t v = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    int64_t i = w + 4 * k + c;
                    if (i >= n) i -= n;              // w < n, so one wrap suffices
                    if (i >= n) i = 0;               // tables smaller than the window
                    v |= (uint32_t)t.digests[i] << (8 * c);
                }
                dw[k] = v;
            }
        }
        // masks over the window: empty slots, digest matches, and the
        // positions this window examines (from s, at most `left` of them)
        uint32_t E = 0, M = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t by = (dw[k] >> (8 * c)) & 0xffu;
                E |= (by == 0u ? 1u : 0u) << (4 * k + c);
                M |= (by == d ? 1u : 0u) << (4 * k + c);
            }
        const int lo = (int)(s - w);
        const int span = left < 32 - lo ? (int)left : 32 - lo;
        const uint32_t win = (span >= 32 ? 0xffffffffu : ((1u << span) - 1u)) << lo;
        E &= win;
        M &= win;
        // candidates: digest matches before the first empty slot, in order
        uint32_t cand = M & (E ? (E & (~E + 1u)) - 1u : 0xffffffffu);
        while (cand) {
            const int i = __builtin_ffs((int)cand) - 1;
            cand &= cand - 1u;
            int64_t slot = w + i;
            if (slot >= n) slot -= n;
            if (t.keys[slot] == key) return slot;
        }
        if (E) return -1;
        left -= span;
        s = w + 32;
        if (s >= n) s -= n;
        if (s >= n) s = 0;
    }
    return -1;
}

// The keys of slots at .. at + W - 1 in probe order (wrapping past the end),
// for the claiming probes of the write side: one round trip examines W slots
// (W / 2 16-byte loads) instead of one, which shortens the long probe chains
// of a well-filled table.  Plain loads: the caller's compare-and-swap settles
// any slot that changed since.  The rebuild's insert reads kKeyWin slots per
// round trip; admission, which claims slots in a full table, reads
// kAdmitKeyWin (wider windows slowed the rebuild: 313 -> 319 us at 16 slots,
// 341 us at 32, while admission went from 159 to 155 and 151 us).
constexpr int kKeyWin = 8;
constexpr int kAdmitKeyWin = 32;
typedef int64_t i64x2u __attribute__((ext_vector_type(2), aligned(8)));

template <int W>
__device__ inline void key_window(const int64_t* keys, int64_t at, int64_t cap, int64_t (&w)[W]) {
    static_assert(W % 2 == 0, "pairs of keys");
    if (at + W <= cap) {
#pragma unroll
        for (int q = 0; q < W / 2; ++q) {
            const i64x2u v = *(const i64x2u*)(keys + at + 2 * q);
            w[2 * q] = v.x;
            w[2 * q + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < W; ++j) {
            int64_t i = at + j;
            while (i >= cap) i -= cap;                  // tables smaller than the window wrap again
            w[j] = keys[i];
        }
    }
}

__device__ inline int64_t resolve_row(const TabDev& t, int64_t raw) {
    if (t.kind == REC_DIRECT) return floor_mod_magic(raw, t.rows, t.magic, t.shift);
    return hash_probe(t, raw);
}

// ---------------------------------------------------------------------------
// Scan / plan
constexpr int kScanThreads = 256;
constexpr int kScanItems = 4;
constexpr int kScanChunk = kScanThreads * kScanItems;     // 1024 lengths per block

__host__ __device__ inline int64_t scan_blocks(int64_t n) { return (n + kScanChunk - 1) / kScanChunk; }

// Sums of key-major KJT lengths [T][B] for the embedding bags to derive their
// own offsets, in three levels per table t: blocks of G*1024 samples (G chosen
// so that T * blocks <= 128), segments of 1024 samples, chunks of 32.
//   bs[t*nK + K]             block sums (flat: everything before block (t, K)
//                            is the sum of bs[0 .. t*nK + K))
//   segp[(t*nK + K)*G + g]   sum of the segments of the block before g
//   chp[((t*nK + K)*G + g)*32 + c]   sum of the chunks of the segment before c
// so a bag wave needs at most 4 strided loads per lane plus two values.
constexpr int kKjtChunk = 32;
constexpr int kKjtSegChunks = kScanChunk / kKjtChunk;      // 32 chunks per segment
struct KjtLayout {
    int64_t nK;            // blocks per table
    int64_t G;             // 1024-sample segments per block
    size_t off_segp, off_chp, bytes;   // bs at 0
};
__host__ __device__ inline KjtLayout kjt_layout(int32_t T, int64_t B) {
    KjtLayout k;
    const int64_t nseg = scan_blocks(B);                  // 1024-sample segments per table
    k.G = ((int64_t)T * nseg + 127) / 128;
    if (k.G < 1) k.G = 1;
    k.nK = (nseg + k.G - 1) / k.G;
    const size_t blocks = (size_t)T * (size_t)k.nK;
    k.off_segp = 8 * blocks;
    k.off_chp = k.off_segp + 8 * blocks * (size_t)k.G;
    k.bytes = k.off_chp + 8 * blocks * (size_t)k.G * kKjtSegChunks;
    return k;
}

// DIN plan buffer layout (bytes from the start).  Pmax = B * max_len bounds
// the packed positions P = sum_b min(len_b, max_len); packed position p of
// sample b, step j is pos_start[b] + j.  The attention splits [0, P) into
// groups, one at a time per workgroup: group g nominally starts at g * span
// (din_span: four requested ranges, else P over the workgroups) and really at
// the nearest sample start, so that no sample is cut between workgroups (a
// sample cut between two waves of one workgroup is merged in LDS).
//   [0, 64)        int32 header: B, max_len, R requested (0 = even split),
//                  groups ceil(P / span), P, nblocks, (unused), empty samples
//   sums           per 1024-sample block: int64 (clamped, raw) block sums, then
//                  64 pairs of 16-sample chunk sums (kPlanSumWords words)
//   pos_start      int32[B+1]
//   sample_base    int64[B]: index in seq_values of sample b's first position
//   pos_b          int32[Pmax]: sample of packed position p
//   pos_jr         int32[Pmax]: j | (L - 1 - j) << 16 (step, steps left)
//   pos_rows       int32[3][Pmax]: resolved row of the adgroup/cate/brand id
//                  (a hash miss is -1)
//   empty          int32[B]: the samples with no positions (header: count)
//   group_start    int32[ngroups]: group g's first position, the sample start
//                  nearest to g * span (the earlier one on a tie; P for group
//                  ceil(P / span)); entries past that one are not written
enum { kHdrB = 0, kHdrMaxLen, kHdrRReq, kHdrNGroups, kHdrP, kHdrNBlocks, kHdrUnused6,
       kHdrNEmpty };
constexpr int kPlanChunk = 16;                                  // samples per build block
constexpr int kPlanSumWords = 2 + 2 * (kScanChunk / kPlanChunk);   // 130
constexpr int kMinRange = 16;
constexpr int kMaxRange = 1 << 20;
constexpr int kPartialFloats = 52;       // a cut sample's piece: max, sum, 2 words, 48 sums
constexpr int kDinWaves = 8;             // waves per attention workgroup (two per SIMD)
constexpr int kMaxDinGroups = 4096;      // attention workgroups the plan provides for

struct PlanLayout {
    int64_t nblocks, pmax, ngroups;
    size_t off_sums, off_pos, off_sbase, off_pb, off_pjr, off_prows, off_empty, off_group, bytes;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline PlanLayout plan_layout(int64_t B, int32_t max_len) {
    PlanLayout p;
    p.nblocks = scan_blocks(B);
    p.pmax = B * (int64_t)max_len;
    // groups: ceil(P / 4R) + 1 at the smallest R, and at least one per
    // attention workgroup (each reads its first group's bounds before it
    // knows P)
    const int64_t ng = p.pmax / (kDinWaves * kMinRange) + 2;
    p.ngroups = ng > kMaxDinGroups + 1 ? ng : kMaxDinGroups + 1;
    p.off_sums = 64;
    p.off_pos = align16(p.off_sums + 8 * (size_t)kPlanSumWords * (size_t)p.nblocks);
    p.off_sbase = align16(p.off_pos + 4 * (size_t)(B + 1));
    p.off_pb = align16(p.off_sbase + 8 * (size_t)B);
    p.off_pjr = align16(p.off_pb + 4 * (size_t)p.pmax);
    p.off_prows = align16(p.off_pjr + 4 * (size_t)p.pmax);
    p.off_empty = align16(p.off_prows + 12 * (size_t)p.pmax);
    p.off_group = align16(p.off_empty + 4 * (size_t)B);
    p.bytes = align16(p.off_group + 4 * (size_t)p.ngroups);
    return p;
}

// Attention workgroups on a device with `waves` attention waves.
__host__ __device__ inline int64_t din_groups(int64_t waves) {
    const int64_t g = waves / kDinWaves;
    return g < 1 ? 1 : (g > kMaxDinGroups ? kMaxDinGroups : g);
}

// Nominal positions per group (before its ends move to sample starts): four
// requested ranges, else P spread over the attention's workgroups.
__host__ __device__ inline int64_t din_span(int64_t P, int32_t req, int64_t waves) {
    if (req > 0) return (int64_t)kDinWaves * req;
    const int64_t g = din_groups(waves);
    const int64_t s = (P + g - 1) / g;
    return s < 1 ? 1 : s;
}

// ---------------------------------------------------------------------------
// Launchers (return the hipError_t of the launch)
hipError_t launch_lengths_to_offsets(const int32_t* lengths, int64_t n, int64_t* offsets,
                                     hipStream_t s);
struct PlanArgs {
    TabDev tab[3];
    const int64_t* seq_values;
    int64_t seq_stride;
    const int64_t* seq_offsets;      // caller's layout, or NULL = packed
    const int32_t* seq_lengths;
    int64_t B;
    int32_t max_len;
    int32_t range_positions;   // stored in the header: 0 = even split
    int32_t waves;             // waves of the attention launch on this device
    int64_t* seq_offsets_out;
    int64_t* rows_out;
    void* plan;
};
hipError_t launch_din_plan(const PlanArgs& a, hipStream_t s);

// Tail slots the plan clears: every range the attention can form (the even
// split makes at most one per wave, a requested size ceil(pmax / size)).

struct EmbArgs {
    TabDev tab[REC_MAX_TABLES];
    const int64_t* values;
    const int32_t* lengths;
    const int64_t* offsets;       // given offsets, or NULL: derived from the KJT sums
    const int64_t* kjt_bs;        // KJT sums (kjt_layout) when offsets is NULL
    const int64_t* kjt_segp;
    const int64_t* kjt_chp;
    int64_t nK, G;
    int64_t* offsets_out;         // derived offsets [T*B+1], or NULL
    float* out;
    int64_t* rows_out;
    int64_t B;
    int32_t T;
};
hipError_t launch_embbag(const EmbArgs& a, hipStream_t s);
hipError_t launch_kjt_sums(const int32_t* lengths, int32_t T, int64_t B, void* sums, hipStream_t s);

struct HashArgs {
    TabDev tab;
    const int64_t* keys;
    int64_t n;
    int64_t* slot_out;
    float* rows_out;
};
hipError_t launch_hash_lookup(const HashArgs& a, hipStream_t s);

struct HashInsArgs {
    int64_t* keys;              // the table's arrays, written
    uint8_t* digests;
    uint64_t* scores;           // NULL unless mode != REC_SCORE_NONE
    float* values;
    int64_t capacity;
    const int64_t* in_keys;     // the pairs
    const float* in_values;
    int64_t n;
    int32_t mode;
    uint64_t step;
    int64_t* slot_out;
    int32_t* pair_slot;         // workspace: [n] slot of each pair (-1 not stored, -2 empty marker)
    int32_t* winner;            // workspace: [capacity] last pair index stored in each slot
};
hipError_t launch_hash_insert(const HashInsArgs& a, hipStream_t s);

// DLRM interaction: Z staged in LDS as 32 * ceil(F / 32) rows of dlrm_stride(d)
// floats, at most kDlrmMaxLdsFloats (144 KiB).
constexpr int kDlrmMaxLdsFloats = 36864;
int dlrm_stride(int d);
hipError_t launch_dlrm_interact(const float* z, int64_t B, int F, int d, float* out, int num_cus,
                                hipStream_t s);
// Frequency admission and eviction (rec_admit.hip).
struct AdmitArgs {
    TabDev tab;                   // the table for lookups
    int64_t* keys;                // the table's arrays, written
    uint8_t* digests;
    uint64_t* scores;             // NULL for REC_SCORE_NONE
    float* values;
    int64_t capacity, max_keys;
    int64_t* ckeys;               // the counter table
    uint64_t* ccounts;
    int64_t ccap;
    const int64_t* in_keys;       // the batch
    const float* init_values;
    int64_t n;
    uint64_t threshold;
    uint64_t step;
    int32_t mode;
    int64_t* slot_out;
    int64_t* counts_out;
    // workspace (admit_layout)
    int64_t* set_key;
    uint32_t* set_cnt;
    int32_t* set_first;
    int64_t nset;
    int32_t* flag;
    int32_t* rank;
    uint64_t* total;
    int64_t* cslot;
    int32_t* blk_cnt;
    int64_t nbn;
    int32_t* blk_stored;
    int64_t nbs;
    int64_t* hdr;
    uint32_t* sel_hist;           // eviction selection: counts per pass, and
    int64_t* sel_state;           // the chosen prefix and rank per pass (NULL for NO_EVICTION)
};
struct AdmitLayout {
    int64_t nset, nbn, nbs;
    size_t set_key, set_cnt, set_first, flag, rank, total, cslot, blk_cnt, blk_stored, hdr;
    size_t sel_hist, sel_state, bytes;
};
AdmitLayout admit_layout(int64_t n, int64_t capacity, bool evict);
hipError_t launch_hash_admit(AdmitArgs a, hipStream_t s);

// The DLRM forward around the interaction (rec_dlrm_fwd.hip).
constexpr int kDlrmMaxDense = 128;           // dense features
constexpr int kDlrmMaxZ = 1024;              // (S + 1) * d floats per sample
constexpr int kDlrmMaxPairs = 528;           // (S + 1)(S + 2) / 2 at S = 31
struct DlrmArgs {
    TabDev tab[32];
    int32_t mode[32];
    int64_t B;
    int32_t S, dim, n_dense;
    const float* dense;
    const int64_t* values;
    const int32_t* lengths;
    const int64_t* offsets;
    const float *wb1, *bb1, *wb2, *bb2, *wt1, *bt1, *wt2, *bt2, *wt3;
    float bt3;
    float* z;
    float* inter;
    float* logit;
    float* prob;
};
hipError_t launch_dlrm_fwd(const DlrmArgs& a, hipStream_t s);
// More than kDlrmMaxTablesFused tables or (S + 1) * d above kDlrmMaxZ: z and
// the interaction output through memory; tabs/modes hold all S tables.
constexpr int kDlrmMaxTablesFused = 31;
constexpr int kDlrmMaxTables = 255;
hipError_t launch_dlrm_fwd_wide(const DlrmArgs& a, const TabDev* tabs, const int32_t* modes, int num_cus,
                                hipStream_t s);
// Sparse backward + AdaGrad (rec_bwd.hip).  One table: its lookup
// descriptor (direct floor-mod constants or hash keys/digests), the arrays
// the step writes, and its first row in the flat row space of all tables.
struct BwdTab {
    TabDev tab;
    float* weights;
    float* accum;
    int64_t rows;
    uint32_t base;
    int32_t pad_;
};

struct BwdArgs {
    const int64_t* values;
    const int32_t* lengths;
    const int64_t* offsets;
    const float* grad_pooled;     // [B][T*16]
    const int64_t* seq_values;    // [3][seq_stride]
    const float* grad_seq;        // [3][P][16]
    int64_t seq_stride;
    int64_t B, nnz, P, n;         // n = nnz + 3P contributions
    int32_t T;
    int32_t seq_table[3];
    uint32_t total_rows;
    float lr, eps;
    uint32_t* keys_in;            // [n] flat row of each contribution
    uint32_t* src_in;             // [n] its gradient row
    const uint32_t* keys;         // sorted (set by the launcher)
    const uint32_t* src;
    float* hpart;                 // [chunks][16] head pieces
    float* tpart;                 // [chunks][16] tail pieces
};

int64_t bwd_sort_tiles(int64_t n);            // tiles of the radix sort (256 counters each)
// Stable LSD radix sort of n (key, value) pairs over the low key_bits bits
// of the keys, 8 bits per pass, ping-ponging between the two buffer pairs;
// hist needs bwd_sort_tiles(n) * 256 words, tot 256.  Returns the
// pair of buffers holding the result.
hipError_t launch_radix_sort(uint32_t* kin, uint32_t* vin, uint32_t* kout, uint32_t* vout, int64_t n,
                             int key_bits, uint32_t* hist, uint32_t* tot,
                             hipStream_t s, const uint32_t** keys_sorted, const uint32_t** vals_sorted);
hipError_t launch_embbag_adagrad(BwdArgs a, const BwdTab* tabs, uint32_t* keys_out, uint32_t* src_out,
                                 uint32_t* sort_hist, uint32_t* sort_tot, int key_bits, hipStream_t s);

// DIN attention backward (rec_din_bwd.hip).
struct DinBwdArgs {
    TabDev tabs[3];
    const int64_t* seq_values;
    int64_t seq_stride;
    const int64_t* seq_offsets;
    const int32_t* seq_lengths;
    int32_t max_len;
    int32_t bf16;                 // w1/w2 are bf16 bit patterns
    int64_t B;
    const float* query;
    int64_t query_ld;
    int32_t qcol[3];
    float b3;
    const void* w1;
    const float* b1;              // may be NULL (zero)
    const void* w2;
    const float* b2;              // may be NULL (zero)
    const float* w3;
    const float* gatt;            // [B][48]
    float* gq;                    // [B][48]
    float* gs;                    // [3][seq_stride][16] or NULL
    float* w1t;                   // [192][256] fp32 workspace
    float* w2t;                   // [256][64] fp32 workspace
    // per position index (workspace): its sample (-1: no position), the
    // sequence row, [x, 1], [h1, 1], [h2, 1], the score, the softmax weight,
    // de, dz1, dz2 and the query-gradient terms
    int32_t* map;
    float *S, *X, *H1, *H2, *E, *PW, *DE, *DZ1, *DZ2, *GQP;
    int32_t wgrad;                // weight gradients requested
    float* part;                  // [splits][part_stride]
    int64_t part_stride;
    float *dw1, *db1, *dw2, *db2, *dw3, *db3;
};

int64_t din_bwd_part_stride();
int din_bwd_splits();
hipError_t launch_din_bwd(const DinBwdArgs& a, hipStream_t s);

hipError_t launch_hash_clear(int64_t* keys, uint8_t* digests, uint64_t* scores, int64_t capacity,
                             hipStream_t s);

struct DinArgs {
    TabDev tab[3];
    const float* query;
    int64_t query_ld;
    int32_t qcol[3];
    int32_t max_len;
    const void* w1;
    const float* b1;
    const void* w2;
    const float* b2;
    const float* w3;
    float b3;
    int32_t dtype;
    const int32_t* plan_hdr;
    const int32_t* pos_start;
    const int32_t* pos_b;
    const int32_t* pos_jr;
    const int32_t* pos_rows;
    const int32_t* group_start;
    int64_t ngroups;
    const int32_t* empty;
    int64_t pmax;
    float* out;
    float* scores;
    float* weights;
    int64_t B;
    int32_t waves;          // waves of the attention launch (sets the even split)
};
int din_waves(int num_cus);
// The whole forward's first two launches: KJT and plan sums together, then the
// plan's build pass and the embedding bags together (rec_fwd.hip).
hipError_t launch_fwd_front(const PlanArgs& p, const EmbArgs& e, hipStream_t s);
hipError_t launch_din(const DinArgs& a, hipStream_t s);
hipError_t launch_din_pack(const void* w1, const void* w2, void* packed, hipStream_t s);

// Deep tower + final MLP (rec_tower.hip).  Layers 0-2 are the deep tower
// 256 -> 512 -> 256 -> 128, layer 3 the final hidden layer 176 -> 64; wo/bo
// the 64 -> 1 logit.
struct TowerArgs {
    const void* w[4];
    const float* b[4];
    const float* wo;
    float bo;
    int32_t dtype;
    const float* pooled;
    int64_t pooled_ld;
    const float* att;
    float* deep_out;
    float* logit;
    float* prob;
    int64_t B;
};
constexpr int kTowerSamples = 32;            // samples per workgroup
hipError_t launch_towers(const TowerArgs& a, hipStream_t s);
hipError_t launch_tower_pack(const void* const w[4], void* packed, hipStream_t s);

}  // namespace rec
