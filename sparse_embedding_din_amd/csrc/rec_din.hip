// DIN target attention over packed (padding-free) click sequences.
//
// Pages: "MultiTowerDIN：当前现状分析" §4.1 (sequences padded to 100 while the
// real length is ~3-5: the main waste), §4.2 (attention input [q, s, q-s,
// q*s]; attn MLP with hidden units 256 and 64; a linear score; mask and
// softmax; weighted sum), §4.4 (query [B,48], output [B,48]).
//
// Work split.  rec_din_plan resolved every sequence id to its row, laid the
// batch out as P packed positions and cut [0, P) into groups: group g starts
// at the sample start nearest to g * span (span = P over the workgroups of a
// persistent grid, one 8-wave workgroup per CU (two waves per SIMD), unless
// the caller asks for a fixed range length), so no sample is cut between
// workgroups.  Workgroup k takes groups k, k + grid, ...; a group's
// 16-position tiles are split as evenly as possible over its eight waves, so
// every wave gets about the same number of rows whatever the length mix.  A
// wave walks its tiles one per round (built with four waves, kRoundTiles = 2:
// pairs while two are left), and per tile:
//   1. reads the positions' sample, step and three resolved rows from the
//      plan, then s (3 rows of 64 B) and q (3 x 16 floats of the pooled
//      output); lane (n, g) holds features 12g..12g+11 of position n;
//   2. forms its inputs in registers — never in memory;
//   3. runs the 192->256->64 MLP on the matrix cores with the weights as the
//      A operand (bf16: staged once per workgroup in LDS, 104 KiB) and the
//      positions as the B operand; the 256-wide layer is produced 32 units at
//      a time and fed straight into the 64-wide layer, because a 16x16
//      accumulator tile is already laid out as the next product's operand;
//   4. reduces the score across the four lane groups, then runs an online,
//      segmented softmax: DPP row shifts scan max and sums within each
//      sample's run of lanes, and one open sample carries its running max,
//      sum and weighted sum into the next tile.
// A sample cut between two waves of a workgroup leaves one unnormalised
// (max, sum, weighted sum) per piece in LDS; after a barrier the wave that
// holds the sample's first piece merges the pieces with the standard
// rescaling of partial softmax sums and writes the output.  Samples without
// positions (listed by the plan) are zeroed by the workgroups before their
// first group.
// The first layer's input is [q, s, q-s, q*s] with W1 = [W1q | W1s | W1d |
// W1m] (48 columns each).  Since W1d (q - s) = W1d q - W1d s, the bf16 path
// evaluates the same sum as (W1q + W1d) q + (W1s - W1d) s + W1m (q*s): 144
// inputs per position instead of 192, so a quarter fewer first-layer
// products and weight bytes.  The two column sums are formed in fp32 from the
// bf16 weights and rounded to bf16 once (rec_din_pack_mlp, or on chip for
// unpacked weights).  The fp32 path keeps the 192 inputs.
// Inside an MFMA the order of the K index is free as long as the A and B
// operands agree, so each lane's 36 inputs are laid out to match its own 12
// features, and the weights are permuted to the same order.
#include "rec_internal.h"
#include "rec_mfma.h"

namespace rec {
namespace {

struct Sub {
    float q[12];     // as loaded until masked (mask_sub)
    float s[12];
    int64_t pos;     // packed position
    int32_t b;
    int32_t j;       // step in the sample
    int32_t rem;     // steps left in the sample
    int32_t jl;      // steps of the sample before this one inside the range
    int32_t rl;      // steps of the sample after this one inside the range
    uint32_t keep;   // bit r: the 4 floats r of s are a real row (valid and not a miss)
    bool valid;
};

// v of lane n - D of the same 16-lane row (0 for n < D)
template <int D>
__device__ inline float dpp_row_shr(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x110 + D, 0xF, 0xF, true));
}

// Segmented inclusive scans inside 16-lane rows.  mk[i] is 1 where lane
// n - 2^i belongs to the same sample as lane n, else 0.
struct SegMask {
    float mk[4];
};

__device__ inline SegMask seg_mask(int n, int st) {
    SegMask m;
    m.mk[0] = n - 1 >= st ? 1.f : 0.f;
    m.mk[1] = n - 2 >= st ? 1.f : 0.f;
    m.mk[2] = n - 4 >= st ? 1.f : 0.f;
    m.mk[3] = n - 8 >= st ? 1.f : 0.f;
    return m;
}

__device__ inline float seg_max(float v, const SegMask& m) {
    float t;
    t = dpp_row_shr<1>(v); v = m.mk[0] != 0.f ? fmaxf(v, t) : v;
    t = dpp_row_shr<2>(v); v = m.mk[1] != 0.f ? fmaxf(v, t) : v;
    t = dpp_row_shr<4>(v); v = m.mk[2] != 0.f ? fmaxf(v, t) : v;
    t = dpp_row_shr<8>(v); v = m.mk[3] != 0.f ? fmaxf(v, t) : v;
    return v;
}

// N segmented sums at once, step-major: the N independent chains fill the
// wait a DPP read of a just-written register needs.
template <int D, int N>
__device__ inline void seg_step(float (&v)[N], float mk) {
    float t[N];
#pragma unroll
    for (int f = 0; f < N; ++f) t[f] = dpp_row_shr<D>(v[f]);
#pragma unroll
    for (int f = 0; f < N; ++f) v[f] = fmaf(t[f], mk, v[f]);
}

template <int N>
__device__ inline void seg_sums(float (&v)[N], const SegMask& m) {
    seg_step<1>(v, m.mk[0]);
    seg_step<2>(v, m.mk[1]);
    seg_step<4>(v, m.mk[2]);
    seg_step<8>(v, m.mk[3]);
}

// lane 15 of each 16-lane row, in every lane of the row (DPP row_newbcast)
__device__ inline float row_bcast15(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x15F, 0xF, 0xF, false));
}

// p + the value of the lane 16 (or 32) lanes away: the two halves returned by
// a permlane swap of p with itself are p's own rows and their partners
__device__ inline float add_xor16(float p) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float add_xor32(float p) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Gathering one tile for lane (n, g) takes two dependent rounds: its packed
// position's sample, step and the two resolved rows its features need
// (load_entries), then the three 16-byte pieces of s and of q (load_data).
// Loads are unconditional (a lane past the range's end re-reads its last
// position, a hash miss reads row 0) and masked afterwards.
struct Ent {
    int32_t b, jr, ra, rb;
};

// A lane's 12 features span two of the three sub-features (fa, fb); their
// table and query-column are selected once per wave from values pinned to
// scalar registers (readfirstlane), so the compiler cannot turn the per-lane
// choice into a load from the kernel arguments inside the loop.
struct LaneSrc {
    const float* va;
    const float* vb;
    int32_t qa, qb, fa, fb;
};

typedef const float __attribute__((address_space(1))) gfloat;

__device__ inline const float* uniform_ptr(const float* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    // back to a global-memory pointer, so its loads stay global (not flat)
    return (const float*)(gfloat*)(((uint64_t)hi << 32) | lo);
}

__device__ inline LaneSrc lane_src(const DinArgs& a, int lane) {
    const int g = lane >> 4;
    LaneSrc L;
    L.fa = (3 * g) >> 2;
    L.fb = (3 * g + 2) >> 2;
    const float* t0 = uniform_ptr(a.tab[0].values);
    const float* t1 = uniform_ptr(a.tab[1].values);
    const float* t2 = uniform_ptr(a.tab[2].values);
    const int q0 = __builtin_amdgcn_readfirstlane(a.qcol[0]);
    const int q1 = __builtin_amdgcn_readfirstlane(a.qcol[1]);
    const int q2 = __builtin_amdgcn_readfirstlane(a.qcol[2]);
    L.va = L.fa == 0 ? t0 : (L.fa == 1 ? t1 : t2);
    L.vb = L.fb == 0 ? t0 : (L.fb == 1 ? t1 : t2);
    L.qa = L.fa == 0 ? q0 : (L.fa == 1 ? q1 : q2);
    L.qb = L.fb == 0 ? q0 : (L.fb == 1 ? q1 : q2);
    return L;
}

__device__ inline void load_entries(const DinArgs& a, const LaneSrc& L, int base, int cnt, int idx,
                                    Ent& E) {
    const int64_t p = base + min(idx, cnt - 1);
    E.b = a.pos_b[p];
    E.jr = a.pos_jr[p];
    E.ra = a.pos_rows[L.fa * a.pmax + p];
    E.rb = a.pos_rows[L.fb * a.pmax + p];
}

__device__ inline void load_data(const DinArgs& a, const LaneSrc& L, const Ent& E, int base, int cnt,
                                 int idx, int lane, Sub& S) {
    const int g = lane >> 4;
    const int ic = min(idx, cnt - 1);
    S.valid = idx < cnt;
    S.pos = base + ic;
    S.b = E.b;
    S.j = E.jr & 0xffff;
    S.rem = E.jr >> 16;
    S.jl = min(S.j, ic);
    S.rl = min(S.rem, cnt - 1 - ic);
    const float* qrow = a.query + (int64_t)E.b * a.query_ld;
    S.keep = 0;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int c4 = 3 * g + r;
        const int w = c4 & 3;
        const bool first = (c4 >> 2) == L.fa;
        const int32_t rr = first ? E.ra : E.rb;
        gfloat* vb = (gfloat*)(first ? L.va : L.vb);
        const int qc = first ? L.qa : L.qb;
        S.keep |= (S.valid && rr >= 0) ? 1u << r : 0u;
        const f32x4 sv = *(const __attribute__((address_space(1))) f32x4*)(vb + (int64_t)(rr >= 0 ? rr : 0) * 16 + 4 * w);
        const float4 qv = *(const float4*)(qrow + qc + 4 * w);
        S.s[4 * r + 0] = sv[0];
        S.s[4 * r + 1] = sv[1];
        S.s[4 * r + 2] = sv[2];
        S.s[4 * r + 3] = sv[3];
        S.q[4 * r + 0] = qv.x;
        S.q[4 * r + 1] = qv.y;
        S.q[4 * r + 2] = qv.z;
        S.q[4 * r + 3] = qv.w;
    }
}

// Zero what load_data fetched for a lane past the range (q and s) or a hash
// miss (s).  Done just before the values are first used, not when the loads
// are issued, so the wait for them falls after the previous round's work.
__device__ inline void mask_sub(Sub& S) {
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const bool k = (S.keep >> r) & 1u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S.s[4 * r + i] = k ? S.s[4 * r + i] : 0.f;
            S.q[4 * r + i] = S.valid ? S.q[4 * r + i] : 0.f;
        }
    }
}

// Input i (0..47) of a lane: block tau = i / 12 of [q, s, q-s, q*s] at the
// lane's feature f = i % 12.  Column of W1: 48 tau + 12 g + f.
__device__ inline float x_in(const Sub& S, int i) {
    const int tau = i / 12, f = i % 12;
    return tau == 0 ? S.q[f] : (tau == 1 ? S.s[f] : (tau == 2 ? S.q[f] - S.s[f] : S.q[f] * S.s[f]));
}

// Input i (0..35) of a lane in the factored bf16 layer: block tau = i / 12 of
// [q, s, q*s] at the lane's feature f = i % 12.  Column of the factored
// weights: 48 tau + 12 g + f.
__device__ inline float x_in3(const Sub& S, int i) {
    const int tau = i / 12, f = i % 12;
    return tau == 0 ? S.q[f] : (tau == 1 ? S.s[f] : S.q[f] * S.s[f]);
}

// e = w3 . relu(h2) + b3 for a lane's 16 units of h2 (bias already in),
// summed over the four lane groups.
__device__ inline float score_from_h2(const f32x4 (&acc2)[4], const float* w3s, float b3, int g) {
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = mt * 16 + 4 * g + i;
            p += fmaxf(acc2[mt][i], 0.f) * w3s[u];
        }
    }
    p = add_xor16(p);
    p = add_xor32(p);
    return p + b3;
}


// The factored W1 image in LDS, per hidden block hb of 32 units (576
// 16-byte units): the full fragments (kb, rt) for K steps kb = 0..3 (inputs
// 8 kb .. 8 kb + 7 of each lane), 64 lanes x 16 B each, then the half
// fragments rt = 0, 1 (inputs 32..35), 64 lanes x 8 B each; W2 follows.
constexpr int kW1BlockU4 = 576;
constexpr int kW1U4 = 8 * kW1BlockU4;                 // 72 KiB
constexpr int kW2U4 = 8 * 4 * 64;                     // 32 KiB
constexpr int kWtU4 = kW1U4 + kW2U4;                  // 104 KiB
static_assert(kWtU4 * 16 == REC_DIN_PACKED_BYTES, "packed image size");

// One hidden block's first-layer fragments of a lane: full[kb * 2 + rt], half[rt].
struct W1Frag {
    uint4 full[8];
    uint2 half[2];
};

__device__ inline void load_w1(const uint4* w1p, int hb, int lane, W1Frag& f) {
    const uint4* b = w1p + hb * kW1BlockU4;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.full[i] = b[i * 64 + lane];
    const uint2* h = (const uint2*)(b + 512);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) f.half[rt] = h[rt * 64 + lane];
}

// Layer 1 for one hidden block: two 16-row tiles x NSUB position tiles, four
// K steps of 32 and one of 16, innermost in issue order so 2*NSUB independent
// accumulations are in flight.  The accumulators start from the block's bias
// (the first product's C operand), so no separate bias add is needed.
template <int NSUB>
__device__ inline void l1_block(const bf16x8 (&xf)[NSUB][4], const s16x4 (&xh)[NSUB], const W1Frag& w1,
                                const f32x4 bA, const f32x4 bB, f32x4 (&acc1)[NSUB][2]) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        acc1[s][0] = bA;
        acc1[s][1] = bB;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                acc1[s][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, w1.full[kb * 2 + rt]), xf[s][kb], acc1[s][rt], 0, 0, 0);
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            acc1[s][rt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(s16x4, w1.half[rt]), xh[s], acc1[s][rt], 0, 0, 0);
}

// The bf16 MLP for NSUB position tiles, software-pipelined over the eight
// hidden blocks: while block hb's layer-1 results go through ReLU and bf16
// into its layer-2 products, block hb+1's layer-1 products are already
// issued.  W1 fragments and b1 slices are read from LDS one block ahead of
// use (a b1 read at the block's start stalled its first product); a
// scheduling fence per block keeps the compiler from hoisting every block's
// reads (which would not fit in registers).  Layer-2 accumulators start from
// b2 the same way.
template <int NSUB>
__device__ inline void mlp_bf16(const Sub* S, const uint4* w1p, const uint4* w2p, const float* b1s,
                                const float* b2s, const float* w3s, float b3, int lane,
                                float* e) {
    const int g = lane >> 4;
    bf16x8 xf[NSUB][4];
    s16x4 xh[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
#pragma unroll
        for (int i = 0; i < 32; ++i) xf[s][i >> 3][i & 7] = (__bf16)x_in3(S[s], i);
        bf16x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = (__bf16)x_in3(S[s], 32 + i);
        xh[s] = __builtin_bit_cast(s16x4, t);
    }
    f32x4 acc2[NSUB][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const f32x4 b2v = *(const f32x4*)(b2s + mt * 16 + 4 * g);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) acc2[s][mt] = b2v;
    }
    W1Frag fw1[2];
    uint4 fw2[4];
    f32x4 fb1[2][2];                // each block's b1 slice, read with its W1 fragments
    f32x4 acc1[2][NSUB][2];
    load_w1(w1p, 0, lane, fw1[0]);
    fb1[0][0] = *(const f32x4*)(b1s + 4 * g);
    fb1[0][1] = *(const f32x4*)(b1s + 16 + 4 * g);
    l1_block<NSUB>(xf, xh, fw1[0], fb1[0][0], fb1[0][1], acc1[0]);
    fb1[1][0] = *(const f32x4*)(b1s + 32 + 4 * g);
    fb1[1][1] = *(const f32x4*)(b1s + 48 + 4 * g);
    load_w1(w1p, 1, lane, fw1[1]);
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
        __builtin_amdgcn_sched_barrier(0);
        const int cur = hb & 1, nxt = cur ^ 1;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fw2[mt] = w2p[(hb * 4 + mt) * 64 + lane];
        if (hb + 1 < 8) l1_block<NSUB>(xf, xh, fw1[nxt], fb1[nxt][0], fb1[nxt][1], acc1[nxt]);
        if (hb + 2 < 8) {
            // LDS reads complete in order: the b1 slice, needed first, goes first
            fb1[cur][0] = *(const f32x4*)(b1s + (hb + 2) * 32 + 4 * g);
            fb1[cur][1] = *(const f32x4*)(b1s + (hb + 2) * 32 + 16 + 4 * g);
            load_w1(w1p, hb + 2, lane, fw1[cur]);
        }
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            uint4 hp;
            hp.x = relu_pk_bf16(acc1[cur][s][0][0], acc1[cur][s][0][1]);
            hp.y = relu_pk_bf16(acc1[cur][s][0][2], acc1[cur][s][0][3]);
            hp.z = relu_pk_bf16(acc1[cur][s][1][0], acc1[cur][s][1][1]);
            hp.w = relu_pk_bf16(acc1[cur][s][1][2], acc1[cur][s][1][3]);
            const bf16x8 h = __builtin_bit_cast(bf16x8, hp);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc2[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, fw2[mt]), h, acc2[s][mt], 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) e[s] = score_from_h2(acc2[s], w3s, b3, g);
}

template <int NSUB>
__device__ inline void mlp_f32(const Sub* S, const float* __restrict__ w1,
                               const float* __restrict__ w2, const float* b1s, const float* b2s,
                               const float* w3s, float b3, int lane, float* e) {
    const int m = lane & 15, g = lane >> 4;
    float x[NSUB][48];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 48; ++i) x[s][i] = x_in(S[s], i);
    f32x4 acc2[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc2[s][mt] = *(const f32x4*)(b2s + mt * 16 + 4 * (lane >> 4));
    for (int hb = 0; hb < 8; ++hb) {
        f32x4 acc1[NSUB][2];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            acc1[s][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc1[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const float* r0 = w1 + (int64_t)(hb * 32 + m) * 192 + 12 * g;
        const float* r1 = r0 + 16 * 192;
#pragma unroll
        for (int i = 0; i < 48; ++i) {
            const int k = 48 * (i / 12) + (i % 12);
            const float a0 = r0[k], a1 = r1[k];
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                acc1[s][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, x[s][i], acc1[s][0], 0, 0, 0);
                acc1[s][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, x[s][i], acc1[s][1], 0, 0, 0);
            }
        }
        float h[NSUB][2][4];
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    h[s][rt][i] = fmaxf(acc1[s][rt][i] + b1s[hb * 32 + rt * 16 + 4 * g + i], 0.f);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const float* wr = w2 + (int64_t)(mt * 16 + m) * 256 + hb * 32 + 4 * g;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a2 = wr[rt * 16 + i];
#pragma unroll
                    for (int s = 0; s < NSUB; ++s)
                        acc2[s][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, h[s][rt][i], acc2[s][mt], 0, 0, 0);
                }
        }
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) e[s] = score_from_h2(acc2[s], w3s, b3, g);
}

// A group of T tiles gives wave w the tiles [group_tile_lo(T, w),
// group_tile_lo(T, w + 1)); group_wave_of is the wave holding tile t.
__device__ inline int group_tile_lo(int T, int w) { return (T * w) / kDinWaves; }
__device__ inline int group_wave_of(int T, int t) {
    int w = 0;
#pragma unroll
    for (int k = 1; k < kDinWaves; ++k) w += t >= group_tile_lo(T, k) ? 1 : 0;
    return w;
}

// Online segmented softmax and weighted sum for one 16-position tile of a
// wave's range.  A sample's run inside the range ends at the lane where
// rl == 0: a sample wholly inside the range writes its output there; one cut
// by the range's start (head) or end (tail) leaves its unnormalised state in
// the wave's LDS slot `pc` (head) or `pc + kPartialFloats` (tail); a tail
// piece also records its sample and the wave whose range holds the sample's
// last position (in a group starting at gA of T tiles), which is all the
// merge needs to find the other pieces.
__device__ inline void softmax_tile(const DinArgs& a, const Sub& S, float e, int lane, int64_t gA,
                                    int T, float* pc, float& m_open, float& l_open,
                                    float (&acc_open)[12]) {
    const int n = lane & 15, g = lane >> 4;
    const int j = S.valid ? S.jl : 0;
    const int rem = S.valid ? S.rl : 0;
    const int st = n - min(j, n);                 // first lane of this sample in the tile
    const int en = n + min(rem, 15 - n);          // last lane of this sample in the tile
    const bool cont = j > n;                      // sample began in an earlier tile
    const SegMask mk = seg_mask(n, st);
    const float ev = S.valid ? e : -INFINITY;
    if (a.scores && S.valid && g == 0) a.scores[S.pos] = e;
    const float mx = seg_max(ev, mk);
    const float mseg = __shfl(mx, (lane & 48) + en, 64);
    const float mref = cont ? fmaxf(mseg, m_open) : mseg;
    const float w = S.valid ? __expf(ev - mref) : 0.f;
    float v[13];
    v[12] = w;
#pragma unroll
    for (int f = 0; f < 12; ++f) v[f] = w * S.s[f];
    seg_sums(v, mk);
    float l = v[12];
    float A[12];
#pragma unroll
    for (int f = 0; f < 12; ++f) A[f] = v[f];
    if (cont) {
        const float sc = __expf(m_open - mref);
        l += l_open * sc;
#pragma unroll
        for (int f = 0; f < 12; ++f) A[f] += acc_open[f] * sc;
    }
    const bool end = S.valid && n == en && rem == 0;
    const bool whole = S.j == S.jl && S.rem == S.rl;
    if (end) {
        if (whole) {
            const float inv = __builtin_amdgcn_rcpf(l);
            float4* o = (float4*)(a.out + (int64_t)S.b * 48 + 12 * g);
#pragma unroll
            for (int q = 0; q < 3; ++q)
                o[q] = make_float4(A[4 * q] * inv, A[4 * q + 1] * inv, A[4 * q + 2] * inv, A[4 * q + 3] * inv);
        } else {
            const bool is_head = S.j > S.jl;
            float* ps = is_head ? pc : pc + kPartialFloats;
            if (g == 0)
                *(float4*)ps = make_float4(mref, l, __int_as_float(S.b),
                                           __int_as_float(group_wave_of(T, (int)((S.pos + S.rem - gA) >> 4))));
            float4* o = (float4*)(ps + 4 + 12 * g);
#pragma unroll
            for (int q = 0; q < 3; ++q) o[q] = make_float4(A[4 * q], A[4 * q + 1], A[4 * q + 2], A[4 * q + 3]);
        }
    }
    // the sample that runs past lane 15 (if any) carries its state onward;
    // max and sum are the same in every row, the weighted sums are per row
    const int open = __builtin_amdgcn_readlane((int)(S.valid && rem > 0), 15);
    if (open) {
        m_open = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mref), 15));
        l_open = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 15));
#pragma unroll
        for (int f = 0; f < 12; ++f) acc_open[f] = row_bcast15(A[f]);
    }
    if (a.weights) {
        __threadfence();
        uint64_t done = __ballot(g == 0 && end && whole);
        while (done) {
            const int src = __ffsll((unsigned long long)done) - 1;
            done &= done - 1;
            const float M = __shfl(mref, src, 64);
            const float Ls = __shfl(l, src, 64);
            const int64_t pl = __shfl(S.pos, src, 64);
            const int jl = __shfl(j, src, 64);
            const int64_t so = pl - jl;
            for (int jj = lane; jj <= jl; jj += 64)
                a.weights[so + jj] = __expf(a.scores[so + jj] - M) / Ls;
        }
    }
}

// The packed A-operand image, in 8-byte slots of 4 consecutive bf16 of one
// weight row: per hidden block hb, the factored W1's full fragments (kb, rt,
// lane, half) and half fragments (rt, lane), then W2's (hb, mt, lane, rt).
// Input i of lane g*16 + m (fragment kb = i / 8 for i < 32, the half
// fragment for i = 32..35) is factored column 48 tau + 12 g + f (tau = i / 12,
// f = i % 12); W2 fragment element 4 rt + i is hidden unit hb*32 + rt*16 +
// 4g + i.
constexpr int kW1Slots = 2 * kW1U4;               // 9216
constexpr int kW2Slots = 2 * kW2U4;               // 4096

__device__ inline float bf16_value(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Slot d < kW1Slots of the image: 4 factored first-layer weights, formed in
// fp32 from the bf16 W1 [256][192] and rounded to bf16 (q: W1q + W1d; s:
// W1s - W1d; q*s: W1m).
__device__ inline uint2 w1_slot(const uint16_t* __restrict__ w1, int d) {
    const int hb = d / (2 * kW1BlockU4), r = d % (2 * kW1BlockU4);
    int lane, rt, i0;
    if (r < 1024) {
        const int frag = r >> 7;
        lane = (r >> 1) & 63;
        rt = frag & 1;
        i0 = (frag >> 1) * 8 + (r & 1) * 4;
    } else {
        rt = (r - 1024) >> 6;
        lane = r & 63;
        i0 = 32;
    }
    const int row = hb * 32 + rt * 16 + (lane & 15);
    const int tau = i0 / 12, c = 12 * (lane >> 4) + i0 % 12;
    const uint16_t* w = w1 + row * 192;
    bf16x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float x;
        if (tau == 0) x = bf16_value(w[c + j]) + bf16_value(w[96 + c + j]);
        else if (tau == 1) x = bf16_value(w[48 + c + j]) - bf16_value(w[96 + c + j]);
        else x = bf16_value(w[144 + c + j]);
        v[j] = (__bf16)x;
    }
    return __builtin_bit_cast(uint2, v);
}

// Slot d < kW2Slots of the W2 part: W2 [64][256] values copied.
__device__ inline uint2 w2_slot(const uint16_t* __restrict__ w2, int d) {
    const int rt = d & 1, lane = (d >> 1) & 63, rest = d >> 7;
    const int mt = rest & 3, hb = rest >> 2;
    const int g = lane >> 4, m = lane & 15;
    return *(const uint2*)(w2 + (mt * 16 + m) * 256 + hb * 32 + rt * 16 + 4 * g);
}

__global__ __launch_bounds__(256) void k_din_pack(const uint16_t* __restrict__ w1,
                                                  const uint16_t* __restrict__ w2,
                                                  uint2* __restrict__ packed) {
    const int d = blockIdx.x * 256 + threadIdx.x;     // 8-byte slot
    if (d < kW1Slots) packed[d] = w1_slot(w1, d);
    else if (d < kW1Slots + kW2Slots) packed[d] = w2_slot(w2, d - kW1Slots);
}

// Positions per round of a wave: two 16-position tiles when a wave has its
// SIMD alone (each weight fragment read from LDS feeds two products), one
// when two waves share a SIMD (the other wave's products hide each read's
// latency, and the wave fits in half the registers).
constexpr int kRoundTiles = kDinWaves >= 8 ? 1 : 2;

template <int DT>
__global__ __launch_bounds__(64 * kDinWaves) void k_din_attn(const DinArgs a) {
    constexpr bool kPacked = DT == REC_BF16_PACKED;
    constexpr bool kBF = DT == REC_BF16 || kPacked;
    constexpr int kThreads = 64 * kDinWaves;
    __shared__ uint4 s_wt[kBF ? kWtU4 : 1];
    __shared__ float s_b1[256];
    __shared__ float s_b2[64];
    __shared__ float s_w3[64];
    uint4* s_w1 = s_wt;
    uint4* s_w2 = s_wt + kW1U4;

    __shared__ __attribute__((aligned(16))) float s_piece[kDinWaves * 2 * kPartialFloats];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Workgroup k takes the groups k, k + gridDim.x, ...: a group is the
    // positions between two sample starts about `span` apart, its tiles
    // split over the eight waves.  The group count (the plan computed it) and
    // the first group's bounds are read at once (every workgroup has a slot;
    // one past the last group is not used), ahead of the weight staging, so
    // they are scalar loads that the staging's vector loads do not delay.
    const int ng = a.plan_hdr[kHdrNGroups];
    int gi = blockIdx.x;
    int64_t gA = a.group_start[gi], gE = a.group_start[gi + 1];
    __builtin_amdgcn_sched_barrier(0);      // keep those loads ahead of the staging
    // Weight staging depends on nothing else and completes under the group
    // bookkeeping and the first gathers.
    if (kPacked) {
        // the packed image is the LDS image: copy it straight from memory into
        // LDS (global_load_lds, 1 KiB per wave instruction, no registers)
        const uint4* src = (const uint4*)a.w1;
        static_assert(kWtU4 % kThreads == 0, "whole wave copies");
#pragma unroll
        for (int i = 0; i < kWtU4 / kThreads; ++i) {
            const int c0 = (i * kDinWaves + wave) * 64;
            __builtin_amdgcn_global_load_lds((const void*)(src + c0 + lane),
                                             (__attribute__((address_space(3))) void*)(s_wt + c0), 16, 0, 0);
        }
    }
    float vb1 = 0.f, vb2 = 0.f, vw3 = 0.f;
    if (threadIdx.x < 256) vb1 = a.b1[threadIdx.x];
    if (threadIdx.x < 64) {
        vb2 = a.b2[threadIdx.x];
        vw3 = a.w3[threadIdx.x];
    }

    const int stride = gridDim.x * kDinWaves;
    const int n = lane & 15;
    const LaneSrc src = lane_src(a, lane);
    // this wave's range of a group [A, E): the group's 16-position tiles
    // split as evenly as they go, wave w taking tiles [tile_lo(w), tile_lo(w+1))
    auto wave_range = [&](int64_t A, int64_t E, bool live, int64_t& p0, int& cnt) {
        const int64_t N = live ? E - A : 0;
        const int T = (int)((N + 15) / 16);
        const int t0 = group_tile_lo(T, wave), t1 = group_tile_lo(T, wave + 1);
        p0 = A + 16 * (int64_t)t0;
        cnt = (int)(min((int64_t)16 * t1, N) - 16 * (int64_t)t0);
        if (cnt < 0) cnt = 0;
    };
    int64_t p0;
    int cnt;
    wave_range(gA, gE, gi < ng, p0, cnt);
    Sub S[kRoundTiles];
    bool ready = cnt > 0;           // S holds the first round of the wave's range
    if (ready) {
        Ent E[kRoundTiles];
#pragma unroll
        for (int s = 0; s < kRoundTiles; ++s) load_entries(a, src, p0, cnt, 16 * s + n, E[s]);
#pragma unroll
        for (int s = 0; s < kRoundTiles; ++s) load_data(a, src, E[s], p0, cnt, 16 * s + n, lane, S[s]);
    }

    if (kBF && !kPacked) {
        // plain bf16 weights: every thread forms its share of the image's slots
        uint2* d = (uint2*)s_wt;
        for (int i = threadIdx.x; i < kW1Slots; i += kThreads) d[i] = w1_slot((const uint16_t*)a.w1, i);
        for (int i = threadIdx.x; i < kW2Slots; i += kThreads)
            d[kW1Slots + i] = w2_slot((const uint16_t*)a.w2, i);
    }
    if (threadIdx.x < 256) s_b1[threadIdx.x] = vb1;
    if (threadIdx.x < 64) {
        s_b2[threadIdx.x] = vb2;
        s_w3[threadIdx.x] = vw3;
    }
    if (kPacked) __builtin_amdgcn_s_waitcnt(0);        // the LDS copies have landed
    __syncthreads();

    // samples without positions: zero output, spread over every wave
    {
        const int32_t ne = a.plan_hdr[kHdrNEmpty];
        for (int i = (blockIdx.x * kDinWaves + wave) * 64 + lane; i < ne; i += stride * 64) {
            float4* o = (float4*)(a.out + (int64_t)a.empty[i] * 48);
#pragma unroll
            for (int q = 0; q < 12; ++q) o[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    float* const pc = s_piece + wave * 2 * kPartialFloats;     // this wave's head, tail
    float acc_open[12];
    // Groups (uniform over the workgroup), then the wave's rounds of up to 32
    // positions.  While one round's MLP runs, the next round's entries are in
    // flight -- the next round of this range, else this wave's first round of
    // the next group -- and its s and q loads are issued before this round's
    // softmax.
    for (; gi < ng; gi += gridDim.x) {
        const int gn = gi + gridDim.x;
        int64_t nA = 0, nE = 0;
        if (gn < ng) {
            nA = a.group_start[gn];
            nE = a.group_start[gn + 1];
        }
        int64_t p0n;
        int cntn;
        wave_range(nA, nE, gn < ng, p0n, cntn);
        const int gT = (int)((gE - gA + 15) / 16);
        float m_open = -INFINITY, l_open = 0.f;
#pragma unroll
        for (int f = 0; f < 12; ++f) acc_open[f] = 0.f;
        if (lane == 0) pc[kPartialFloats + 2] = __int_as_float(-1);     // no tail piece yet
        if (cnt > 0 && !ready) {
            Ent E[kRoundTiles];
#pragma unroll
            for (int s = 0; s < kRoundTiles; ++s) load_entries(a, src, p0, cnt, 16 * s + n, E[s]);
#pragma unroll
            for (int s = 0; s < kRoundTiles; ++s) load_data(a, src, E[s], p0, cnt, 16 * s + n, lane, S[s]);
            // Wait here: the compiler's wait counting merges this path with
            // the round loop's back edge, and loads still pending here would
            // make it wait for every load in flight (the next round's
            // prefetches included) at the first use of these registers.
            __builtin_amdgcn_s_waitcnt(0);
        }
        for (int sb = 0; sb < cnt; sb += 16 * kRoundTiles) {
            int64_t q0 = p0;
            int qc = cnt, qs = sb + 16 * kRoundTiles;
            if (qs >= cnt) {
                q0 = p0n;
                qc = cntn;
                qs = 0;
            }
            const bool more = qs < qc;
            Ent E[kRoundTiles];
            if (more) {
#pragma unroll
                for (int s = 0; s < kRoundTiles; ++s) load_entries(a, src, q0, qc, qs + 16 * s + n, E[s]);
            }
            float e[kRoundTiles];
            const bool two = kRoundTiles == 2 && cnt - sb > 16;
#pragma unroll
            for (int s = 0; s < kRoundTiles; ++s) mask_sub(S[s]);
            if constexpr (kRoundTiles == 2) {
                if (kBF) {
                    if (two) mlp_bf16<2>(S, s_w1, s_w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                    else mlp_bf16<1>(S, s_w1, s_w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                } else {
                    if (two) mlp_f32<2>(S, (const float*)a.w1, (const float*)a.w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                    else mlp_f32<1>(S, (const float*)a.w1, (const float*)a.w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                }
            } else {
                if (kBF) mlp_bf16<1>(S, s_w1, s_w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                else mlp_f32<1>(S, (const float*)a.w1, (const float*)a.w2, s_b1, s_b2, s_w3, a.b3, lane, e);
            }
            Sub Sn[kRoundTiles];
            if (more) {
#pragma unroll
                for (int s = 0; s < kRoundTiles; ++s) load_data(a, src, E[s], q0, qc, qs + 16 * s + n, lane, Sn[s]);
            }
            softmax_tile(a, S[0], e[0], lane, gA, gT, pc, m_open, l_open, acc_open);
            if constexpr (kRoundTiles == 2) {
                if (two) softmax_tile(a, S[1], e[1], lane, gA, gT, pc, m_open, l_open, acc_open);
            }
#pragma unroll
            for (int s = 0; s < kRoundTiles; ++s) S[s] = Sn[s];
        }
        ready = cnt > 0 && cntn > 0;
        __syncthreads();
        // a sample cut between waves: its tail piece (waves 0-2) and the head
        // pieces of the waves up to the one where it ends; lane c < 48 owns
        // weighted sum c
        if (wave < kDinWaves - 1) {
            const float* tl = pc + kPartialFloats;
            const int b = __float_as_int(tl[2]);
            if (b >= 0) {
                const int w1 = __float_as_int(tl[3]);
                float m = tl[0], l = tl[1];
                float acc = lane < 48 ? tl[4 + lane] : 0.f;
                for (int h = wave + 1; h <= w1; ++h) {
                    if (group_tile_lo(gT, h) == group_tile_lo(gT, h + 1)) continue;   // no tiles
                    const float* hp = s_piece + h * 2 * kPartialFloats;
                    const float mn = fmaxf(m, hp[0]);
                    const float sa = __expf(m - mn), sh = __expf(hp[0] - mn);
                    l = l * sa + hp[1] * sh;
                    acc = acc * sa + (lane < 48 ? hp[4 + lane] : 0.f) * sh;
                    m = mn;
                }
                if (lane < 48) a.out[(int64_t)b * 48 + lane] = acc * __builtin_amdgcn_rcpf(l);
                if (a.weights) {
                    const int64_t ps = a.pos_start[b], pe = a.pos_start[b + 1];
                    for (int64_t q = ps + lane; q < pe; q += 64) a.weights[q] = __expf(a.scores[q] - m) / l;
                }
            }
        }
        __syncthreads();
        gA = nA;
        gE = nE;
        p0 = p0n;
        cnt = cntn;
    }
}

}  // namespace

int din_waves(int num_cus) { return num_cus * kDinWaves; }

hipError_t launch_din(const DinArgs& a, hipStream_t s) {
    // one workgroup per CU; the plan holds group bounds for up to
    // kMaxDinGroups workgroups (more groups are looped over)
    const dim3 grid((unsigned)din_groups(a.waves)), block(64 * kDinWaves);
    if (a.dtype == REC_BF16_PACKED)
        REC_LAUNCH(REC_TIME_DIN_ATTN, k_din_attn<REC_BF16_PACKED>, grid, block, 0, s, a);
    else if (a.dtype == REC_BF16)
        REC_LAUNCH(REC_TIME_DIN_ATTN, k_din_attn<REC_BF16>, grid, block, 0, s, a);
    else
        REC_LAUNCH(REC_TIME_DIN_ATTN, k_din_attn<REC_F32>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_din_pack(const void* w1, const void* w2, void* packed, hipStream_t s) {
    hipLaunchKernelGGL(k_din_pack, dim3((kW1Slots + kW2Slots) / 256), dim3(256), 0, s, (const uint16_t*)w1,
                       (const uint16_t*)w2, (uint2*)packed);
    return hipGetLastError();
}

}  // namespace rec
