// DIN target attention over packed (padding-free) click sequences.
//
// Pages: "MultiTowerDIN：当前现状分析" §4.1 (sequences padded to 100 while the
// real length is ~3-5: the main waste), §4.2 (attention input [q, s, q-s,
// q*s]; attn MLP with hidden units 256 and 64; a linear score; mask and
// softmax; weighted sum), §4.4 (query [B,48], output [B,48]).
//
// Work split.  rec_din_plan cut the batch into tasks: runs of whole samples of
// about C packed positions.  A persistent grid (one 8-wave workgroup per CU)
// hands tasks to waves round-robin.  A wave walks its task's positions in
// tiles of 16 (pairs when two are left), and per tile:
//   1. gathers s (3 rows of 64 B) and q (3 x 16 floats from the pooled
//      output) for 16 positions; lane (n, g) holds features 12g..12g+11 of
//      position n, so each position's 192 B come in as 4 x 48 B;
//   2. forms the 192 inputs [q, s, q-s, q*s] in registers (bf16 or fp32) —
//      never written to memory;
//   3. runs the 192->256->64 MLP on the matrix cores with the weights as the
//      A operand (bf16: both layers staged once per workgroup in LDS, 128 KiB)
//      and positions as the B operand; the 256-wide layer is produced 32 units
//      at a time and fed straight into the 64-wide layer, because a 16x16
//      accumulator tile is already laid out as the next product's operand;
//   4. reduces the score across the four lane groups, then runs an online,
//      segmented softmax: DPP row shifts scan max and sums within each
//      sample's run of lanes, and one open sample carries its running max,
//      sum and weighted sum into the next tile.
// Inside an MFMA the order of the K index is free as long as the A and B
// operands agree, so each lane's 48 inputs are laid out to match its own 12
// features, and the weights are permuted to the same order while staging.
#include "rec_internal.h"

namespace rec {
namespace {

#ifndef REC_MLP_SCHED
#define REC_MLP_SCHED 1
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSmap = kMaxTaskPositions + REC_MAX_SEQ_LEN;   // position slots per wave

struct PosEnt {
    int64_t gidx;   // seq_offsets[b] + j: index of the position in seq_values
    int32_t b;      // sample
    int32_t jr;     // j | (L - 1 - j) << 16
};

struct Sub {
    float q[12];
    float s[12];
    int64_t gidx;
    int32_t b;
    int32_t j;
    int32_t rem;
    bool valid;
};

__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__device__ inline float dpp_row_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + D, 0xF, 0xF, false));
}

// Inclusive scans inside 16-lane rows, restarted at each lane's segment start.
__device__ inline float seg_max(float v, int n, int st) {
    float t;
    t = dpp_row_shr<1>(v); if (n - 1 >= st) v = fmaxf(v, t);
    t = dpp_row_shr<2>(v); if (n - 2 >= st) v = fmaxf(v, t);
    t = dpp_row_shr<4>(v); if (n - 4 >= st) v = fmaxf(v, t);
    t = dpp_row_shr<8>(v); if (n - 8 >= st) v = fmaxf(v, t);
    return v;
}

__device__ inline float seg_sum(float v, int n, int st) {
    float t;
    t = dpp_row_shr<1>(v); if (n - 1 >= st) v += t;
    t = dpp_row_shr<2>(v); if (n - 2 >= st) v += t;
    t = dpp_row_shr<4>(v); if (n - 4 >= st) v += t;
    t = dpp_row_shr<8>(v); if (n - 8 >= st) v += t;
    return v;
}

// Gather q and s for the position idx of lane (n, g); g picks features
// 12g..12g+11, i.e. the 16-byte chunks 3g..3g+2 of the 48-float vector.
// Every load is unconditional (positions past the task's end re-read its
// last position, a hash miss reads slot 0) and masked afterwards, so a lane
// keeps its id load, then its six 16-byte loads, in flight together.
template <bool kHash>
__device__ inline void gather(const DinArgs& a, const PosEnt* pt, int idx, int Ptask, int lane,
                              Sub& S) {
    const int n = lane & 15, g = lane >> 4;
    S.valid = idx < Ptask;
    const PosEnt pe = pt[min(idx, Ptask - 1)];
    S.gidx = pe.gidx;
    S.b = pe.b;
    S.j = pe.jr & 0xffff;
    S.rem = pe.jr >> 16;
    // lanes of group f < 3 resolve sub-feature f's id of position n (group 3
    // repeats group 2's work)
    const int f = g < 3 ? g : 2;
    const int64_t raw = a.seq_values[(int64_t)f * a.seq_stride + pe.gidx];
    int64_t row;
    if (kHash) {
        row = resolve_row(f == 0 ? a.tab[0] : (f == 1 ? a.tab[1] : a.tab[2]), raw);
    } else {
        const int64_t rows = f == 0 ? a.tab[0].rows : (f == 1 ? a.tab[1].rows : a.tab[2].rows);
        const uint64_t magic = f == 0 ? a.tab[0].magic : (f == 1 ? a.tab[1].magic : a.tab[2].magic);
        const int32_t shift = f == 0 ? a.tab[0].shift : (f == 1 ? a.tab[1].shift : a.tab[2].shift);
        row = floor_mod_magic(raw, rows, magic, shift);
    }
    if (a.rows_out && S.valid && g < 3) a.rows_out[(int64_t)g * a.seq_stride + pe.gidx] = row;
    const int fa = (3 * g) >> 2, fb = (3 * g + 2) >> 2;
    const int64_t rowA = __shfl(row, fa * 16 + n, 64);
    const int64_t rowB = __shfl(row, fb * 16 + n, 64);
    const float* qrow = a.query + (int64_t)pe.b * a.query_ld;
    float4 sv[3], qv[3];
    bool keep[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int c4 = 3 * g + r;
        const int ff = c4 >> 2, w = c4 & 3;
        const int64_t rr = (ff == fa) ? rowA : rowB;
        const float* vb = ff == 0 ? a.tab[0].values : (ff == 1 ? a.tab[1].values : a.tab[2].values);
        const int qc = ff == 0 ? a.qcol[0] : (ff == 1 ? a.qcol[1] : a.qcol[2]);
        keep[r] = S.valid && rr >= 0;
        sv[r] = *(const float4*)(vb + (rr >= 0 ? rr : 0) * 16 + 4 * w);
        qv[r] = *(const float4*)(qrow + qc + 4 * w);
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        S.s[4 * r + 0] = keep[r] ? sv[r].x : 0.f;
        S.s[4 * r + 1] = keep[r] ? sv[r].y : 0.f;
        S.s[4 * r + 2] = keep[r] ? sv[r].z : 0.f;
        S.s[4 * r + 3] = keep[r] ? sv[r].w : 0.f;
        S.q[4 * r + 0] = S.valid ? qv[r].x : 0.f;
        S.q[4 * r + 1] = S.valid ? qv[r].y : 0.f;
        S.q[4 * r + 2] = S.valid ? qv[r].z : 0.f;
        S.q[4 * r + 3] = S.valid ? qv[r].w : 0.f;
    }
}

// Input i (0..47) of a lane: block tau = i / 12 of [q, s, q-s, q*s] at the
// lane's feature f = i % 12.  Column of W1: 48 tau + 12 g + f.
__device__ inline float x_in(const Sub& S, int i) {
    const int tau = i / 12, f = i % 12;
    return tau == 0 ? S.q[f] : (tau == 1 ? S.s[f] : (tau == 2 ? S.q[f] - S.s[f] : S.q[f] * S.s[f]));
}

__device__ inline float score_from_h2(const f32x4 (&acc2)[4], const float* b2s, const float* w3s,
                                      float b3, int g) {
    float p = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = mt * 16 + 4 * g + i;
            p += fmaxf(acc2[mt][i] + b2s[u], 0.f) * w3s[u];
        }
    }
    p += __shfl_xor(p, 16, 64);
    p += __shfl_xor(p, 32, 64);
    return p + b3;
}

// A fragments of one hidden block hb: 12 of W1 (6 k-blocks x 2 row tiles)
// and 4 of W2, read from LDS in one batch so their latency is paid once per
// block; the next block's batch is issued before this block's products.
struct Frags {
    uint4 w1[12];
    uint4 w2[4];
};

__device__ inline void load_frags(Frags& f, const uint4* w1p, const uint4* w2p, int hb, int lane) {
#pragma unroll
    for (int i = 0; i < 12; ++i) f.w1[i] = w1p[(hb * 12 + i) * 64 + lane];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) f.w2[mt] = w2p[(hb * 4 + mt) * 64 + lane];
}

template <int NSUB>
__device__ inline void mlp_bf16_pipe(const Sub* S, const uint4* w1p, const uint4* w2p,
                                     const float* b1s, const float* b2s, const float* w3s,
                                     float b3, int lane, float* e);

template <int NSUB>
__device__ inline void mlp_bf16(const Sub* S, const uint4* w1p, const uint4* w2p, const float* b1s,
                                const float* b2s, const float* w3s, float b3, int lane,
                                float* e) {
    if (REC_MLP_SCHED >= 4) {
        mlp_bf16_pipe<NSUB>(S, w1p, w2p, b1s, b2s, w3s, b3, lane, e);
        return;
    }
    const int g = lane >> 4;
    bf16x8 xf[NSUB][6];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 48; ++i) xf[s][i >> 3][i & 7] = (__bf16)x_in(S[s], i);
    f32x4 acc2[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc2[s][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frags fr[2];
    load_frags(fr[0], w1p, w2p, 0, lane);
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
        const Frags& cur = fr[hb & 1];
        if (hb + 1 < 8) load_frags(fr[(hb + 1) & 1], w1p, w2p, hb + 1, lane);
#if REC_MLP_SCHED == 1
        // keep the next block's reads ahead of this block's products
        __builtin_amdgcn_sched_barrier(0);
#elif REC_MLP_SCHED == 2
        __builtin_amdgcn_iglp_opt(0);
#elif REC_MLP_SCHED == 3
        __builtin_amdgcn_iglp_opt(1);
#endif
        f32x4 acc1[NSUB][2];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            acc1[s][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc1[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < 6; ++kb) {
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, cur.w1[kb * 2 + 0]);
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, cur.w1[kb * 2 + 1]);
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                acc1[s][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xf[s][kb], acc1[s][0], 0, 0, 0);
                acc1[s][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xf[s][kb], acc1[s][1], 0, 0, 0);
            }
        }
        const float4 bA = *(const float4*)(b1s + hb * 32 + 4 * g);
        const float4 bB = *(const float4*)(b1s + hb * 32 + 16 + 4 * g);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            bf16x8 h;
            h[0] = (__bf16)fmaxf(acc1[s][0][0] + bA.x, 0.f);
            h[1] = (__bf16)fmaxf(acc1[s][0][1] + bA.y, 0.f);
            h[2] = (__bf16)fmaxf(acc1[s][0][2] + bA.z, 0.f);
            h[3] = (__bf16)fmaxf(acc1[s][0][3] + bA.w, 0.f);
            h[4] = (__bf16)fmaxf(acc1[s][1][0] + bB.x, 0.f);
            h[5] = (__bf16)fmaxf(acc1[s][1][1] + bB.y, 0.f);
            h[6] = (__bf16)fmaxf(acc1[s][1][2] + bB.z, 0.f);
            h[7] = (__bf16)fmaxf(acc1[s][1][3] + bB.w, 0.f);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc2[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, cur.w2[mt]), h, acc2[s][mt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) e[s] = score_from_h2(acc2[s], b2s, w3s, b3, g);
}

// Software-pipelined variant: the 256-wide layer's products for block hb+1
// are issued before the bias/ReLU/bf16 epilogue of block hb, so the vector
// ALU work of one block runs under the matrix-core work of the next.
template <int NSUB>
__device__ inline void mlp_bf16_pipe(const Sub* S, const uint4* w1p, const uint4* w2p,
                                     const float* b1s, const float* b2s, const float* w3s,
                                     float b3, int lane, float* e) {
    const int g = lane >> 4;
    bf16x8 xf[NSUB][6];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 48; ++i) xf[s][i >> 3][i & 7] = (__bf16)x_in(S[s], i);
    f32x4 acc2[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc2[s][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 f1[2][12], f2[2][4];
    f32x4 acc1[2][NSUB][2];
#pragma unroll
    for (int i = 0; i < 12; ++i) f1[0][i] = w1p[i * 64 + lane];
#pragma unroll
    for (int i = 0; i < 12; ++i) f1[1][i] = w1p[(12 + i) * 64 + lane];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) f2[0][mt] = w2p[mt * 64 + lane];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        acc1[0][s][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[0][s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < 6; ++kb)
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            acc1[0][s][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f1[0][2 * kb]), xf[s][kb], acc1[0][s][0], 0, 0, 0);
            acc1[0][s][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f1[0][2 * kb + 1]), xf[s][kb], acc1[0][s][1], 0, 0, 0);
        }
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
        const int c = hb & 1, nx = (hb + 1) & 1;
        // reads one block ahead: W1 of hb+2 (into the buffer hb just freed), W2 of hb+1
        if (hb + 2 < 8) {
#pragma unroll
            for (int i = 0; i < 12; ++i) f1[c][i] = w1p[((hb + 2) * 12 + i) * 64 + lane];
        }
        if (hb + 1 < 8) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) f2[nx][mt] = w2p[((hb + 1) * 4 + mt) * 64 + lane];
        }
        if (hb + 1 < 8) {
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                acc1[nx][s][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc1[nx][s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kb = 0; kb < 6; ++kb)
#pragma unroll
                for (int s = 0; s < NSUB; ++s) {
                    acc1[nx][s][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f1[nx][2 * kb]), xf[s][kb], acc1[nx][s][0], 0, 0, 0);
                    acc1[nx][s][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f1[nx][2 * kb + 1]), xf[s][kb], acc1[nx][s][1], 0, 0, 0);
                }
        }
        const float4 bA = *(const float4*)(b1s + hb * 32 + 4 * g);
        const float4 bB = *(const float4*)(b1s + hb * 32 + 16 + 4 * g);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            bf16x8 h;
            h[0] = (__bf16)fmaxf(acc1[c][s][0][0] + bA.x, 0.f);
            h[1] = (__bf16)fmaxf(acc1[c][s][0][1] + bA.y, 0.f);
            h[2] = (__bf16)fmaxf(acc1[c][s][0][2] + bA.z, 0.f);
            h[3] = (__bf16)fmaxf(acc1[c][s][0][3] + bA.w, 0.f);
            h[4] = (__bf16)fmaxf(acc1[c][s][1][0] + bB.x, 0.f);
            h[5] = (__bf16)fmaxf(acc1[c][s][1][1] + bB.y, 0.f);
            h[6] = (__bf16)fmaxf(acc1[c][s][1][2] + bB.z, 0.f);
            h[7] = (__bf16)fmaxf(acc1[c][s][1][3] + bB.w, 0.f);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc2[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f2[c][mt]), h, acc2[s][mt], 0, 0, 0);
        }
#if REC_MLP_SCHED == 5
        __builtin_amdgcn_iglp_opt(1);
#elif REC_MLP_SCHED >= 6
        // order this block: its LDS reads, then the next block's 256-wide
        // products each followed by a few epilogue ALU ops, then the 64-wide
        // products
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int k = 0; k < (hb + 1 < 8 ? 12 * NSUB : 0); ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, REC_MLP_SCHED == 6 ? 3 : 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * NSUB, 0);
        __builtin_amdgcn_sched_barrier(0);
#endif
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s) e[s] = score_from_h2(acc2[s], b2s, w3s, b3, g);
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
        for (int mt = 0; mt < 4; ++mt) acc2[s][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    for (int s = 0; s < NSUB; ++s) e[s] = score_from_h2(acc2[s], b2s, w3s, b3, g);
}

// Online segmented softmax and weighted sum for one 16-position tile.
__device__ inline void softmax_tile(const DinArgs& a, const Sub& S, float e, int lane,
                                    float& m_open, float& l_open, float (&acc_open)[12]) {
    const int n = lane & 15, g = lane >> 4;
    const int j = S.valid ? S.j : 0;
    const int rem = S.valid ? S.rem : 0;
    const int st = n - min(j, n);                 // first lane of this sample in the tile
    const int en = n + min(rem, 15 - n);          // last lane of this sample in the tile
    const bool cont = j > n;                      // sample began in an earlier tile
    const float ev = S.valid ? e : -INFINITY;
    if (a.scores && S.valid && g == 0) a.scores[S.gidx] = e;
    const float mx = seg_max(ev, n, st);
    const float mseg = __shfl(mx, (lane & 48) + en, 64);
    const float mref = cont ? fmaxf(mseg, m_open) : mseg;
    const float w = S.valid ? __expf(ev - mref) : 0.f;
    float l = seg_sum(w, n, st);
    float A[12];
#pragma unroll
    for (int f = 0; f < 12; ++f) A[f] = seg_sum(w * S.s[f], n, st);
    if (cont) {
        const float sc = __expf(m_open - mref);
        l += l_open * sc;
#pragma unroll
        for (int f = 0; f < 12; ++f) A[f] += acc_open[f] * sc;
    }
    const bool fin = S.valid && n == en && rem == 0;
    if (fin) {
        float4* o = (float4*)(a.out + (int64_t)S.b * 48 + 12 * g);
#pragma unroll
        for (int r = 0; r < 3; ++r)
            o[r] = make_float4(A[4 * r] / l, A[4 * r + 1] / l, A[4 * r + 2] / l, A[4 * r + 3] / l);
    }
    // the sample that runs past lane 15 (if any) carries its state onward
    const int last = (lane & 48) + 15;
    m_open = __shfl(mref, last, 64);
    l_open = __shfl(l, last, 64);
#pragma unroll
    for (int f = 0; f < 12; ++f) acc_open[f] = __shfl(A[f], last, 64);
    if (a.weights) {
        __threadfence();
        uint64_t done = __ballot(g == 0 && fin);
        while (done) {
            const int src = __ffsll((unsigned long long)done) - 1;
            done &= done - 1;
            const float M = __shfl(mref, src, 64);
            const float Ls = __shfl(l, src, 64);
            const int64_t gl = __shfl(S.gidx, src, 64);
            const int jl = __shfl(j, src, 64);
            const int64_t so = gl - jl;
            for (int jj = lane; jj <= jl; jj += 64)
                a.weights[so + jj] = __expf(a.scores[so + jj] - M) / Ls;
        }
    }
}

// Per-wave task bookkeeping: the task's sample range and packed start come
// from one read of the plan; then one lane per sample reads its packed start,
// length and sequence offset and fills the wave's position table (index in
// seq_values, sample, j and positions left).  Samples with no position get
// their zero output here.
__device__ inline int setup_task(const DinArgs& a, int t, PosEnt* pt, int lane) {
    const int2 i0 = a.task_info[t], i1 = a.task_info[t + 1];
    const int b0 = i0.x, b1 = i1.x, base = i0.y;
    wave_sync();
    for (int c0 = b0; c0 < b1; c0 += 64) {
        const int b = min(c0 + lane, b1 - 1);
        const int ps = a.pos_start[b], pn = a.pos_start[b + 1];
        const int64_t so = a.seq_offsets[b];
        if (c0 + lane < b1) {
            const int st = ps - base, L = pn - ps;
            if (L == 0) {
                float4* o = (float4*)(a.out + (int64_t)b * 48);
#pragma unroll
                for (int r = 0; r < 12; ++r) o[r] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            for (int j = 0; j < L; ++j) {
                PosEnt pe;
                pe.gidx = so + j;
                pe.b = b;
                pe.jr = j | ((L - 1 - j) << 16);
                pt[st + j] = pe;
            }
        }
    }
    wave_sync();
    return i1.y - base;
}

// Permuted A-operand images: slot (hb, kb, rt, lane, half) of W1 and
// (hb, mt, lane, rt) of W2, each 8 bytes = 4 consecutive bf16 of one row.
__device__ inline void w1_slot_source(int d, int* row, int* col) {
    const int half = d & 1, lane = (d >> 1) & 63, rest = d >> 7;
    const int rt = rest & 1, hbkb = rest >> 1, kb = hbkb % 6, hb = hbkb / 6;
    const int g = lane >> 4, m = lane & 15;
    const int i0 = kb * 8 + half * 4;             // first of the lane's 48 inputs in this slot
    *row = hb * 32 + rt * 16 + m;
    *col = 48 * (i0 / 12) + 12 * g + (i0 % 12);
}

__device__ inline void w2_slot_source(int d, int* row, int* col) {
    const int rt = d & 1, lane = (d >> 1) & 63, rest = d >> 7;
    const int mt = rest & 3, hb = rest >> 2;
    const int g = lane >> 4, m = lane & 15;
    *row = mt * 16 + m;
    *col = hb * 32 + rt * 16 + 4 * g;
}

__global__ __launch_bounds__(256) void k_din_pack(const uint16_t* __restrict__ w1,
                                                  const uint16_t* __restrict__ w2,
                                                  uint2* __restrict__ packed) {
    const int d = blockIdx.x * 256 + threadIdx.x;     // 8-byte slot
    int row, col;
    if (d < 12288) {
        w1_slot_source(d, &row, &col);
        packed[d] = *(const uint2*)(w1 + row * 192 + col);
    } else if (d < 16384) {
        w2_slot_source(d - 12288, &row, &col);
        packed[d] = *(const uint2*)(w2 + row * 256 + col);
    }
}

template <int DT, bool kHash>
__global__ __launch_bounds__(64 * kDinWaves) void k_din_attn(const DinArgs a) {
    constexpr bool kPacked = DT == REC_BF16_PACKED;
    constexpr bool kBF = DT == REC_BF16 || kPacked;
    constexpr int kThreads = 64 * kDinWaves;
    __shared__ uint4 s_wt[kBF ? (8 * 6 * 2 + 8 * 4) * 64 : 1];
    uint4* s_w1 = s_wt;
    uint4* s_w2 = s_wt + 8 * 6 * 2 * 64;
    __shared__ float s_b1[256];
    __shared__ float s_b2[64];
    __shared__ float s_w3[64];
    __shared__ PosEnt s_pos[kDinWaves][kSmap];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int num_tasks = a.plan_hdr[kHdrNumTasks];
    const int first = blockIdx.x * kDinWaves;
    if (first >= num_tasks) return;

    // Every weight load of this thread is issued at once (W1: 256 rows x 24
    // chunks of 16 B; W2: 64 rows x 32 chunks); the first task's bookkeeping
    // and gathers run while they are in flight.
    constexpr int kW1Per = (kBF && !kPacked) ? 256 * 24 / kThreads : 0;
    constexpr int kW2Per = (kBF && !kPacked) ? 64 * 32 / kThreads : 0;
    uint4 v1[kW1Per > 0 ? kW1Per : 1], v2[kW2Per > 0 ? kW2Per : 1];
    if (kPacked) {
        // the packed image is the LDS image: copy it straight from memory into
        // LDS (global_load_lds, 1 KiB per wave instruction, no registers)
        const uint4* src = (const uint4*)a.w1;
        constexpr int kChunks = (8 * 6 * 2 + 8 * 4) * 64;      // 16-byte chunks
#pragma unroll
        for (int i = 0; i < kChunks / kThreads; ++i) {
            const int c0 = (i * kDinWaves + wave) * 64;
            __builtin_amdgcn_global_load_lds((const void*)(src + c0 + lane),
                                             (__attribute__((address_space(3))) void*)(s_wt + c0), 16, 0, 0);
        }
    } else if (kBF) {
        const uint4* w1g = (const uint4*)a.w1;
        const uint4* w2g = (const uint4*)a.w2;
#pragma unroll
        for (int i = 0; i < kW1Per; ++i) v1[i] = w1g[threadIdx.x + i * kThreads];
#pragma unroll
        for (int i = 0; i < kW2Per; ++i) v2[i] = w2g[threadIdx.x + i * kThreads];
    }
    float vb1 = 0.f, vb2 = 0.f, vw3 = 0.f;
    if (threadIdx.x < 256) vb1 = a.b1[threadIdx.x];
    if (threadIdx.x < 64) {
        vb2 = a.b2[threadIdx.x];
        vw3 = a.w3[threadIdx.x];
    }

    PosEnt* pt = s_pos[wave];
    const int stride = gridDim.x * kDinWaves;
    int t = first + wave;
    int Ptask = t < num_tasks ? setup_task(a, t, pt, lane) : 0;
    int sb = 0;
    Sub S[2];
    bool two = false;
    if (Ptask > 0) {
        gather<kHash>(a, pt, lane & 15, Ptask, lane, S[0]);
        two = Ptask > 16;
        if (two) gather<kHash>(a, pt, 16 + (lane & 15), Ptask, lane, S[1]);
    }

    if (kBF && !kPacked) {
        // W1 [256][192] bf16 as 8-byte runs of 4 columns -> permuted A fragments:
        // column k = 48 tau + 12 g + f lands in lane g*16 + m, element i = 12 tau + f
        // of the lane's 48 (fragment kb = i / 8, slot i % 8).
        uint2* d1 = (uint2*)s_w1;
#pragma unroll
        for (int i = 0; i < kW1Per; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int o = c / 24;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = 8 * (c % 24) + 4 * h;
                const int tau = k / 48, c48 = k % 48, g = c48 / 12, f0 = c48 % 12;
                const int ii = 12 * tau + f0, kb = ii >> 3, j0 = ii & 7;
                const int hb = o >> 5, rt = (o >> 4) & 1, m = o & 15;
                const uint2 val = h ? make_uint2(v1[i].z, v1[i].w) : make_uint2(v1[i].x, v1[i].y);
                d1[(((hb * 6 + kb) * 2 + rt) * 64 + g * 16 + m) * 2 + (j0 >> 2)] = val;
            }
        }
        // W2 [64][256] bf16: fragment slot j = 4 rt + i <-> hidden hb*32 + rt*16 + 4g + i
        uint2* d2 = (uint2*)s_w2;
#pragma unroll
        for (int i = 0; i < kW2Per; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int o = c >> 5;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = 8 * (c & 31) + 4 * h;
                const int hb = k >> 5, rt = (k >> 4) & 1, g = (k >> 2) & 3;
                const int mt = o >> 4, m = o & 15;
                const uint2 val = h ? make_uint2(v2[i].z, v2[i].w) : make_uint2(v2[i].x, v2[i].y);
                d2[((hb * 4 + mt) * 64 + g * 16 + m) * 2 + rt] = val;
            }
        }
    }
    if (threadIdx.x < 256) s_b1[threadIdx.x] = vb1;
    if (threadIdx.x < 64) {
        s_b2[threadIdx.x] = vb2;
        s_w3[threadIdx.x] = vw3;
    }
    if (kPacked) __builtin_amdgcn_s_waitcnt(0);        // the LDS copies have landed
    __syncthreads();

    float m_open = -INFINITY, l_open = 0.f, acc_open[12];
#pragma unroll
    for (int f = 0; f < 12; ++f) acc_open[f] = 0.f;
    while (t < num_tasks) {
        if (sb < Ptask) {
            float e[2];
            if (two) {
                if (kBF) mlp_bf16<2>(S, s_w1, s_w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                else mlp_f32<2>(S, (const float*)a.w1, (const float*)a.w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                softmax_tile(a, S[0], e[0], lane, m_open, l_open, acc_open);
                softmax_tile(a, S[1], e[1], lane, m_open, l_open, acc_open);
            } else {
                if (kBF) mlp_bf16<1>(S, s_w1, s_w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                else mlp_f32<1>(S, (const float*)a.w1, (const float*)a.w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                softmax_tile(a, S[0], e[0], lane, m_open, l_open, acc_open);
            }
            sb += 32;
        }
        if (sb >= Ptask) {
            t += stride;
            if (t >= num_tasks) break;
            Ptask = setup_task(a, t, pt, lane);
            sb = 0;
            m_open = -INFINITY;
            l_open = 0.f;
#pragma unroll
            for (int f = 0; f < 12; ++f) acc_open[f] = 0.f;
        }
        if (sb < Ptask) {
            gather<kHash>(a, pt, sb + (lane & 15), Ptask, lane, S[0]);
            two = Ptask - sb > 16;
            if (two) gather<kHash>(a, pt, sb + 16 + (lane & 15), Ptask, lane, S[1]);
        }
    }
}

}  // namespace

hipError_t launch_din(const DinArgs& a, int num_cus, hipStream_t s) {
    int64_t blocks = (a.max_tasks + kDinWaves - 1) / kDinWaves;
    if (blocks > num_cus) blocks = num_cus;
    if (blocks < 1) blocks = 1;
    const bool hash = a.tab[0].kind == REC_HASH || a.tab[1].kind == REC_HASH || a.tab[2].kind == REC_HASH;
    const dim3 grid((unsigned)blocks), block(64 * kDinWaves);
    if (a.dtype == REC_BF16_PACKED) {
        if (hash) hipLaunchKernelGGL((k_din_attn<REC_BF16_PACKED, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_din_attn<REC_BF16_PACKED, false>), grid, block, 0, s, a);
    } else if (a.dtype == REC_BF16) {
        if (hash) hipLaunchKernelGGL((k_din_attn<REC_BF16, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_din_attn<REC_BF16, false>), grid, block, 0, s, a);
    } else {
        if (hash) hipLaunchKernelGGL((k_din_attn<REC_F32, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_din_attn<REC_F32, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_din_pack(const void* w1, const void* w2, void* packed, hipStream_t s) {
    hipLaunchKernelGGL(k_din_pack, dim3(16384 / 256), dim3(256), 0, s, (const uint16_t*)w1,
                       (const uint16_t*)w2, (uint2*)packed);
    return hipGetLastError();
}

}  // namespace rec
