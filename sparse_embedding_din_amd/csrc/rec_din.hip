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

__device__ inline TabDev pick_tab(const DinArgs& a, int f) {
    return f == 0 ? a.tab[0] : (f == 1 ? a.tab[1] : a.tab[2]);
}

// Gather q and s for the position idx of lane (n, g); g picks features
// 12g..12g+11, i.e. the 16-byte chunks 3g..3g+2 of the 48-float vector.
__device__ inline void gather(const DinArgs& a, const PosEnt* pt, int idx, int Ptask, int lane,
                              Sub& S) {
    const int n = lane & 15, g = lane >> 4;
    S.valid = idx < Ptask;
    PosEnt pe;
    pe.gidx = 0; pe.b = 0; pe.jr = 0;
    if (S.valid) pe = pt[idx];
    S.gidx = pe.gidx;
    S.b = pe.b;
    S.j = pe.jr & 0xffff;
    S.rem = pe.jr >> 16;
    // lanes of group f < 3 resolve sub-feature f's id of position n
    int64_t row = -1;
    if (g < 3 && S.valid) {
        const TabDev tb = pick_tab(a, g);
        const int64_t raw = a.seq_values[(int64_t)g * a.seq_stride + pe.gidx];
        row = resolve_row(tb, raw);
        if (a.rows_out) a.rows_out[(int64_t)g * a.seq_stride + pe.gidx] = row;
    }
    const int fa = (3 * g) >> 2, fb = (3 * g + 2) >> 2;
    const int64_t rowA = __shfl(row, fa * 16 + n, 64);
    const int64_t rowB = __shfl(row, fb * 16 + n, 64);
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int c4 = 3 * g + r;
        const int f = c4 >> 2, w = c4 & 3;
        const int64_t rr = (f == fa) ? rowA : rowB;
        const float* vb = f == 0 ? a.tab[0].values : (f == 1 ? a.tab[1].values : a.tab[2].values);
        float4 sv = make_float4(0.f, 0.f, 0.f, 0.f), qv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (S.valid) {
            if (rr >= 0) sv = *(const float4*)(vb + rr * 16 + 4 * w);
            qv = *(const float4*)(a.query + (int64_t)pe.b * a.query_ld + a.qcol[f] + 4 * w);
        }
        S.s[4 * r + 0] = sv.x; S.s[4 * r + 1] = sv.y; S.s[4 * r + 2] = sv.z; S.s[4 * r + 3] = sv.w;
        S.q[4 * r + 0] = qv.x; S.q[4 * r + 1] = qv.y; S.q[4 * r + 2] = qv.z; S.q[4 * r + 3] = qv.w;
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

template <int NSUB>
__device__ inline void mlp_bf16(const Sub* S, const uint4* w1p, const uint4* w2p, const float* b1s,
                                const float* b2s, const float* w3s, float b3, int lane,
                                float* e) {
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
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
        f32x4 acc1[NSUB][2];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            acc1[s][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc1[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < 6; ++kb) {
            const uint4 u0 = w1p[((hb * 6 + kb) * 2 + 0) * 64 + lane];
            const uint4 u1 = w1p[((hb * 6 + kb) * 2 + 1) * 64 + lane];
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, u0);
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, u1);
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                acc1[s][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xf[s][kb], acc1[s][0], 0, 0, 0);
                acc1[s][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xf[s][kb], acc1[s][1], 0, 0, 0);
            }
        }
        const float4 bA = *(const float4*)(b1s + hb * 32 + 4 * g);
        const float4 bB = *(const float4*)(b1s + hb * 32 + 16 + 4 * g);
        bf16x8 a2[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) a2[mt] = __builtin_bit_cast(bf16x8, w2p[(hb * 4 + mt) * 64 + lane]);
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
                acc2[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[mt], h, acc2[s][mt], 0, 0, 0);
        }
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

template <int DT>
__global__ __launch_bounds__(64 * kDinWaves) void k_din_attn(const DinArgs a) {
    constexpr bool kBF = DT == REC_BF16;
    __shared__ uint4 s_w1[kBF ? 8 * 6 * 2 * 64 : 1];
    __shared__ uint4 s_w2[kBF ? 8 * 4 * 64 : 1];
    __shared__ float s_b1[256];
    __shared__ float s_b2[64];
    __shared__ float s_w3[64];
    __shared__ PosEnt s_pos[kDinWaves][kSmap];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int num_tasks = a.plan_hdr[kHdrNumTasks];
    const int first = blockIdx.x * kDinWaves;
    if (first >= num_tasks) return;
    constexpr int kThreads = 64 * kDinWaves;
    if (kBF) {
        // W1 [256][192] bf16 in 4-element chunks -> permuted A fragments
        const uint2* w1g = (const uint2*)a.w1;
        uint2* d1 = (uint2*)s_w1;
        for (int c = threadIdx.x; c < 256 * 48; c += kThreads) {
            const int o = c / 48, k = 4 * (c % 48);
            const int tau = k / 48, c48 = k % 48, g = c48 / 12, f0 = c48 % 12;
            const int i = 12 * tau + f0, kb = i >> 3, j0 = i & 7;
            const int hb = o >> 5, rt = (o >> 4) & 1, m = o & 15;
            d1[(((hb * 6 + kb) * 2 + rt) * 64 + g * 16 + m) * 2 + (j0 >> 2)] = w1g[c];
        }
        // W2 [64][256] bf16: fragment element j = 4 rt + i <-> hidden hb*32 + rt*16 + 4g + i
        const uint2* w2g = (const uint2*)a.w2;
        uint2* d2 = (uint2*)s_w2;
        for (int c = threadIdx.x; c < 64 * 64; c += kThreads) {
            const int o = c >> 6, k = 4 * (c & 63);
            const int hb = k >> 5, rt = (k >> 4) & 1, g = (k >> 2) & 3;
            const int mt = o >> 4, m = o & 15;
            d2[((hb * 4 + mt) * 64 + g * 16 + m) * 2 + rt] = w2g[c];
        }
    }
    for (int c = threadIdx.x; c < 256; c += kThreads) s_b1[c] = a.b1[c];
    for (int c = threadIdx.x; c < 64; c += kThreads) {
        s_b2[c] = a.b2[c];
        s_w3[c] = a.w3[c];
    }
    __syncthreads();

    PosEnt* pt = s_pos[wave];
    for (int t = first + wave; t < num_tasks; t += gridDim.x * kDinWaves) {
        const int b0 = a.task_first[t], b1 = a.task_first[t + 1];
        const int base = a.pos_start[b0];
        const int Ptask = a.pos_start[b1] - base;
        wave_sync();
        for (int c0 = b0; c0 < b1; c0 += 64) {
            const int b = c0 + lane;
            if (b < b1) {
                const int st = a.pos_start[b] - base;
                const int L = a.pos_start[b + 1] - a.pos_start[b];
                const int64_t so = a.seq_offsets[b];
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
        float m_open = -INFINITY, l_open = 0.f, acc_open[12];
#pragma unroll
        for (int f = 0; f < 12; ++f) acc_open[f] = 0.f;
        for (int sb = 0; sb < Ptask; sb += 32) {
            Sub S[2];
            float e[2];
            gather(a, pt, sb + (lane & 15), Ptask, lane, S[0]);
            if (Ptask - sb > 16) {
                gather(a, pt, sb + 16 + (lane & 15), Ptask, lane, S[1]);
                if (kBF) mlp_bf16<2>(S, s_w1, s_w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                else mlp_f32<2>(S, (const float*)a.w1, (const float*)a.w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                softmax_tile(a, S[0], e[0], lane, m_open, l_open, acc_open);
                softmax_tile(a, S[1], e[1], lane, m_open, l_open, acc_open);
            } else {
                if (kBF) mlp_bf16<1>(S, s_w1, s_w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                else mlp_f32<1>(S, (const float*)a.w1, (const float*)a.w2, s_b1, s_b2, s_w3, a.b3, lane, e);
                softmax_tile(a, S[0], e[0], lane, m_open, l_open, acc_open);
            }
        }
    }
}

}  // namespace

hipError_t launch_din(const DinArgs& a, int num_cus, hipStream_t s) {
    int64_t blocks = (a.max_tasks + kDinWaves - 1) / kDinWaves;
    if (blocks > num_cus) blocks = num_cus;
    if (blocks < 1) blocks = 1;
    if (a.dtype == REC_BF16)
        hipLaunchKernelGGL(k_din_attn<REC_BF16>, dim3((unsigned)blocks), dim3(64 * kDinWaves), 0, s, a);
    else
        hipLaunchKernelGGL(k_din_attn<REC_F32>, dim3((unsigned)blocks), dim3(64 * kDinWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
