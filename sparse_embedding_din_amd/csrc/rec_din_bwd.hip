// Backward of the DIN target attention ("当前现状分析" §4.2 and §4.4 forward;
// the run-config table's training step through it): given the gradient of
// the attention output, the gradients of the query, of every sequence row and
// of the attention MLP's weights.
//
// Per sample b with L = min(len_b, max_len) positions the forward is
// recomputed and differentiated by the chain rule read backwards:
//   dp_j = g . s_j,  de_j = p_j (dp_j - sum_k p_k dp_k),  ds_j = p_j g
//   dz2_j = de_j w3 where h2_j > 0,  dz1_j = W2^T dz2_j where h1_j > 0
//   dx_j = W1^T dz1_j,  dq += dx[q] + dx[q-s] + s_j * dx[q*s],
//   ds_j += dx[s] - dx[q-s] + q * dx[q*s]
//   dW1 = sum_j dz1_j x_j^T, dW2 = sum_j dz2_j h1_j^T, dw3 = sum_j de_j h2_j
//   (and the biases: the sums of dz1, dz2, de).
//
// fp32 throughout; the per-position products run on the matrix cores
// (v_mfma_f32_16x16x4f32, 16 positions per tile):
//   k_dinb_prep    every position index marked as having no sample yet;
//                  W1^T and W2^T in fp32, the A operands of the forward;
//   k_dinb_map     the sample of every position index;
//   k_dinb_fwd     the forward of 32 positions per workgroup: S, [x, 1],
//                  [h1, 1], [h2, 1] and the score of every position;
//   k_dinb_soft    one wave per sample: the softmax weights p_j and de_j;
//   k_dinb_bwdt    the backward of 32 positions per workgroup: dz2, dz1, dx,
//                  each position's sequence-row gradient and query terms
//                  (zero rows where no position reads: past a sample's
//                  first max_len, gaps of a padded layout);
//   k_dinb_gq      the query gradient, each sample's terms in position order;
//   k_dinb_wgrad   the weight gradients as sums over positions of outer
//                  products, [dz1]^T [x, 1] (dW1 and db1), [dz2]^T [h1, 1]
//                  (dW2 and db2), [de]^T [h2, 1] (dw3 and db3), on the
//                  matrix cores with positions as K: one workgroup per range
//                  of positions (kDinbSplits ranges), whose sums
//                  k_dinb_reduce adds in range order.
// Every sum has one order: results are bit-identical run to run.
#include "rec_internal.h"
#include "rec_mfma.h"

namespace rec {
namespace {

constexpr int kDinbSplits = 256;      // position ranges of the weight gradients
constexpr int kLdX = 193, kLdH1 = 257, kLdH2 = 65;       // rows carry a trailing 1

__device__ inline float bf16_bits(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline float wload(const void* w, int64_t i, int bf16) {
    return bf16 ? bf16_bits(((const uint16_t*)w)[i]) : ((const float*)w)[i];
}

// Every position index marked as having no sample yet (k_dinb_map then marks
// the real ones), and W1^T [192][256] and W2^T [256][64] in fp32, the
// forward tile's A operands (so that its weight reads are coalesced).
__global__ __launch_bounds__(256) void k_dinb_prep(DinBwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t p = i; p < a.seq_stride; p += (int64_t)gridDim.x * blockDim.x) a.map[p] = -1;
    if (i < 256 * 192) {
        const int64_t o = i / 192, c = i - o * 192;
        a.w1t[c * 256 + o] = wload(a.w1, i, a.bf16);
    } else if (i < 256 * 192 + 64 * 256) {
        const int64_t j = i - 256 * 192, o = j / 256, c = j - o * 256;
        a.w2t[c * 64 + o] = wload(a.w2, j, a.bf16);
    }
}

// Sample of every position index: map[p] = b for p = off_b + j, j < L_b.
__global__ __launch_bounds__(256) void k_dinb_map(DinBwdArgs a) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < a.B;
         b += (int64_t)gridDim.x * blockDim.x) {
        const int32_t len = a.seq_lengths[b];
        const int L = len < a.max_len ? len : a.max_len;
        const int64_t off = a.seq_offsets[b];
        for (int j = 0; j < L; ++j) a.map[off + j] = (int32_t)b;
    }
}

constexpr int kTP = 32;          // positions per workgroup: two 16-position MFMA tiles
constexpr int kLdS = 260;        // LDS row stride (floats) of the h1 / dz1 rows

// v_mfma_f32_16x16x4f32, lane l = 16 g + n: A element (row n, K slot g), B
// element (K slot g, column n); the result holds rows 4g .. 4g+3 of column n.
// Columns are positions throughout; the K order of a product is free as long
// as A and B agree.
__device__ inline f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The lane's 12 features c = 12 g + f of position p's query (q) and
// sequence row (s); zero where p has no sample, s zero on a hash miss.
__device__ inline void lane_inputs(const DinBwdArgs& a, int64_t p, int b, int g, float* q, float* s) {
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int c = 12 * g + 4 * r, f = c >> 4, d = c & 15;
        float4 sv = make_float4(0.f, 0.f, 0.f, 0.f), qv = sv;
        if (b >= 0) {
            const TabDev& t = a.tabs[f];
            const int64_t x = a.seq_values[(int64_t)f * a.seq_stride + p];
            const int64_t row = t.kind == REC_HASH ? hash_probe(t, x) : floor_mod_magic(x, t.rows, t.magic, t.shift);
            if (row >= 0) sv = *(const float4*)(t.values + row * REC_DIM + d);
            const float* qr = a.query + (int64_t)b * a.query_ld + a.qcol[f] + d;
            qv = make_float4(qr[0], qr[1], qr[2], qr[3]);
        }
        s[4 * r] = sv.x; s[4 * r + 1] = sv.y; s[4 * r + 2] = sv.z; s[4 * r + 3] = sv.w;
        q[4 * r] = qv.x; q[4 * r + 1] = qv.y; q[4 * r + 2] = qv.z; q[4 * r + 3] = qv.w;
    }
}

// Forward of 32 positions on the matrix cores (fp32 operands): each of the
// four waves builds the inputs x = [q, s, q-s, q*s] of all 32 positions in
// registers (input i = 12 tau + f of lane g is column 48 tau + 12 g + f of
// W1), runs h1 = relu(W1 x + b1) for its 64 hidden units and stages them in
// LDS; then wave w runs h2 = relu(W2 h1 + b2) for units 16 w .. 16 w + 15 and
// its share of the score, the four shares added in wave order.  Stores S,
// [h1, 1], [h2, 1], the score and, with weight gradients, [x, 1].
__global__ __launch_bounds__(256) void k_dinb_fwd(DinBwdArgs a) {
    __shared__ __attribute__((aligned(16))) float hs[kTP * kLdS];
    __shared__ float sc[4][kTP];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
    const int64_t p0 = (int64_t)blockIdx.x * kTP;
    int64_t p[2];
    int bs[2];
    float x[2][48];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        p[s] = p0 + 16 * s + n;
        bs[s] = p[s] < a.seq_stride ? a.map[p[s]] : -1;
        float q[12], sv[12];
        lane_inputs(a, p[s], bs[s], g, q, sv);
#pragma unroll
        for (int f = 0; f < 12; ++f) {
            x[s][f] = q[f];
            x[s][12 + f] = sv[f];
            x[s][24 + f] = q[f] - sv[f];
            x[s][36 + f] = q[f] * sv[f];
        }
        if (bs[s] >= 0) {
            if (w == 0) {
#pragma unroll
                for (int r = 0; r < 3; ++r)
                    *(float4*)(a.S + p[s] * 48 + 12 * g + 4 * r) =
                        make_float4(sv[4 * r], sv[4 * r + 1], sv[4 * r + 2], sv[4 * r + 3]);
            } else if (w == 1 && a.wgrad) {
#pragma unroll
                for (int i = 0; i < 48; ++i) a.X[p[s] * kLdX + 48 * (i / 12) + 12 * g + (i % 12)] = x[s][i];
                if (g == 0) a.X[p[s] * kLdX + 192] = 1.0f;
            } else if (w == 2 && g == 0) {
                a.H1[p[s] * kLdH1 + 256] = 1.0f;
                a.H2[p[s] * kLdH2 + 64] = 1.0f;
            }
        }
    }
    // layer 1: hidden blocks 2w and 2w + 1 (32 units each, two row tiles)
#pragma unroll 1
    for (int hh = 0; hh < 2; ++hh) {
        const int hb = 2 * w + hh;
        f32x4 acc[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 bv = {0.f, 0.f, 0.f, 0.f};
            if (a.b1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) bv[i] = a.b1[hb * 32 + rt * 16 + 4 * g + i];
            }
            acc[0][rt] = bv;
            acc[1][rt] = bv;
        }
        const float* wr = a.w1t + (int64_t)(12 * g) * 256 + hb * 32 + n;
#pragma unroll
        for (int i = 0; i < 48; ++i) {
            const int k = 48 * (i / 12) + (i % 12);          // + 12 g, in wr
            const float a0 = wr[k * 256], a1 = wr[k * 256 + 16];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                acc[s][0] = mfma4(a0, x[s][i], acc[s][0]);
                acc[s][1] = mfma4(a1, x[s][i], acc[s][1]);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int u = hb * 32 + rt * 16 + 4 * g + i;
                    const float h = fmaxf(acc[s][rt][i], 0.0f);
                    hs[(16 * s + n) * kLdS + u] = h;
                    if (bs[s] >= 0) a.H1[p[s] * kLdH1 + u] = h;
                }
    }
    __syncthreads();
    // layer 2: outputs 16 w .. 16 w + 15, K = the 256 units as 64 steps of 4
    // (unit 4 k4 + g), two accumulators per tile for independent chains
    f32x4 acc2[2][2];
    {
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (a.b2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = a.b2[16 * w + 4 * g + i];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            acc2[s][0] = bv;
            acc2[s][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const float* w2r = a.w2t + (int64_t)g * 64 + 16 * w + n;
    // eight chunks of eight steps, the next chunk's weights in flight
    float aw[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) aw[0][j] = w2r[4 * j * 64];
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        if (ch + 1 < 8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) aw[(ch + 1) & 1][j] = w2r[4 * (8 * (ch + 1) + j) * 64];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int u = 4 * (8 * ch + j);                  // + g
#pragma unroll
            for (int s = 0; s < 2; ++s)
                acc2[s][j & 1] = mfma4(aw[ch & 1][j], hs[(16 * s + n) * kLdS + u + g], acc2[s][j & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = 16 * w + 4 * g + i;
            const float h2 = fmaxf(acc2[s][0][i] + acc2[s][1][i], 0.0f);
            if (bs[s] >= 0) a.H2[p[s] * kLdH2 + o] = h2;
            part += a.w3[o] * h2;
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        if (g == 0) sc[w][16 * s + n] = part;
    }
    __syncthreads();
    if (threadIdx.x < kTP) {
        const int64_t pp = p0 + threadIdx.x;
        if (pp < a.seq_stride && a.map[pp] >= 0)
            a.E[pp] = a.b3 + (((sc[0][threadIdx.x] + sc[1][threadIdx.x]) + sc[2][threadIdx.x]) + sc[3][threadIdx.x]);
    }
}

// Softmax of each sample over its scores, one wave per sample: p_j,
// dp_j = g . s_j and de_j = p_j (dp_j - sum_k p_k dp_k).  Lane l takes the
// positions j = l, l + 64, ... (any length up to max_len); the max, the
// denominator and sum_k exp(e_k - m) dp_k are reduced by fixed shuffle
// trees.  The second pass parks exp(e_j - m) in PW and dp_j in DE, which the
// same lane rewrites in the third.
__global__ __launch_bounds__(256) void k_dinb_soft(DinBwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int32_t len = a.seq_lengths[b];
    const int L = len < a.max_len ? len : a.max_len;
    if (L <= 0) return;
    const int64_t off = a.seq_offsets[b];
    const float* g = a.gatt + b * 48;
    float m = -INFINITY;
    for (int j = lane; j < L; j += 64) m = fmaxf(m, a.E[off + j]);
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    float den = 0.0f, edp = 0.0f;
    for (int j = lane; j < L; j += 64) {
        const int64_t p = off + j;
        float dp = 0.0f;
        for (int c = 0; c < 48; ++c) dp += g[c] * a.S[p * 48 + c];
        const float ex = expf(a.E[p] - m);
        den += ex;
        edp += ex * dp;
        a.PW[p] = ex;
        a.DE[p] = dp;
    }
    for (int d = 32; d >= 1; d >>= 1) {
        den += __shfl_xor(den, d, 64);
        edp += __shfl_xor(edp, d, 64);
    }
    const float pdp = edp / den;
    for (int j = lane; j < L; j += 64) {
        const int64_t p = off + j;
        const float pw = a.PW[p] / den;
        a.PW[p] = pw;
        a.DE[p] = pw * (a.DE[p] - pdp);
    }
}

template <bool BF>
__device__ inline float wld(const void* w, int64_t i) {
    if constexpr (BF) return bf16_bits(((const uint16_t*)w)[i]);
    else return ((const float*)w)[i];
}

// Backward of 32 positions on the matrix cores (fp32 operands):
// dz2 = de w3 where h2 > 0 (every wave, all 64 units, from [h2, 1] and de);
// wave w: dz1 = W2^T dz2 where h1 > 0 for units 64 w .. 64 w + 63, staged in
// LDS; then dx = W1^T dz1 for inputs 48 w .. 48 w + 47, i.e. the block
// tau = w of [q, s, q-s, q*s]; the four blocks meet in LDS for each
// position's sequence-row gradient and its terms of the query gradient.
// Weights are read in their own layout and type.
template <bool BF>
__global__ __launch_bounds__(256) void k_dinb_bwdt(DinBwdArgs a) {
    __shared__ __attribute__((aligned(16))) float ds[kTP * kLdS];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
    const int64_t p0 = (int64_t)blockIdx.x * kTP;
    int64_t p[2];
    int bs[2];
    float dz2[2][16];                  // step st: unit 16 (st / 4) + 4 g + st % 4
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        p[s] = p0 + 16 * s + n;
        bs[s] = p[s] < a.seq_stride ? a.map[p[s]] : -1;
        const float de = bs[s] >= 0 ? a.DE[p[s]] : 0.0f;
#pragma unroll
        for (int st = 0; st < 16; ++st) {
            const int o = 16 * (st >> 2) + 4 * g + (st & 3);
            const float h2 = bs[s] >= 0 ? a.H2[p[s] * kLdH2 + o] : 0.0f;
            dz2[s][st] = h2 > 0.0f ? de * a.w3[o] : 0.0f;
        }
        if (w == 0 && a.wgrad && bs[s] >= 0) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                *(float4*)(a.DZ2 + p[s] * 64 + 16 * mt + 4 * g) =
                    make_float4(dz2[s][4 * mt], dz2[s][4 * mt + 1], dz2[s][4 * mt + 2], dz2[s][4 * mt + 3]);
        }
    }
    // dz1 for the row tiles ut = 4w .. 4w + 3: A = W2[o][16 ut + n]
    f32x4 acc[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[s][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 16; ++st) {
        const int o = 16 * (st >> 2) + 4 * g + (st & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float av = wld<BF>(a.w2, (int64_t)o * 256 + (4 * w + j) * 16 + n);
#pragma unroll
            for (int s = 0; s < 2; ++s) acc[s][j] = mfma4(av, dz2[s][st], acc[s][j]);
        }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u0 = (4 * w + j) * 16 + 4 * g;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float h1 = bs[s] >= 0 ? a.H1[p[s] * kLdH1 + u0 + i] : 0.0f;
                v[i] = h1 > 0.0f ? acc[s][j][i] : 0.0f;
                ds[(16 * s + n) * kLdS + u0 + i] = v[i];
            }
            if (a.wgrad && bs[s] >= 0)
                *(float4*)(a.DZ1 + p[s] * 256 + u0) = make_float4(v[0], v[1], v[2], v[3]);
        }
    __syncthreads();
    // dx for the row tiles 3w .. 3w + 2, K = the 256 units as 64 steps of 4
    // (unit 4 k4 + g): A = W1[unit][16 (3w + c1) + n]
    f32x4 dx[2][3];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c1 = 0; c1 < 3; ++c1) dx[s][c1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K in eight chunks of eight steps, the next chunk's weights in flight
    // while this chunk's products run
    float aw[2][8][3];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int c1 = 0; c1 < 3; ++c1)
            aw[0][j][c1] = wld<BF>(a.w1, (int64_t)(4 * j + g) * 192 + (3 * w + c1) * 16 + n);
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        if (ch + 1 < 8) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int c1 = 0; c1 < 3; ++c1)
                    aw[(ch + 1) & 1][j][c1] =
                        wld<BF>(a.w1, (int64_t)(4 * (8 * (ch + 1) + j) + g) * 192 + (3 * w + c1) * 16 + n);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int u = 4 * (8 * ch + j) + g;
            float bv[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) bv[s] = ds[(16 * s + n) * kLdS + u];
#pragma unroll
            for (int c1 = 0; c1 < 3; ++c1)
#pragma unroll
                for (int s = 0; s < 2; ++s) dx[s][c1] = mfma4(aw[ch & 1][j][c1], bv[s], dx[s][c1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();                   // every wave is done reading dz1
    // block tau = w of dx, element c = 16 c1 + 4 g + i, into dxs[tau][position][48]
    float* dxs = ds;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c1 = 0; c1 < 3; ++c1)
            *(float4*)(dxs + (w * kTP + 16 * s + n) * 48 + 16 * c1 + 4 * g) =
                make_float4(dx[s][c1][0], dx[s][c1][1], dx[s][c1][2], dx[s][c1][3]);
    __syncthreads();
    for (int idx = threadIdx.x; idx < kTP * 48; idx += 256) {
        const int pi = idx / 48, c = idx - pi * 48;
        const int64_t pp = p0 + pi;
        if (pp >= a.seq_stride) continue;
        const int b = a.map[pp];
        if (b < 0) {                   // no position here: a zero row
            if (a.gs) a.gs[((int64_t)(c >> 4) * a.seq_stride + pp) * REC_DIM + (c & 15)] = 0.0f;
            continue;
        }
        const float d0 = dxs[(0 * kTP + pi) * 48 + c], d1 = dxs[(1 * kTP + pi) * 48 + c];
        const float d2 = dxs[(2 * kTP + pi) * 48 + c], d3 = dxs[(3 * kTP + pi) * 48 + c];
        const float sv = a.S[pp * 48 + c];
        const float qv = a.query[(int64_t)b * a.query_ld + a.qcol[c >> 4] + (c & 15)];
        if (a.gs)
            a.gs[((int64_t)(c >> 4) * a.seq_stride + pp) * REC_DIM + (c & 15)] =
                a.PW[pp] * a.gatt[(int64_t)b * 48 + c] + d1 - d2 + qv * d3;
        a.GQP[pp * 48 + c] = d0 + d2 + sv * d3;
    }
}

// Query gradient: each sample's position terms added in position order.
__global__ __launch_bounds__(256) void k_dinb_gq(DinBwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.B * 48) return;
    const int64_t b = i / 48;
    const int c = (int)(i - b * 48);
    const int32_t len = a.seq_lengths[b];
    const int L = len < a.max_len ? len : a.max_len;
    const int64_t off = a.seq_offsets[b];
    float s = 0.0f;
    int j = 0;
    // four loads in flight per round, added in position order
    for (; j + 4 <= L; j += 4) {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = a.GQP[(off + j + k) * 48 + c];
#pragma unroll
        for (int k = 0; k < 4; ++k) s += v[k];
    }
    for (; j < L; ++j) s += a.GQP[(off + j) * 48 + c];
    a.gq[i] = s;
}

// Weight gradients of one range of positions per workgroup, on the matrix
// cores with the positions as the K index (4 per step, lane group g takes
// position 4 k + g): C[m][n] += A[p][m] B[p][n] for dW1 (A = dz1, B = [x, 1],
// 16 x 13 tiles of 16 x 16), dW2 (A = dz2, B = [h1, 1], 4 x 17 tiles) and dw3
// (A = de, one row, B = [h2, 1], 5 tiles).  Wave w owns dW1's row tiles 2w and
// 2w + 1, dW2's row tile w / 2 with nine of its column tiles (the ninth of the
// odd waves lies past the edge and is dropped), and wave 7 the dw3 tiles.
// Each position's rows are staged once per workgroup in LDS and every wave
// reads its operands there.  Positions without a sample, and columns past an
// edge, enter as zeros.  The range's sums go to its slot of the split sums,
// which k_dinb_reduce adds in range order.
constexpr int kWgWaves = 8;

// A position's operand row in LDS: [x, 1] (193), dz1 (256), [h1, 1] (257),
// dz2 (64), [h2, 1] (65), de (1), padded to a stride of 848 floats (848 mod 64
// = 16, so the four positions a step reads fall in distinct banks).
constexpr int kWgRow = kLdX + 256 + kLdH1 + 64 + kLdH2 + 1;     // 836
constexpr int kWgStride = 848;
constexpr int kWgStage = 16;                                   // positions per staged block
constexpr int kWgPer = (kWgRow + 31) / 32;                     // floats per thread per stage (27)
constexpr int kWgOffDZ1 = kLdX, kWgOffH1 = kWgOffDZ1 + 256, kWgOffDZ2 = kWgOffH1 + kLdH1,
              kWgOffH2 = kWgOffDZ2 + 64, kWgOffDE = kWgOffH2 + kLdH2;
static_assert(kWgStage * 32 == 64 * kWgWaves, "32 threads per staged position");

// Thread t loads floats j = (t % 32) + 32 k of position pb + t / 32's row
// (zeros past the range or for a position without a sample).
__device__ inline void wg_stage_load(const DinBwdArgs& a, int64_t pb, int64_t p1, float (&v)[kWgPer]) {
    const int t = threadIdx.x, l = t & 31;
    const int64_t p = pb + (t >> 5);
    const bool ok = p < p1 && a.map[p] >= 0;
#pragma unroll
    for (int k = 0; k < kWgPer; ++k) {
        const int j = l + 32 * k;
        float x = 0.0f;
        if (ok && j < kWgRow) {
            if (j < kWgOffDZ1) x = a.X[p * kLdX + j];
            else if (j < kWgOffH1) x = a.DZ1[p * 256 + (j - kWgOffDZ1)];
            else if (j < kWgOffDZ2) x = a.H1[p * kLdH1 + (j - kWgOffH1)];
            else if (j < kWgOffH2) x = a.DZ2[p * 64 + (j - kWgOffDZ2)];
            else if (j < kWgOffDE) x = a.H2[p * kLdH2 + (j - kWgOffH2)];
            else x = a.DE[p];
        }
        v[k] = x;
    }
}

__device__ inline void wg_stage_store(float* buf, const float (&v)[kWgPer]) {
    const int t = threadIdx.x, l = t & 31;
    float* row = buf + (t >> 5) * kWgStride;
#pragma unroll
    for (int k = 0; k < kWgPer; ++k) {
        const int j = l + 32 * k;
        if (j < kWgRow) row[j] = v[k];
    }
}

__global__ __launch_bounds__(64 * kWgWaves) void k_dinb_wgrad(DinBwdArgs a, int64_t chunk) {
    __shared__ float s_op[2][kWgStage * kWgStride];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
    const int64_t p0 = (int64_t)blockIdx.x * chunk;
    const int64_t p1 = p0 + chunk < a.seq_stride ? p0 + chunk : a.seq_stride;
    const int c2lo = (w & 1) ? 9 : 0, r2 = w >> 1;
    f32x4 acc1[2][13], acc2[9], acc3[5];
#pragma unroll
    for (int c = 0; c < 13; ++c) acc1[0][c] = acc1[1][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 9; ++c) acc2[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 5; ++c) acc3[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Stages of 16 positions through LDS: the workgroup reads each position's
    // rows once (32 threads a row, coalesced), the next stage's loads in
    // flight while this stage's products run.  Steps of four positions, in
    // order, as the products were before: the sums are the same.
    float v[kWgPer];
    if (p0 < p1) {
        wg_stage_load(a, p0, p1, v);
        wg_stage_store(s_op[0], v);
    }
    __syncthreads();
    int buf = 0;
    for (int64_t sb = p0; sb < p1; sb += kWgStage) {
        const bool more = sb + kWgStage < p1;
        if (more) wg_stage_load(a, sb + kWgStage, p1, v);
        const float* st = s_op[buf];
#pragma unroll
        for (int k = 0; k < kWgStage / 4; ++k) {
            if (sb + 4 * k >= p1) break;                     // uniform
            const float* r = st + (4 * k + g) * kWgStride;   // position sb + 4k + g
            float A1[2], B1[13], A2, B2[9];
#pragma unroll
            for (int t = 0; t < 2; ++t) A1[t] = r[kWgOffDZ1 + 16 * (2 * w + t) + n];
#pragma unroll
            for (int c = 0; c < 13; ++c) B1[c] = 16 * c + n < kLdX ? r[16 * c + n] : 0.0f;
            A2 = r[kWgOffDZ2 + 16 * r2 + n];
#pragma unroll
            for (int c = 0; c < 9; ++c) {
                const int col = 16 * (c2lo + c) + n;
                B2[c] = col < kLdH1 ? r[kWgOffH1 + col] : 0.0f;
            }
#pragma unroll
            for (int c = 0; c < 13; ++c) {
                acc1[0][c] = mfma4(A1[0], B1[c], acc1[0][c]);
                acc1[1][c] = mfma4(A1[1], B1[c], acc1[1][c]);
            }
#pragma unroll
            for (int c = 0; c < 9; ++c) acc2[c] = mfma4(A2, B2[c], acc2[c]);
            if (w == kWgWaves - 1) {
                const float A3 = n == 0 ? r[kWgOffDE] : 0.0f;
#pragma unroll
                for (int c = 0; c < 5; ++c) {
                    const int col = 16 * c + n;
                    acc3[c] = mfma4(A3, col < kLdH2 ? r[kWgOffH2 + col] : 0.0f, acc3[c]);
                }
            }
        }
        if (more) wg_stage_store(s_op[buf ^ 1], v);
        __syncthreads();
        buf ^= 1;
    }
    // result element i of a tile: row 4 g + i, column n
    float* out = a.part + (int64_t)blockIdx.x * a.part_stride;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < 13; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * (2 * w + t) + 4 * g + i, col = 16 * c + n;
                if (col < kLdX) out[(int64_t)m * kLdX + col] = acc1[t][c][i];
            }
    float* out2 = out + 256 * kLdX;
#pragma unroll
    for (int c = 0; c < 9; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * r2 + 4 * g + i, col = 16 * (c2lo + c) + n;
            if (col < kLdH1) out2[(int64_t)m * kLdH1 + col] = acc2[c][i];
        }
    if (w == kWgWaves - 1 && g == 0) {
        float* out3 = out2 + 64 * kLdH1;
#pragma unroll
        for (int c = 0; c < 5; ++c) {
            const int col = 16 * c + n;
            if (col < kLdH2) out3[col] = acc3[c][0];
        }
    }
}

__global__ __launch_bounds__(256) void k_dinb_reduce(DinBwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.part_stride) return;
    float s = 0.0f;
    for (int k = 0; k < kDinbSplits; ++k) s += a.part[k * a.part_stride + i];
    const int64_t n0 = 256 * kLdX, n1 = 64 * kLdH1;
    if (i < n0) {
        const int64_t m = i / kLdX, n = i - m * kLdX;
        if (n < 192) a.dw1[m * 192 + n] = s; else a.db1[m] = s;
    } else if (i < n0 + n1) {
        const int64_t j = i - n0, m = j / kLdH1, n = j - m * kLdH1;
        if (n < 256) a.dw2[m * 256 + n] = s; else a.db2[m] = s;
    } else {
        const int64_t n = i - n0 - n1;
        if (n < 64) a.dw3[n] = s; else a.db3[0] = s;
    }
}

}  // namespace

int64_t din_bwd_part_stride() { return 256 * kLdX + 64 * kLdH1 + kLdH2; }
int din_bwd_splits() { return kDinbSplits; }

hipError_t launch_din_bwd(const DinBwdArgs& a, hipStream_t s) {
    int64_t pgrid = (a.seq_stride + 255) / 256;
    const int64_t tgrid = (256 * 192 + 64 * 256 + 255) / 256;
    pgrid = pgrid < tgrid ? tgrid : (pgrid < 65536 ? pgrid : 65536);
    hipLaunchKernelGGL(k_dinb_prep, dim3((unsigned)pgrid), dim3(256), 0, s, a);
    const int64_t bgrid = (a.B + 255) / 256;
    hipLaunchKernelGGL(k_dinb_map, dim3((unsigned)(bgrid < 65536 ? bgrid : 65536)), dim3(256), 0, s, a);
    const int64_t tiles = (a.seq_stride + kTP - 1) / kTP;
    if (tiles > 0) hipLaunchKernelGGL(k_dinb_fwd, dim3((unsigned)tiles), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_dinb_soft, dim3((unsigned)((a.B + 3) / 4)), dim3(256), 0, s, a);
    if (tiles > 0) {
        if (a.bf16) hipLaunchKernelGGL(k_dinb_bwdt<true>, dim3((unsigned)tiles), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(k_dinb_bwdt<false>, dim3((unsigned)tiles), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(k_dinb_gq, dim3((unsigned)((a.B * 48 + 255) / 256)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.wgrad) return e;
    const int64_t chunk = ((a.seq_stride + kDinbSplits - 1) / kDinbSplits + 3) & ~(int64_t)3;
    hipLaunchKernelGGL(k_dinb_wgrad, dim3((unsigned)kDinbSplits), dim3(64 * kWgWaves), 0, s, a, chunk);
    hipLaunchKernelGGL(k_dinb_reduce, dim3((unsigned)((a.part_stride + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
