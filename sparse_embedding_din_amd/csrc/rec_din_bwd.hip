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
// Plain fp32 arithmetic (a first, correctness-first version; its matrix
// products are small per position and run on the vector units):
//   k_dinb_transpose  W1^T and W2^T in fp32 into the workspace, so that the
//                  forward products read weights coalesced as the backward's do;
//   k_dinb_clear   every position index: its validity flag and its rows of
//                  grad_seq set to zero (positions past a sample's first
//                  max_len, and gaps of a padded layout, stay zero);
//   k_dinb_sample  one 256-thread workgroup per sample: the scores, the
//                  softmax, then position by position the backward above;
//                  with weight gradients requested it stores per position
//                  [x, 1], [h1, 1], [h2, 1], dz1, dz2 and de;
//   k_dinb_wgrad   the weight gradients as sums over positions of outer
//                  products, [dz1]^T [x, 1] (dW1 and db1), [dz2]^T [h1, 1]
//                  (dW2 and db2), [de]^T [h2, 1] (dw3 and db3): 64 x 64
//                  output tiles, blocks of positions staged in LDS, the
//                  positions split in kDinbSplits ranges, partial sums then
//                  added in split order by k_dinb_reduce.
// Every sum has one order: results are bit-identical run to run.
#include "rec_internal.h"

namespace rec {
namespace {

constexpr int kDinbSplits = 64;
constexpr int kLdX = 193, kLdH1 = 257, kLdH2 = 65;       // rows carry a trailing 1
constexpr int kJobs = 3;
// job j: C[M][N] = sum_p A[p][m] Bm[p][n]
__constant__ int kJobM[kJobs] = {256, 64, 1};
__constant__ int kJobN[kJobs] = {kLdX, kLdH1, kLdH2};

__device__ inline float bf16_bits(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline float wload(const void* w, int64_t i, int bf16) {
    return bf16 ? bf16_bits(((const uint16_t*)w)[i]) : ((const float*)w)[i];
}

// Component d of the row of raw id x in table t (0 on a hash miss).
__device__ inline float seq_elem(const TabDev& t, int64_t x, int d) {
    const int64_t r = t.kind == REC_HASH ? hash_probe(t, x) : floor_mod_magic(x, t.rows, t.magic, t.shift);
    return r < 0 ? 0.0f : t.values[r * REC_DIM + d];
}

__global__ __launch_bounds__(256) void k_dinb_clear(DinBwdArgs a) {
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < a.seq_stride;
         p += (int64_t)gridDim.x * blockDim.x) {
        a.map[p] = -1;
        if (a.gs) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                float4* r = (float4*)(a.gs + ((int64_t)k * a.seq_stride + p) * REC_DIM);
#pragma unroll
                for (int u = 0; u < 4; ++u) r[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
}

// W1^T [192][256] and W2^T [256][64] in fp32, once per call, so that every
// product below reads the weights with consecutive threads on consecutive
// addresses.
__global__ __launch_bounds__(256) void k_dinb_transpose(DinBwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

constexpr int kPT = 32;          // positions per tile (two tiles' LDS fit a CU)
constexpr int kPPT = kPT / 16;   // positions per thread
constexpr int kXS = 196;         // LDS row stride of x / dx rows (192 + 4)
constexpr int kHS = 260;         // LDS row stride of h1 / dz1 rows (256 + 4)
constexpr int kWBF = 16 * 260;   // staged weight block (floats)

struct TileLds {
    float xs[kPT * kXS];         // x rows, later dz2 (stride 65) and dx rows
    float hs[kPT * kHS];         // h1 rows, later dz1 rows
    float wb[kWBF];              // a block of weight rows
};

__device__ inline void unpack16(const float* p, float* v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float4 x = *(const float4*)(p + 4 * u);
        v[4 * u] = x.x; v[4 * u + 1] = x.y; v[4 * u + 2] = x.z; v[4 * u + 3] = x.w;
    }
}

// Forward of kPT positions: x (from the query of the position's sample and its
// sequence row), h1 = relu(W1 x + b1), h2 = relu(W2 h1 + b2), the score; as
// LDS-tiled products, each block of weight rows staged once for the tile.
// Thread (pr, uc) = (t / 16, t % 16) owns positions kPPT pr .. kPPT pr + kPPT - 1.
__global__ __launch_bounds__(256) void k_dinb_fwd(DinBwdArgs a) {
    __shared__ __attribute__((aligned(16))) TileLds L;
    const int t = threadIdx.x, pr = t >> 4, uc = t & 15;
    const int64_t p0 = (int64_t)blockIdx.x * kPT;
    for (int idx = t; idx < kPT * 48; idx += 256) {
        const int pi = idx / 48, c = idx - pi * 48, f = c >> 4;
        const int64_t p = p0 + pi;
        const int b = p < a.seq_stride ? a.map[p] : -1;
        float sv = 0.0f, qv = 0.0f;
        if (b >= 0) {
            sv = seq_elem(a.tabs[f], a.seq_values[(int64_t)f * a.seq_stride + p], c & 15);
            qv = a.query[(int64_t)b * a.query_ld + a.qcol[f] + (c & 15)];
            a.S[p * 48 + c] = sv;
        }
        float* x = L.xs + pi * kXS;
        x[c] = qv;
        x[48 + c] = sv;
        x[96 + c] = qv - sv;
        x[144 + c] = qv * sv;
    }
    __syncthreads();
    // h1: units 16 uc .. 16 uc + 15
    float acc[kPPT][16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float bj = a.b1 ? a.b1[16 * uc + j] : 0.0f;
#pragma unroll
        for (int i = 0; i < kPPT; ++i) acc[i][j] = bj;
    }
    for (int kb = 0; kb < 192; kb += 16) {
        for (int e = t; e < 16 * 256; e += 256) {
            const int kk = e >> 8, u = e & 255;
            L.wb[kk * 260 + u] = a.w1t[(kb + kk) * 256 + u];
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < 16; ++kk) {
            float xv[kPPT], wv[16];
#pragma unroll
            for (int i = 0; i < kPPT; ++i) xv[i] = L.xs[(kPPT * pr + i) * kXS + kb + kk];
            unpack16(L.wb + kk * 260 + 16 * uc, wv);
#pragma unroll
            for (int i = 0; i < kPPT; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[i][j] += xv[i] * wv[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kPPT; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) L.hs[(kPPT * pr + i) * kHS + 16 * uc + j] = acc[i][j] > 0.0f ? acc[i][j] : 0.0f;
    __syncthreads();
    // h2: units 4 uc .. 4 uc + 3
    float a2[kPPT][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float bj = a.b2 ? a.b2[4 * uc + j] : 0.0f;
#pragma unroll
        for (int i = 0; i < kPPT; ++i) a2[i][j] = bj;
    }
    for (int kb = 0; kb < 256; kb += 64) {
        for (int e = t; e < 64 * 64; e += 256) {
            const int kk = e >> 6, u = e & 63;
            L.wb[kk * 65 + u] = a.w2t[(kb + kk) * 64 + u];
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < 64; ++kk) {
            float hv[kPPT];
#pragma unroll
            for (int i = 0; i < kPPT; ++i) hv[i] = L.hs[(kPPT * pr + i) * kHS + kb + kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = L.wb[kk * 65 + 4 * uc + j];
#pragma unroll
                for (int i = 0; i < kPPT; ++i) a2[i][j] += hv[i] * w;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kPPT; ++i) {
        float h2[4], part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h2[j] = a2[i][j] > 0.0f ? a2[i][j] : 0.0f;
            part += a.w3[4 * uc + j] * h2[j];
        }
        // the score's 64 terms: the 16 threads of these positions, a fixed tree
        part += __shfl_xor(part, 8, 16);
        part += __shfl_xor(part, 4, 16);
        part += __shfl_xor(part, 2, 16);
        part += __shfl_xor(part, 1, 16);
        const int64_t p = p0 + kPPT * pr + i;
        if (p < a.seq_stride && a.map[p] >= 0) {
            if (uc == 0) {
                a.E[p] = a.b3 + part;
                a.H2[p * kLdH2 + 64] = 1.0f;
                a.H1[p * kLdH1 + 256] = 1.0f;
                a.X[p * kLdX + 192] = 1.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) a.H2[p * kLdH2 + 4 * uc + j] = h2[j];
#pragma unroll
            for (int j = 0; j < 16; ++j) a.H1[p * kLdH1 + 16 * uc + j] = L.hs[(kPPT * pr + i) * kHS + 16 * uc + j];
#pragma unroll
            for (int j = 0; j < 12; ++j) a.X[p * kLdX + 12 * uc + j] = L.xs[(kPPT * pr + i) * kXS + 12 * uc + j];
        }
    }
}

// Softmax of each sample over its scores, one wave per sample: p_j,
// dp_j = g . s_j and de_j = p_j (dp_j - sum_k p_k dp_k), reductions as
// fixed shuffle trees.
__global__ __launch_bounds__(256) void k_dinb_soft(DinBwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int32_t len = a.seq_lengths[b];
    const int L = len < a.max_len ? len : a.max_len;
    if (L <= 0) return;
    const int64_t off = a.seq_offsets[b];
    const float* g = a.gatt + b * 48;
    float e[2], dp[2];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = lane + 64 * u;
        e[u] = -INFINITY;
        dp[u] = 0.0f;
        if (j < L) {
            const int64_t p = off + j;
            e[u] = a.E[p];
            float d = 0.0f;
            for (int c = 0; c < 48; ++c) d += g[c] * a.S[p * 48 + c];
            dp[u] = d;
            m = fmaxf(m, e[u]);
        }
    }
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    float ex[2], den = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        ex[u] = lane + 64 * u < L ? expf(e[u] - m) : 0.0f;
        den += ex[u];
    }
    for (int d = 32; d >= 1; d >>= 1) den += __shfl_xor(den, d, 64);
    float pw[2], pdp = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        pw[u] = ex[u] / den;
        pdp += pw[u] * dp[u];
    }
    for (int d = 32; d >= 1; d >>= 1) pdp += __shfl_xor(pdp, d, 64);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = lane + 64 * u;
        if (j < L) {
            a.PW[off + j] = pw[u];
            a.DE[off + j] = pw[u] * (dp[u] - pdp);
        }
    }
}

// Backward of kPT positions: dz2 = de w3 where h2 > 0, dz1 = W2^T dz2 where
// h1 > 0, dx = W1^T dz1 (LDS-tiled as the forward), then each position's
// sequence-row gradient and its terms of the query gradient.
__global__ __launch_bounds__(256) void k_dinb_bwdt(DinBwdArgs a) {
    __shared__ __attribute__((aligned(16))) TileLds L;
    const int t = threadIdx.x, pr = t >> 4, uc = t & 15;
    const int64_t p0 = (int64_t)blockIdx.x * kPT;
    float* d2 = L.xs;                               // dz2 rows, stride 65
    for (int idx = t; idx < kPT * 64; idx += 256) {
        const int pi = idx >> 6, o = idx & 63;
        const int64_t p = p0 + pi;
        const bool ok = p < a.seq_stride && a.map[p] >= 0;
        const float v = (ok && a.H2[p * kLdH2 + o] > 0.0f) ? a.DE[p] * a.w3[o] : 0.0f;
        d2[pi * 65 + o] = v;
        if (ok && a.wgrad) a.DZ2[p * 64 + o] = v;
    }
    __syncthreads();
    // dz1: units 16 uc .. 16 uc + 15; W2 rows staged 16 at a time
    float acc[kPPT][16];
#pragma unroll
    for (int i = 0; i < kPPT; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
    for (int kb = 0; kb < 64; kb += 16) {
        for (int e = t; e < 16 * 256; e += 256) {
            const int kk = e >> 8, u = e & 255;
            L.wb[kk * 260 + u] = wload(a.w2, (int64_t)(kb + kk) * 256 + u, a.bf16);
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < 16; ++kk) {
            float dv[kPPT], wv[16];
#pragma unroll
            for (int i = 0; i < kPPT; ++i) dv[i] = d2[(kPPT * pr + i) * 65 + kb + kk];
            unpack16(L.wb + kk * 260 + 16 * uc, wv);
#pragma unroll
            for (int i = 0; i < kPPT; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[i][j] += dv[i] * wv[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kPPT; ++i) {
        const int64_t p = p0 + kPPT * pr + i;
        const bool ok = p < a.seq_stride && a.map[p] >= 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int u = 16 * uc + j;
            const float v = (ok && a.H1[p * kLdH1 + u] > 0.0f) ? acc[i][j] : 0.0f;
            L.hs[(kPPT * pr + i) * kHS + u] = v;
            if (ok && a.wgrad) a.DZ1[p * 256 + u] = v;
        }
    }
    __syncthreads();
    // dx: columns 12 uc .. 12 uc + 11; W1 rows staged 16 at a time (stride 196)
    float ax[kPPT][12];
#pragma unroll
    for (int i = 0; i < kPPT; ++i)
#pragma unroll
        for (int j = 0; j < 12; ++j) ax[i][j] = 0.0f;
    for (int kb = 0; kb < 256; kb += 16) {
        for (int e = t; e < 16 * 192; e += 256) {
            const int kk = e / 192, c = e - kk * 192;
            L.wb[kk * kXS + c] = wload(a.w1, (int64_t)(kb + kk) * 192 + c, a.bf16);
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < 16; ++kk) {
            float dv[kPPT], wv[12];
#pragma unroll
            for (int i = 0; i < kPPT; ++i) dv[i] = L.hs[(kPPT * pr + i) * kHS + kb + kk];
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const float4 x = *(const float4*)(L.wb + kk * kXS + 12 * uc + 4 * u);
                wv[4 * u] = x.x; wv[4 * u + 1] = x.y; wv[4 * u + 2] = x.z; wv[4 * u + 3] = x.w;
            }
#pragma unroll
            for (int i = 0; i < kPPT; ++i)
#pragma unroll
                for (int j = 0; j < 12; ++j) ax[i][j] += dv[i] * wv[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kPPT; ++i)
#pragma unroll
        for (int j = 0; j < 12; ++j) L.xs[(kPPT * pr + i) * kXS + 12 * uc + j] = ax[i][j];
    __syncthreads();
    for (int idx = t; idx < kPT * 48; idx += 256) {
        const int pi = idx / 48, c = idx - pi * 48;
        const int64_t p = p0 + pi;
        const int b = p < a.seq_stride ? a.map[p] : -1;
        if (b < 0) continue;
        const float* dx = L.xs + pi * kXS;
        const float sv = a.S[p * 48 + c];
        const float qv = a.query[(int64_t)b * a.query_ld + a.qcol[c >> 4] + (c & 15)];
        if (a.gs)
            a.gs[((int64_t)(c >> 4) * a.seq_stride + p) * REC_DIM + (c & 15)] =
                a.PW[p] * a.gatt[(int64_t)b * 48 + c] + dx[48 + c] - dx[96 + c] + qv * dx[144 + c];
        a.GQP[p * 48 + c] = dx[c] + dx[96 + c] + sv * dx[144 + c];
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
    for (int j = 0; j < L; ++j) s += a.GQP[(off + j) * 48 + c];
    a.gq[i] = s;
}

// Weight gradients: block (tile, split).  Tiles of 64 x 64 outputs of the
// three jobs in order; thread (tm, tn) owns the 4 x 4 outputs (m0 + 4 tm + i,
// n0 + 4 tn + j).  Blocks of kWB positions of A's and B's tile columns are
// staged in LDS by coalesced loads (positions without a valid flag, and
// columns past the edge, staged as zeros), then multiplied from LDS.
constexpr int kWT = 64;
constexpr int kWB = 32;

__device__ inline int wgrad_tiles(int job) {
    return ((kJobM[job] + kWT - 1) / kWT) * ((kJobN[job] + kWT - 1) / kWT);
}

__global__ __launch_bounds__(256) void k_dinb_wgrad(DinBwdArgs a, int64_t chunk) {
    __shared__ __attribute__((aligned(16))) float As[kWB][kWT];
    __shared__ __attribute__((aligned(16))) float Bs[kWB][kWT];
    const int t = threadIdx.x, tm = t >> 4, tn = t & 15;
    int tile = blockIdx.x, job = 0;
    for (; job < kJobs; ++job) {
        const int nt = wgrad_tiles(job);
        if (tile < nt) break;
        tile -= nt;
    }
    const int M = kJobM[job], N = kJobN[job];
    const int ntn = (N + kWT - 1) / kWT;
    const int m0 = (tile / ntn) * kWT, n0 = (tile % ntn) * kWT;
    const float* A = job == 0 ? a.DZ1 : job == 1 ? a.DZ2 : a.DE;
    const float* Bm = job == 0 ? a.X : job == 1 ? a.H1 : a.H2;
    const int64_t p0 = (int64_t)blockIdx.y * chunk;
    const int64_t p1 = p0 + chunk < a.seq_stride ? p0 + chunk : a.seq_stride;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    for (int64_t pb = p0; pb < p1; pb += kWB) {
#pragma unroll
        for (int u = 0; u < kWB * kWT / 256; ++u) {
            const int e = t + u * 256, r = e / kWT, c = e - r * kWT;
            const int64_t p = pb + r;
            const bool ok = p < p1 && a.map[p] >= 0;
            As[r][c] = (ok && m0 + c < M) ? A[p * M + m0 + c] : 0.0f;
            Bs[r][c] = (ok && n0 + c < N) ? Bm[p * N + n0 + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int r = 0; r < kWB; ++r) {
            const float4 av = *(const float4*)&As[r][4 * tm];
            const float4 bv = *(const float4*)&Bs[r][4 * tn];
            const float ai[4] = {av.x, av.y, av.z, av.w}, bj[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += ai[i] * bj[j];
        }
        __syncthreads();
    }
    int64_t base = 0;
    for (int j = 0; j < job; ++j) base += (int64_t)kJobM[j] * kJobN[j];
    float* out = a.part + (int64_t)blockIdx.y * a.part_stride + base;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * tm + i;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + 4 * tn + j;
            if (m < M && n < N) out[(int64_t)m * N + n] = acc[i][j];
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
    const int64_t cgrid = (a.seq_stride + 255) / 256;
    if (cgrid > 0) {
        hipLaunchKernelGGL(k_dinb_clear, dim3((unsigned)(cgrid < 65536 ? cgrid : 65536)), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(k_dinb_transpose, dim3((256 * 192 + 64 * 256 + 255) / 256), dim3(256), 0, s, a);
    const int64_t bgrid = (a.B + 255) / 256;
    hipLaunchKernelGGL(k_dinb_map, dim3((unsigned)(bgrid < 65536 ? bgrid : 65536)), dim3(256), 0, s, a);
    const int64_t tiles = (a.seq_stride + kPT - 1) / kPT;
    if (tiles > 0) hipLaunchKernelGGL(k_dinb_fwd, dim3((unsigned)tiles), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_dinb_soft, dim3((unsigned)((a.B + 3) / 4)), dim3(256), 0, s, a);
    if (tiles > 0) hipLaunchKernelGGL(k_dinb_bwdt, dim3((unsigned)tiles), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_dinb_gq, dim3((unsigned)((a.B * 48 + 255) / 256)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.wgrad) return e;
    int ntiles = 0;
    const int M[kJobs] = {256, 64, 1}, N[kJobs] = {kLdX, kLdH1, kLdH2};
    for (int j = 0; j < kJobs; ++j) ntiles += ((M[j] + kWT - 1) / kWT) * ((N[j] + kWT - 1) / kWT);
    const int64_t chunk = (a.seq_stride + kDinbSplits - 1) / kDinbSplits;
    hipLaunchKernelGGL(k_dinb_wgrad, dim3((unsigned)ntiles, kDinbSplits), dim3(256), 0, s, a, chunk);
    hipLaunchKernelGGL(k_dinb_reduce, dim3((unsigned)((a.part_stride + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
