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

constexpr int kDinbThreads = 256;
constexpr int kDinbSplits = 16;
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
        if (a.valid) a.valid[p] = 0;
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

// x of position j (thread t < 192 forms x[t]) into xs.
__device__ inline void form_x(const float* q, const float* sj, float* xs, int t) {
    if (t < 192) {
        const int blk = t / 48, c = t - blk * 48;
        const float qc = q[c], sc = sj[c];
        xs[t] = blk == 0 ? qc : blk == 1 ? sc : blk == 2 ? qc - sc : qc * sc;
    }
}

// h1 = relu(W1 x + b1) (thread t < 256 owns unit t), then h2 = relu(W2 h1 +
// b2): unit o = t & 63, its 256 inputs split over the four waves (quarter
// t >> 6), the four partial sums added in quarter order.  Ends with h1 and
// h2 in LDS, after a barrier.  part holds 256 floats of scratch.
__device__ inline void mlp_fwd(const DinBwdArgs& a, const float* xs, float* h1, float* h2,
                               float* part, int t) {
    {
        float acc = a.b1 ? a.b1[t] : 0.0f;
#pragma unroll 16
        for (int i = 0; i < 192; ++i) acc += a.w1t[i * 256 + t] * xs[i];
        h1[t] = acc > 0.0f ? acc : 0.0f;
    }
    __syncthreads();
    {
        const int o = t & 63, i0 = (t >> 6) * 64;
        float acc = 0.0f;
#pragma unroll 16
        for (int i = i0; i < i0 + 64; ++i) acc += a.w2t[i * 64 + o] * h1[i];
        part[t] = acc;
    }
    __syncthreads();
    if (t < 64) {
        const float acc = (a.b2 ? a.b2[t] : 0.0f) + ((part[t] + part[64 + t]) + (part[128 + t] + part[192 + t]));
        h2[t] = acc > 0.0f ? acc : 0.0f;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kDinbThreads) void k_dinb_sample(DinBwdArgs a) {
    __shared__ float q[48], g[48];
    __shared__ float sj[REC_MAX_SEQ_LEN][48];
    __shared__ float xs[192], h1[256], h2[64], dz2[64], dz1[256], dx[192], part[256];
    __shared__ float e[REC_MAX_SEQ_LEN], pw[REC_MAX_SEQ_LEN], dp[REC_MAX_SEQ_LEN], de[REC_MAX_SEQ_LEN];
    const int t = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int32_t len = a.seq_lengths[b];
    const int L = len < a.max_len ? len : a.max_len;
    if (L <= 0) {                                  // att = 0 whatever q: no gradient
        if (t < 48) a.gq[b * 48 + t] = 0.0f;
        return;
    }
    const int64_t off = a.seq_offsets[b];
    if (t < 48) {
        q[t] = a.query[b * a.query_ld + a.qcol[t / 16] + (t & 15)];
        g[t] = a.gatt[b * 48 + t];
    }
    for (int idx = t; idx < L * 48; idx += kDinbThreads) {
        const int j = idx / 48, c = idx - j * 48, f = c / 16;
        sj[j][c] = seq_elem(a.tabs[f], a.seq_values[(int64_t)f * a.seq_stride + off + j], c & 15);
    }
    __syncthreads();
    // scores
    for (int j = 0; j < L; ++j) {
        form_x(q, sj[j], xs, t);
        __syncthreads();
        mlp_fwd(a, xs, h1, h2, part, t);
        if (t == 0) {
            float s = a.b3;
            for (int o = 0; o < 64; ++o) s += a.w3[o] * h2[o];
            e[j] = s;
        }
        __syncthreads();
    }
    // softmax, dp_j = g . s_j, de_j (one thread: L <= 128, a fixed order)
    if (t < L) {
        float d = 0.0f;
        for (int c = 0; c < 48; ++c) d += g[c] * sj[t][c];
        dp[t] = d;
    }
    __syncthreads();
    if (t == 0) {
        float m = e[0];
        for (int j = 1; j < L; ++j) m = fmaxf(m, e[j]);
        float den = 0.0f;
        for (int j = 0; j < L; ++j) den += expf(e[j] - m);
        float pdp = 0.0f;
        for (int j = 0; j < L; ++j) {
            pw[j] = expf(e[j] - m) / den;
            pdp += pw[j] * dp[j];
        }
        for (int j = 0; j < L; ++j) de[j] = pw[j] * (dp[j] - pdp);
    }
    __syncthreads();
    float accq = 0.0f;
    for (int j = 0; j < L; ++j) {
        const int64_t pos = off + j;
        form_x(q, sj[j], xs, t);
        __syncthreads();
        mlp_fwd(a, xs, h1, h2, part, t);
        const float dej = de[j];
        if (t < 64) dz2[t] = h2[t] > 0.0f ? dej * a.w3[t] : 0.0f;
        if (a.valid) {                             // per-position rows for the weight gradients
            if (t < 192) a.X[pos * kLdX + t] = xs[t];
            a.H1[pos * kLdH1 + t] = h1[t];
            if (t < 64) a.H2[pos * kLdH2 + t] = h2[t];
            if (t == 0) {
                a.X[pos * kLdX + 192] = 1.0f;
                a.H1[pos * kLdH1 + 256] = 1.0f;
                a.H2[pos * kLdH2 + 64] = 1.0f;
                a.DE[pos] = dej;
            }
        }
        __syncthreads();
        {
            float acc = 0.0f;
#pragma unroll 16
            for (int o = 0; o < 64; ++o) acc += wload(a.w2, (int64_t)o * 256 + t, a.bf16) * dz2[o];
            dz1[t] = h1[t] > 0.0f ? acc : 0.0f;
        }
        if (a.valid && t < 64) a.DZ2[pos * 64 + t] = dz2[t];
        __syncthreads();
        if (a.valid) a.DZ1[pos * 256 + t] = dz1[t];
        if (t < 192) {
            float acc = 0.0f;
#pragma unroll 16
            for (int o = 0; o < 256; ++o) acc += wload(a.w1, (int64_t)o * 192 + t, a.bf16) * dz1[o];
            dx[t] = acc;
        }
        __syncthreads();
        if (t < 48) {
            const float sc = sj[j][t];
            accq += dx[t] + dx[96 + t] + sc * dx[144 + t];
            if (a.gs) {
                const float ds = pw[j] * g[t] + dx[48 + t] - dx[96 + t] + q[t] * dx[144 + t];
                a.gs[((int64_t)(t / 16) * a.seq_stride + pos) * REC_DIM + (t & 15)] = ds;
            }
        }
        if (a.valid && t == 0) a.valid[pos] = 1;
        __syncthreads();
    }
    if (t < 48) a.gq[b * 48 + t] = accq;
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
            const bool ok = p < p1 && a.valid[p];
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
    hipLaunchKernelGGL(k_dinb_sample, dim3((unsigned)a.B), dim3(kDinbThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.valid) return e;
    int tiles = 0;
    const int M[kJobs] = {256, 64, 1}, N[kJobs] = {kLdX, kLdH1, kLdH2};
    for (int j = 0; j < kJobs; ++j) tiles += ((M[j] + kWT - 1) / kWT) * ((N[j] + kWT - 1) / kWT);
    const int64_t chunk = (a.seq_stride + kDinbSplits - 1) / kDinbSplits;
    hipLaunchKernelGGL(k_dinb_wgrad, dim3((unsigned)tiles, kDinbSplits), dim3(256), 0, s, a, chunk);
    hipLaunchKernelGGL(k_dinb_reduce, dim3((unsigned)((a.part_stride + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
