// The DLRM forward around the interaction: per-table EmbeddingBags of width
// d (sum or mean), the bottom MLP on the dense features, the interaction and
// the top MLP.
//
// Pages: DLRM essay (wmrh.cn/news/12459) §2.3 (four layers with separate
// duties: a bottom MLP brings the dense features to the embedding width,
// EmbeddingBags pool each sparse feature, the interaction layer takes the dot
// product of every pair, one triangle only, and a top MLP turns the dot
// products into the prediction), §3.2 (a bag pools by sum or by mean), §3.3
// and §4.2 (the widths: bottom n_dense -> 128 -> d with ReLU after both
// layers; the interaction's (S+1)(S+2)/2 outputs, j running from i; top ->
// 128 -> 64 -> 1 with ReLU, ReLU and a sigmoid).
//
// Two launches, fp32 throughout:
//   1. k_dlrm_embed: its first blocks pool the bags straight into the
//      interaction input z [B][S+1][d] (vector t+1 of sample b is bag (t, b)),
//      eight lanes per bag, each lane holding d/32 float4 columns of a row,
//      so one wave instruction reads eight rows' worth of 128-byte runs; ids
//      are loaded four at a time ahead of their rows.  The remaining blocks
//      run the bottom MLP for 32 samples each (activations in LDS) into
//      vector 0 of z.
//   2. k_dlrm_top: 16 samples per workgroup: their z rows are staged in LDS,
//      every pair (i <= j) is one thread's dot product over d, and the top
//      MLP runs on the pairs in LDS; the logit and the probability go out.
#include "rec_internal.h"

namespace rec {
namespace {

constexpr int kBagLanes = 8;                 // lanes per bag
constexpr int kIdRound = 4;                  // ids of a bag loaded per round
constexpr int kBottomSamples = 32;
constexpr int kTopSamples = 16;

// One dense layer over activations in LDS: out[r][o] = act(b[o] + sum_i
// W[o][i] in[r][i]) for r < rows, o < nout; W is [nout][nin] in global memory
// (torch's Linear layout), read through the caches.
__device__ inline void dense_layer(const float* in, int in_stride, int nin, const float* __restrict__ W,
                                   const float* __restrict__ bias, int nout, float* out, int out_stride,
                                   int rows, bool relu) {
    for (int idx = threadIdx.x; idx < rows * nout; idx += blockDim.x) {
        const int r = idx / nout, o = idx - r * nout;
        const float* w = W + (int64_t)o * nin;
        const float* x = in + r * in_stride;
        float acc = bias[o];
        for (int i = 0; i < nin; ++i) acc = fmaf(w[i], x[i], acc);
        out[r * out_stride + o] = relu ? fmaxf(acc, 0.f) : acc;
    }
}

template <int NF>
__device__ inline void dlrm_bags(const DlrmArgs& a, int64_t blk) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nbw = (a.B + 31) / 32;                  // 32-sample chunks per table
    const int t = (int)(blk / nbw);
    const int64_t b = (blk % nbw) * 32 + wave * kBagLanes + (lane >> 3);
    const int c = lane & 7;
    const bool live = b < a.B;
    const int64_t bag = (int64_t)t * a.B + (live ? b : a.B - 1);
    const TabDev tab = a.tab[t];
    const int32_t len = live ? a.lengths[bag] : 0;
    const int64_t off = a.offsets[bag];
    const int d = a.dim;
    float4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; __ballot(j0 < len) != 0; j0 += kIdRound) {
        int64_t row[kIdRound];
#pragma unroll
        for (int u = 0; u < kIdRound; ++u) {
            const int64_t raw = a.values[len > 0 ? off + min(j0 + u, len - 1) : 0];
            row[u] = floor_mod_magic(raw, tab.rows, tab.magic, tab.shift);
        }
        float4 v[kIdRound][NF];
#pragma unroll
        for (int u = 0; u < kIdRound; ++u) {
            const float4* src = (const float4*)(tab.values + row[u] * d) + c;
#pragma unroll
            for (int f = 0; f < NF; ++f) v[u][f] = src[8 * f];
        }
#pragma unroll
        for (int u = 0; u < kIdRound; ++u) {
            const bool use = j0 + u < len;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                acc[f].x += use ? v[u][f].x : 0.f;
                acc[f].y += use ? v[u][f].y : 0.f;
                acc[f].z += use ? v[u][f].z : 0.f;
                acc[f].w += use ? v[u][f].w : 0.f;
            }
        }
    }
    if (!live) return;
    if (a.mode[t] == REC_POOL_MEAN && len > 0) {
        const float inv = 1.f / (float)len;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            acc[f].x *= inv;
            acc[f].y *= inv;
            acc[f].z *= inv;
            acc[f].w *= inv;
        }
    }
    float4* o = (float4*)(a.z + (b * (int64_t)(a.S + 1) + 1 + t) * d) + c;
#pragma unroll
    for (int f = 0; f < NF; ++f) o[8 * f] = acc[f];
}

__device__ inline void dlrm_bottom(const DlrmArgs& a, int64_t blk) {
    __shared__ float s_x[kBottomSamples * kDlrmMaxDense];
    __shared__ float s_h[kBottomSamples * 128];
    const int64_t b0 = blk * kBottomSamples;
    const int rows = (int)min((int64_t)kBottomSamples, a.B - b0);
    for (int idx = threadIdx.x; idx < rows * a.n_dense; idx += blockDim.x)
        s_x[idx] = a.dense[b0 * a.n_dense + idx];
    __syncthreads();
    dense_layer(s_x, a.n_dense, a.n_dense, a.wb1, a.bb1, 128, s_h, 128, rows, true);
    __syncthreads();
    const int F = a.S + 1;
    for (int idx = threadIdx.x; idx < rows * a.dim; idx += blockDim.x) {
        const int r = idx / a.dim, o = idx - r * a.dim;
        const float* w = a.wb2 + (int64_t)o * 128;
        const float* x = s_h + r * 128;
        float acc = a.bb2[o];
        for (int i = 0; i < 128; ++i) acc = fmaf(w[i], x[i], acc);
        a.z[(b0 + r) * (int64_t)F * a.dim + o] = fmaxf(acc, 0.f);
    }
}

template <int NF>
__global__ __launch_bounds__(256) void k_dlrm_embed(const DlrmArgs a, int64_t nbag_blocks) {
    if ((int64_t)blockIdx.x < nbag_blocks) dlrm_bags<NF>(a, blockIdx.x);
    else dlrm_bottom(a, blockIdx.x - nbag_blocks);
}

__global__ __launch_bounds__(256) void k_dlrm_top(const DlrmArgs a) {
    __shared__ __attribute__((aligned(16))) float s_z[kTopSamples * kDlrmMaxZ];
    __shared__ float s_i[kTopSamples * kDlrmMaxPairs];
    __shared__ float s_t1[kTopSamples * 128];
    __shared__ float s_t2[kTopSamples * 64];
    __shared__ uint16_t s_pi[kDlrmMaxPairs], s_pj[kDlrmMaxPairs];
    const int F = a.S + 1, d = a.dim, zw = F * d;
    const int np = F * (F + 1) / 2;
    const int64_t b0 = (int64_t)blockIdx.x * kTopSamples;
    const int rows = (int)min((int64_t)kTopSamples, a.B - b0);
    // the pair list in row order: (0,0), (0,1), ..., (F-1,F-1)
    if (threadIdx.x < F) {
        const int i = threadIdx.x;
        int p = i * F - i * (i - 1) / 2;
        for (int j = i; j < F; ++j, ++p) {
            s_pi[p] = (uint16_t)i;
            s_pj[p] = (uint16_t)j;
        }
    }
    const float4* src = (const float4*)(a.z + b0 * (int64_t)zw);
    float4* dst = (float4*)s_z;
    for (int idx = threadIdx.x; idx < rows * zw / 4; idx += blockDim.x) dst[idx] = src[idx];
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows * np; idx += blockDim.x) {
        const int r = idx / np, p = idx - r * np;
        const float* zi = s_z + r * zw + s_pi[p] * d;
        const float* zj = s_z + r * zw + s_pj[p] * d;
        float acc = 0.f;
        for (int k = 0; k < d; ++k) acc = fmaf(zi[k], zj[k], acc);
        s_i[r * np + p] = acc;
        if (a.inter) a.inter[(b0 + r) * np + p] = acc;
    }
    __syncthreads();
    dense_layer(s_i, np, np, a.wt1, a.bt1, 128, s_t1, 128, rows, true);
    __syncthreads();
    dense_layer(s_t1, 128, 128, a.wt2, a.bt2, 64, s_t2, 64, rows, true);
    __syncthreads();
    if (threadIdx.x < rows) {
        const int r = threadIdx.x;
        float l = a.bt3;
        for (int i = 0; i < 64; ++i) l = fmaf(a.wt3[i], s_t2[r * 64 + i], l);
        a.logit[b0 + r] = l;
        if (a.prob) a.prob[b0 + r] = 1.f / (1.f + expf(-l));
    }
}

}  // namespace

hipError_t launch_dlrm_fwd(const DlrmArgs& a, hipStream_t s) {
    const int64_t nbag_blocks = (int64_t)a.S * ((a.B + 31) / 32);
    const int64_t nbottom = (a.B + kBottomSamples - 1) / kBottomSamples;
    const dim3 g1((unsigned)(nbag_blocks + nbottom)), blk(256);
    switch (a.dim / 32) {
        case 1: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<1>, g1, blk, 0, s, a, nbag_blocks); break;
        case 2: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<2>, g1, blk, 0, s, a, nbag_blocks); break;
        case 3: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<3>, g1, blk, 0, s, a, nbag_blocks); break;
        case 4: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<4>, g1, blk, 0, s, a, nbag_blocks); break;
        case 5: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<5>, g1, blk, 0, s, a, nbag_blocks); break;
        case 6: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<6>, g1, blk, 0, s, a, nbag_blocks); break;
        case 7: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<7>, g1, blk, 0, s, a, nbag_blocks); break;
        default: REC_LAUNCH(REC_TIME_DLRM_EMBED, k_dlrm_embed<8>, g1, blk, 0, s, a, nbag_blocks); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)((a.B + kTopSamples - 1) / kTopSamples));
    REC_LAUNCH(REC_TIME_DLRM_TOP, k_dlrm_top, g2, blk, 0, s, a);
    return hipGetLastError();
}

}  // namespace rec
