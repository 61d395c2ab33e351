// DLRM dot-product interaction: per sample, the dot product of every pair
// i <= j of its F vectors of width d, row by row.
//
// Pages: DLRM essay (wmrh.cn/news/12459) §2.3 (the interaction layer takes
// the bottom MLP's output and every pooled embedding and emits their pairwise
// dot products, one triangle only), §4.2 (its code runs j from i, so the
// diagonal is included), §3.1 (the measured case: 217 features, width 96).
//
// On the matrix cores.  A sample's vectors form a small matrix Z [F][d] and
// the output is the upper triangle of Z Z^T, so each 32 x 32 tile of it is a
// run of v_mfma_f32_32x32x2f32 over d (fp32 in, fp32 accumulate; the fp32
// matrix rate is twice the unpacked fp32 vector rate, and the 32 x 32 shape
// reads half the LDS operand bytes per flop of the 16 x 16 one).  One
// workgroup per CU, persistent over samples: Z is staged in LDS, rows padded
// to a multiple of 32 with zeros, with a row stride that spreads the rows of
// an operand read over the banks; the next sample's Z rides in registers
// while the current one is multiplied.  The T(T+1)/2 tile pairs I <= J of the
// T = ceil(F / 32) row tiles are dealt to the eight waves in turn.  Both
// operands want row m of their tile in lane (m, h) at lane half h's K
// positions; giving half h the contiguous half [h d/2, (h+1) d/2) of d (any
// K order is right when both operands use it) lets a lane read four K steps
// with one 16-byte read, feeding two independent accumulators.
#include "rec_internal.h"
#include "rec_mfma.h"

namespace rec {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDlrmWaves = 8;                  // two per SIMD: one wave's LDS waits hide behind the other's products
// float4s per thread that hold a whole staged Z (the LDS stage's size)
constexpr int kDlrmPrefetch = kDlrmMaxLdsFloats / (4 * 64 * kDlrmWaves);

__global__ __launch_bounds__(64 * kDlrmWaves) void k_dlrm_interact(const float* __restrict__ z, int64_t B,
                                                                   int F, int d, int stride,
                                                                   float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) float s_z[kDlrmMaxLdsFloats];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 31, h = lane >> 5;
    const int T = (F + 31) / 32;
    const int dh = d / 2;                       // a lane half's share of d (a multiple of 8)
    const int nv = d / 4;                       // float4s per row
    const int64_t npairs = (int64_t)F * (F + 1) / 2;
    const int ntile = T * (T + 1) / 2;
    // Z of the next sample travels in registers while the current one is
    // multiplied: thread t holds float4 t + q*256 of it (zeros past row F)
    const int nvec = 32 * T * nv;
    float4 pre[kDlrmPrefetch];
    auto fetch = [&](int64_t bs) {
        const float4* src = (const float4*)(z + bs * (int64_t)F * d);
#pragma unroll
        for (int q = 0; q < kDlrmPrefetch; ++q) {
            const int v = threadIdx.x + q * 64 * kDlrmWaves;
            pre[q] = (v < nvec && v / nv < F) ? src[v] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    if ((int64_t)blockIdx.x < B) fetch(blockIdx.x);
    for (int64_t b = blockIdx.x; b < B; b += gridDim.x) {
#pragma unroll
        for (int q = 0; q < kDlrmPrefetch; ++q) {
            const int v = threadIdx.x + q * 64 * kDlrmWaves;
            if (v < nvec) {
                const int r = v / nv, c = v - r * nv;
                *(float4*)(s_z + r * stride + 4 * c) = pre[q];
            }
        }
        __syncthreads();
        if (b + gridDim.x < B) fetch(b + gridDim.x);
        for (int t = wave; t < ntile; t += kDlrmWaves) {
            int I = 0, rem = t;                     // tile pair t, row by row
            while (rem >= T - I) {
                rem -= T - I;
                ++I;
            }
            const int J = I + rem;
            const float* ra = s_z + (I * 32 + m) * stride + h * dh;
            const float* rb = s_z + (J * 32 + m) * stride + h * dh;
            f32x16 acc0 = {}, acc1 = {};
            // the next K step's operands are read before this step's products
            float4 av = *(const float4*)ra;
            float4 bv = *(const float4*)rb;
            for (int k = 0; k < dh; k += 4) {
                const int kn = k + 4 < dh ? k + 4 : k;
                const float4 an = *(const float4*)(ra + kn);
                const float4 bn = *(const float4*)(rb + kn);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bv.x, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bv.y, acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bv.z, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bv.w, acc1, 0, 0, 0);
                av = an;
                bv = bn;
            }
            const f32x16 sum = acc0 + acc1;
            // register r of lane (m, h) holds row 8 (r / 4) + 4 h + r % 4 of
            // the tile, column m
            const int j = J * 32 + m;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = I * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (i < F && j < F && i <= j) {
                    const int64_t row = (int64_t)i * F - (int64_t)i * (i - 1) / 2;   // pairs before row i
                    out[b * npairs + row + (j - i)] = sum[r];
                }
            }
        }
        __syncthreads();                        // before the next sample overwrites Z
    }
}

}  // namespace

int dlrm_stride(int d) { return (d / 4) % 2 == 0 ? d + 4 : d; }

hipError_t launch_dlrm_interact(const float* z, int64_t B, int F, int d, float* out, int num_cus,
                                hipStream_t s) {
    const int64_t grid = B < num_cus ? B : num_cus;
    REC_LAUNCH(REC_TIME_DLRM_INTERACT, k_dlrm_interact, dim3((unsigned)grid), dim3(64 * kDlrmWaves), 0, s, z,
               B, F, d, dlrm_stride(d), out);
    return hipGetLastError();
}

}  // namespace rec
