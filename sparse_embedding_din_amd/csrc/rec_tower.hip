// Deep tower and final MLP of MultiTowerDIN: the rest of the forward after
// the sparse part.
//
// Pages: "MultiTowerDIN：当前现状分析" §4.4 (compute graph: the deep MLP
// 512 -> 256 -> 128 over the pooled deep features, the concat of its [B,128]
// output with the [B,48] attention output into [B,176], the final MLP
// 176 -> 64 -> 1); "MultiTowerDIN：集成 DynamicEmb" §7 (model config: tower
// hidden units [512, 256, 128], final hidden units [64], binary cross entropy,
// so the last unit is a logit).
//
// bf16 path: one workgroup of eight waves (two per SIMD: one wave alone
// issues a matrix-core product only every other slot) carries 16G samples
// (G groups of 16) through all five layers and the activations never leave
// the chip.  The waves split each layer's output units (wave w owns an
// eighth of the 16-unit tiles; the last layer's four tiles are taken by
// waves 0-3 and, redundantly, by 4-7), so every weight is read once per
// workgroup, straight from global memory into registers as the matrix-core
// A operand, and the G sample groups share each weight fragment.  Each layer's results go through
// bias, ReLU and bf16 rounding into LDS in the order the next layer's B
// operand wants them: per K-step of 32 and sample group, 64 lanes x 16 bytes
// in lane order, so every LDS read and write of a wave is one contiguous
// KiB (no bank conflicts, no padding).  Inside a K-step the order of K is
// free as long as both operands agree: a K-step of a hidden input is the
// pair of result tiles (2c, 2c+1), lane (m, g) holding units 4g..4g+3 of
// each -- exactly the accumulator values that lane already has -- and the
// packed weights carry the same order.
//
// At a batch of a few thousand, each CU carries one workgroup and must still
// receive all 600 KB of weights: the kernel is bound by that stream from L2,
// not by the matrix cores.  So each wave reads its fragments as one stream
// through all four layers with a fixed number in flight, and the stream does
// not drain at a layer's end: its loads run on through the epilogue and the
// barrier into the next layer.
//
// fp32 path: the same dataflow with fp32 activations in LDS and one output
// (sample, unit) per thread per pass, plain fp32 fused multiply-adds in
// column order; it exists for exactness checks at small sizes.
#include "rec_internal.h"
#include "rec_mfma.h"

#ifndef TOWER_STREAM
#define TOWER_STREAM 16
#endif
#ifndef TOWER_BIG_B
#define TOWER_BIG_B 16384
#endif

namespace rec {
namespace {

constexpr int kM = kTowerSamples;        // samples per workgroup of the fp32 path
constexpr int kWaves = 8;                // bf16 path
constexpr int kF32Threads = 256;         // fp32 path

// The weight stream of a wave: layer l has kNK[l] K-steps of kNT[l] tiles
// (fragments: one 16 x 32 bf16 tile, 16 bytes per lane), 78 fragments per
// wave in (layer, K-step, tile) order.
constexpr int kNT[4] = {4, 2, 1, 1};
constexpr int kNK[4] = {8, 16, 8, 6};
constexpr int kLdw[4] = {256, 512, 256, 176};
constexpr int kRowsPerWave[4] = {64, 32, 16, 16};
__host__ __device__ constexpr int layer_base(int l) {
    return l == 0 ? 0 : layer_base(l - 1) + kNT[l - 1] * kNK[l - 1];
}
constexpr int kFrags = layer_base(4);
constexpr int kDeepFrags = layer_base(3);       // layers 1-3, own to each wave
// packed image: [wave][72 deep fragments], then [last-layer tile][6]
static_assert((kWaves * kDeepFrags + 4 * kNK[3]) * 1024 == REC_TOWER_PACKED_BYTES,
              "packed tower image size");
// the tile (of 16 units) of layer l a wave's tile t is
__host__ __device__ constexpr int tile_of(int l, int w, int t) {
    return l == 3 ? (w & 3) : (kRowsPerWave[l] / 16) * w + t;
}
__host__ __device__ constexpr int layer_of(int f) {
    return f < layer_base(1) ? 0 : f < layer_base(2) ? 1 : f < layer_base(3) ? 2 : 3;
}

// The 8 K elements lane group g holds in K-step c of layer l, as two runs of
// 4 weight columns starting at *c0 and *c1.  Inputs staged from memory (the
// deep input; att, K-steps 4 and 5 of the last layer) are in natural order,
// 8 consecutive columns per lane group; a hidden input is in result-tile
// order (units 4g.. of tile 2c, then of tile 2c+1).  Columns at or past the
// matrix's width (the last layer's K is 176, padded to 192) read as zero.
__host__ __device__ inline void frag_cols(int l, int c, int g, int* c0, int* c1) {
    if (l == 0 || (l == 3 && c >= 4)) {
        *c0 = 32 * c + 8 * g;
        *c1 = *c0 + 4;
    } else {
        *c0 = 32 * c + 4 * g;
        *c1 = 32 * c + 16 + 4 * g;
    }
}

// Where wave w's fragments come from.  Packed (rec_tower_pack_mlp): the
// wave's fragments are two contiguous runs (its 72 deep-tower fragments, and
// the 6 of its last-layer tile), each fragment 64 lanes x 16 B in lane
// order, so every load is 1 KiB of consecutive memory.  Plain: lane (m, g)
// of K-step c, tile t reads row 16 tile_of(l, w, t) + m of the row-major
// matrix at the columns frag_cols gives; those 64 lanes touch 16 rows, and
// the loads run about twice as slow.
struct WStream {
    const uint4* deep;      // packed: the wave's first fragment
    const uint4* last;      // packed: its last-layer tile's first fragment
    const uint16_t* W[4];
    int w;
};

template <bool kPacked>
__device__ inline uint4 load_frag(const WStream& S, int f, int lane) {
    if (kPacked)
        return f < kDeepFrags ? S.deep[f * 64 + lane] : S.last[(f - kDeepFrags) * 64 + lane];
    const int l = layer_of(f), r = f - layer_base(l), c = r / kNT[l], t = r % kNT[l];
    const int row = 16 * tile_of(l, S.w, t) + (lane & 15);
    int c0, c1;
    frag_cols(l, c, lane >> 4, &c0, &c1);
    if (c0 >= kLdw[l]) return make_uint4(0u, 0u, 0u, 0u);
    const uint16_t* p = S.W[l] + (int64_t)row * kLdw[l];
    const uint2 lo = *(const uint2*)(p + c0), hi = *(const uint2*)(p + c1);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Accumulators start from the bias of their rows (the first product's C).
template <int NT, int G>
__device__ inline void bias_init(f32x4 (&acc)[NT][G], const float* __restrict__ bias, int row0,
                                 int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const f32x4 b = *(const f32x4*)(bias + row0 + 16 * t + 4 * (lane >> 4));
#pragma unroll
        for (int s = 0; s < G; ++s) acc[t][s] = b;
    }
}

// Layer L: acc[t][s] += W(tile t) x in(group s) over its K-steps; `in` holds
// the layer's input as [K-step][group][lane] 16-byte B operands, read one
// K-step ahead.  Each A fragment, once used, is replaced in the ring by the
// one D fragments further down the stream.
template <bool kPacked, int L, int D, int G>
__device__ inline void layer_mma(f32x4 (&acc)[kNT[L]][G], uint4 (&ring)[D], const WStream& S,
                                 const uint4* in, int lane) {
    constexpr int NT = kNT[L], NK = kNK[L], F0 = layer_base(L);
    bf16x8 x[2][G];
#pragma unroll
    for (int s = 0; s < G; ++s) x[0][s] = __builtin_bit_cast(bf16x8, in[s * 64 + lane]);
#pragma unroll
    for (int c = 0; c < NK; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        const int cur = c & 1;
        if (c + 1 < NK) {
#pragma unroll
            for (int s = 0; s < G; ++s)
                x[cur ^ 1][s] = __builtin_bit_cast(bf16x8, in[((c + 1) * G + s) * 64 + lane]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int s = 0; s < G; ++s)
                acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, ring[(F0 + c * NT + t) % D]), x[cur][s], acc[t][s],
                    0, 0, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int f = F0 + c * NT + t;
            if (f + D < kFrags) ring[f % D] = load_frag<kPacked>(S, f + D, lane);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// ReLU + bf16 of a wave's result tiles into the next layer's B operands:
// tiles (2j, 2j+1) form K-step c0 + j, lane (m, g) writing its 4 + 4 values.
template <int NT, int G>
__device__ inline void store_act(const f32x4 (&acc)[NT][G], uint4* out, int c0, int lane) {
#pragma unroll
    for (int j = 0; j < NT / 2; ++j)
#pragma unroll
        for (int s = 0; s < G; ++s) {
            const f32x4 u = acc[2 * j][s], v = acc[2 * j + 1][s];
            out[((c0 + j) * G + s) * 64 + lane] =
                make_uint4(relu_pk_bf16(u[0], u[1]), relu_pk_bf16(u[2], u[3]),
                           relu_pk_bf16(v[0], v[1]), relu_pk_bf16(v[2], v[3]));
        }
}

// A single tile (2c + h) is half of K-step c: its 4 values per lane go to
// the low (h = 0) or high (h = 1) 8 bytes of the lane's operand.
template <int G>
__device__ inline void store_act_half(const f32x4 (&acc)[1][G], uint4* out, int c, int h,
                                      int lane) {
#pragma unroll
    for (int s = 0; s < G; ++s) {
        const f32x4 u = acc[0][s];
        uint2* q = (uint2*)&out[(c * G + s) * 64 + lane] + h;
        *q = make_uint2(relu_pk_bf16(u[0], u[1]), relu_pk_bf16(u[2], u[3]));
    }
}

__device__ inline uint4 pack_bf16x8(float4 a, float4 b) {
    bf16x2 p[4];
    p[0][0] = (__bf16)a.x;
    p[0][1] = (__bf16)a.y;
    p[1][0] = (__bf16)a.z;
    p[1][1] = (__bf16)a.w;
    p[2][0] = (__bf16)b.x;
    p[2][1] = (__bf16)b.y;
    p[3][0] = (__bf16)b.z;
    p[3][1] = (__bf16)b.w;
    return make_uint4(__builtin_bit_cast(uint32_t, p[0]), __builtin_bit_cast(uint32_t, p[1]),
                      __builtin_bit_cast(uint32_t, p[2]), __builtin_bit_cast(uint32_t, p[3]));
}

__device__ inline float logistic(float l) { return 1.f / (1.f + expf(-l)); }

// G groups of 16 samples per workgroup share every weight fragment: 32
// samples while the batch is small enough that one workgroup per CU is all
// the machine gets, 64 once there are enough to fill every CU twice over
// (each CU then takes half as many passes over the weights).
template <bool kPacked, int D, int G>
__global__ __launch_bounds__(64 * kWaves) void k_towers_bf16(const TowerArgs a) {
    constexpr int M = 16 * G;
    __shared__ uint4 s_x[8 * G * 64];     // deep input, then the layer-2 results
    __shared__ uint4 s_h[16 * G * 64];    // layer-1 results
    __shared__ uint4 s_z[6 * G * 64];     // [deep out (K-steps 0-3), att (4-5)]
    __shared__ float s_part[4][M];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t b0 = (int64_t)blockIdx.x * M;

    // Stage the deep input (first 256 pooled columns, K-steps 0-7) and att
    // (K-steps 4-5 of the last layer) as B operands: operand (c, s, lane
    // (m, g)) is sample 16s + m, columns 32c + 8g .. + 7.  Samples past B
    // are read at row B-1 and zeroed.  These loads go out before the weight
    // stream's first ones, so that waiting for them does not wait for the
    // weights.
    constexpr int NTH = 64 * kWaves;
    constexpr int XU = 8 * G * 64 / NTH, AU = (2 * G * 64 + NTH - 1) / NTH;   // operands per thread
    float4 xv[XU][2], av[AU][2];
#pragma unroll
    for (int j = 0; j < XU; ++j) {
        const int u = tid + NTH * j, ln = u & 63, cs = u >> 6, c = cs / G, s = cs % G;
        const int64_t b = min(b0 + 16 * s + (ln & 15), a.B - 1);
        const float4* p = (const float4*)(a.pooled + b * a.pooled_ld + 32 * c + 8 * (ln >> 4));
        xv[j][0] = p[0];
        xv[j][1] = p[1];
    }
#pragma unroll
    for (int j = 0; j < AU; ++j) {
        // operands past the att K-steps (when there are fewer than threads)
        // read a valid row and are never written
        const int u = min(tid + NTH * j, 2 * G * 64 - 1), ln = u & 63, cs = u >> 6, c = cs / G,
                  s = cs % G;
        const int64_t b = min(b0 + 16 * s + (ln & 15), a.B - 1);
        const int col = min(32 * c + 8 * (ln >> 4), 40);
        const float4* p = (const float4*)(a.att + b * 48 + col);
        av[j][0] = p[0];
        av[j][1] = p[1];
    }
    WStream S;
    S.deep = (const uint4*)a.w[0] + (int64_t)w * kDeepFrags * 64;
    S.last = (const uint4*)a.w[0] + (int64_t)(kWaves * kDeepFrags + (w & 3) * kNK[3]) * 64;
#pragma unroll
    for (int l = 0; l < 4; ++l) S.W[l] = (const uint16_t*)a.w[l];
    S.w = w;
    uint4 ring[D];
#pragma unroll
    for (int f = 0; f < D; ++f) ring[f] = load_frag<kPacked>(S, f, lane);

    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < XU; ++j) {
        const int u = tid + NTH * j, ln = u & 63, s = (u >> 6) % G;
        const bool live = b0 + 16 * s + (ln & 15) < a.B;
        s_x[u] = pack_bf16x8(live ? xv[j][0] : zero4, live ? xv[j][1] : zero4);
    }
#pragma unroll
    for (int j = 0; j < AU; ++j) {
        const int u = tid + NTH * j, ln = u & 63, cs = u >> 6, c = cs / G, s = cs % G;
        const bool live = b0 + 16 * s + (ln & 15) < a.B && 32 * c + 8 * (ln >> 4) < 48;
        if (u < 2 * G * 64)
            s_z[4 * G * 64 + u] = pack_bf16x8(live ? av[j][0] : zero4, live ? av[j][1] : zero4);
    }
    f32x4 acc1[4][G];
    bias_init<4, G>(acc1, a.b[0], 64 * w, lane);
    __syncthreads();

    // layer 1: 256 -> 512, wave w owns units 64w .. 64w+63 (K-steps 2w, 2w+1)
    layer_mma<kPacked, 0, D, G>(acc1, ring, S, s_x, lane);
    store_act<4, G>(acc1, s_h, 2 * w, lane);
    f32x4 acc2[2][G];
    bias_init<2, G>(acc2, a.b[1], 32 * w, lane);
    __syncthreads();

    // layer 2: 512 -> 256, units 32w ..; its results replace the deep input
    layer_mma<kPacked, 1, D, G>(acc2, ring, S, s_h, lane);
    store_act<2, G>(acc2, s_x, w, lane);
    f32x4 acc3[1][G];
    bias_init<1, G>(acc3, a.b[2], 16 * w, lane);
    __syncthreads();

    // layer 3: 256 -> 128, units 16w ..: the deep tower's output
    layer_mma<kPacked, 2, D, G>(acc3, ring, S, s_x, lane);
    if (a.deep_out) {
        const int m = lane & 15, g = lane >> 4;
#pragma unroll
        for (int s = 0; s < G; ++s) {
            const int64_t b = b0 + 16 * s + m;
            if (b < a.B) {
                const f32x4 v = acc3[0][s];
                *(float4*)(a.deep_out + b * 128 + 16 * w + 4 * g) =
                    make_float4(fmaxf(v[0], 0.f), fmaxf(v[1], 0.f), fmaxf(v[2], 0.f), fmaxf(v[3], 0.f));
            }
        }
    }
    store_act_half<G>(acc3, s_z, w >> 1, w & 1, lane);
    f32x4 acc4[1][G];
    bias_init<1, G>(acc4, a.b[3], 16 * (w & 3), lane);
    __syncthreads();

    // layer 4: [deep, att] (176, zero-padded to 192) -> 64, units 16 (w & 3) ..
    layer_mma<kPacked, 3, D, G>(acc4, ring, S, s_z, lane);
    // the logit: wo . relu(layer 4) + bo, a partial sum over each of waves
    // 0-3's units
    if (w < 4) {
        const int m = lane & 15, g = lane >> 4;
        const f32x4 wo = *(const f32x4*)(a.wo + 16 * w + 4 * g);
#pragma unroll
        for (int s = 0; s < G; ++s) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) p += fmaxf(acc4[0][s][i], 0.f) * wo[i];
            p += __shfl_xor(p, 16, 64);
            p += __shfl_xor(p, 32, 64);
            if (g == 0) s_part[w][16 * s + m] = p;
        }
    }
    __syncthreads();
    if (tid < M) {
        const int64_t b = b0 + tid;
        if (b < a.B) {
            const float l = a.bo + s_part[0][tid] + s_part[1][tid] + s_part[2][tid] + s_part[3][tid];
            a.logit[b] = l;
            if (a.prob) a.prob[b] = logistic(l);
        }
    }
}

// out[r][o] = relu(bias[o] + sum_i W[o][i] in[r][i]) for the kM rows, fp32.
__device__ inline void dense_f32(const float* in, int nin, const float* __restrict__ W,
                                 const float* __restrict__ bias, int nout, float* out, int ostr) {
    for (int idx = threadIdx.x; idx < kM * nout; idx += kF32Threads) {
        const int r = idx / nout, o = idx % nout;
        float acc = bias[o];
        const float* wr = W + (int64_t)o * nin;
        const float* x = in + r * nin;
        for (int i = 0; i < nin; ++i) acc = fmaf(wr[i], x[i], acc);
        out[r * ostr + o] = fmaxf(acc, 0.f);
    }
}

__global__ __launch_bounds__(kF32Threads) void k_towers_f32(const TowerArgs a) {
    __shared__ float s_x[kM * 256];     // deep input, then layer 2
    __shared__ float s_h[kM * 512];     // layer 1, then layer 4
    __shared__ float s_z[kM * 176];     // [deep out, att]
    const int tid = threadIdx.x;
    const int64_t b0 = (int64_t)blockIdx.x * kM;
    for (int idx = tid; idx < kM * 256; idx += kF32Threads) {
        const int r = idx >> 8, c = idx & 255;
        const int64_t b = b0 + r;
        s_x[idx] = b < a.B ? a.pooled[b * a.pooled_ld + c] : 0.f;
    }
    for (int idx = tid; idx < kM * 48; idx += kF32Threads) {
        const int r = idx / 48, c = idx % 48;
        const int64_t b = b0 + r;
        s_z[r * 176 + 128 + c] = b < a.B ? a.att[b * 48 + c] : 0.f;
    }
    __syncthreads();
    dense_f32(s_x, 256, (const float*)a.w[0], a.b[0], 512, s_h, 512);
    __syncthreads();
    dense_f32(s_h, 512, (const float*)a.w[1], a.b[1], 256, s_x, 256);
    __syncthreads();
    dense_f32(s_x, 256, (const float*)a.w[2], a.b[2], 128, s_z, 176);
    __syncthreads();
    if (a.deep_out) {
        for (int idx = tid; idx < kM * 128; idx += kF32Threads) {
            const int r = idx >> 7, c = idx & 127;
            const int64_t b = b0 + r;
            if (b < a.B) a.deep_out[b * 128 + c] = s_z[r * 176 + c];
        }
    }
    dense_f32(s_z, 176, (const float*)a.w[3], a.b[3], 64, s_h, 64);
    __syncthreads();
    if (tid < kM) {
        const int64_t b = b0 + tid;
        if (b < a.B) {
            float l = a.bo;
            for (int i = 0; i < 64; ++i) l = fmaf(a.wo[i], s_h[tid * 64 + i], l);
            a.logit[b] = l;
            if (a.prob) a.prob[b] = logistic(l);
        }
    }
}

// One thread per 16-byte slot of the packed image: the slot holds the 8 bf16
// the plain layout gives that lane of that fragment.
struct PackArgs {
    const uint16_t* w[4];
    uint4* out;
};

__global__ __launch_bounds__(256) void k_tower_pack(const PackArgs p) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= REC_TOWER_PACKED_BYTES / 16) return;
    const int lane = d & 63, frag = d >> 6;
    int w, f;                      // a wave that reads this fragment, and its index there
    if (frag < kWaves * kDeepFrags) {
        w = frag / kDeepFrags;
        f = frag % kDeepFrags;
    } else {
        w = (frag - kWaves * kDeepFrags) / kNK[3];
        f = kDeepFrags + (frag - kWaves * kDeepFrags) % kNK[3];
    }
    const int l = layer_of(f), r = f - layer_base(l);
    const int nt = l == 0 ? 4 : l == 1 ? 2 : 1;
    const int ldw = l == 0 ? 256 : l == 1 ? 512 : l == 2 ? 256 : 176;
    const int c = r / nt, t = r % nt;
    const int row = 16 * (l == 3 ? (w & 3) : (l == 0 ? 4 : l == 1 ? 2 : 1) * w + t) + (lane & 15);
    const uint16_t* W = l == 0 ? p.w[0] : l == 1 ? p.w[1] : l == 2 ? p.w[2] : p.w[3];
    int c0, c1;
    frag_cols(l, c, lane >> 4, &c0, &c1);
    if (c0 >= ldw) {
        p.out[d] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    const uint2 lo = *(const uint2*)(W + row * ldw + c0), hi = *(const uint2*)(W + row * ldw + c1);
    p.out[d] = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// A-fragments in flight per wave
constexpr int kStream = TOWER_STREAM;

template <int G>
hipError_t launch_bf16(const TowerArgs& a, hipStream_t s) {
    const int64_t blocks = (a.B + 16 * G - 1) / (16 * G);
    if (a.dtype == REC_BF16_PACKED)
        REC_LAUNCH(REC_TIME_TOWERS, (k_towers_bf16<true, kStream, G>), dim3((unsigned)blocks),
                   dim3(64 * kWaves), 0, s, a);
    else
        REC_LAUNCH(REC_TIME_TOWERS, (k_towers_bf16<false, kStream, G>), dim3((unsigned)blocks),
                   dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_towers(const TowerArgs& a, hipStream_t s) {
    if (a.dtype == REC_F32) {
        hipLaunchKernelGGL(k_towers_f32, dim3((unsigned)((a.B + kM - 1) / kM)), dim3(kF32Threads),
                           0, s, a);
        return hipGetLastError();
    }
    return a.B >= TOWER_BIG_B ? launch_bf16<4>(a, s) : launch_bf16<2>(a, s);
}

hipError_t launch_tower_pack(const void* const w[4], void* packed, hipStream_t s) {
    PackArgs p;
    for (int l = 0; l < 4; ++l) p.w[l] = (const uint16_t*)w[l];
    p.out = (uint4*)packed;
    hipLaunchKernelGGL(k_tower_pack, dim3(REC_TOWER_PACKED_BYTES / 16 / 256), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace rec
