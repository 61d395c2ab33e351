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
// One launch, fp32 throughout, 16 samples per 8-wave workgroup:
//   - the bags pool straight into the interaction input z in LDS (vector t+1
//     of a sample is bag (t, b)), eight lanes per bag, each lane holding d/32
//     float4 columns of a row, so one wave instruction reads eight rows' worth
//     of 128-byte runs; ids are loaded four at a time ahead of their rows;
//   - the bottom MLP writes vector 0 of z; z goes out to memory once;
//   - the interaction: per sample G = Z Z^T on the fp32 matrix cores (Z padded
//     to 16 rows; the A and B operands of a product are the same register),
//     whose upper triangle is the pair list;
//   - the top MLP, then the logit and the probability.
// The dense layers run on v_mfma_f32_16x16x4f32 with the weights as the A
// operand read from memory (every workgroup reads the same few hundred KiB,
// so they come from L2) and the activations in LDS as the B operand.
#include "rec_mfma.h"
#include "rec_internal.h"

namespace rec {
namespace {

constexpr int kBagLanes = 8;                 // lanes per bag
constexpr int kIdRound = 4;                  // ids of a bag loaded per round
constexpr int kDenseSamples = 16;             // samples per workgroup
constexpr int kDenseThreads = 512;            // eight waves: two per SIMD

// NU chunks of 16 inputs (from input i0) of one 16-unit tile: the operands
// of all of them are loaded, then their 4 * NU products run.  K order: in
// step 4c + j, lane (m, k) takes input 16c + 4k + j, so a lane's four inputs
// of a chunk are one float4 of its W row (one load covers 16 whole 64-byte
// row pieces) and one 16-byte LDS read of its activations.
template <int NU, bool kVec>
__device__ inline void layer_chunks(const float* in, int ins, int nin, const float* wr, int i0, int m,
                                    int kg, f32x4& acc) {
    float4 av[NU], bv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int i = i0 + 16 * u + 4 * kg;
        if (kVec) {
            const float4 w = *(const float4*)(wr + (i < nin ? i : 0));
            av[u] = i < nin ? w : make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = wr[min(i + j, nin - 1)];
                v[j] = i + j < nin ? w : 0.f;
            }
            av[u] = make_float4(v[0], v[1], v[2], v[3]);
        }
        bv[u] = *(const float4*)(in + m * ins + i);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].x, bv[u].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].y, bv[u].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].z, bv[u].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u].w, bv[u].w, acc, 0, 0, 0);
    }
}

template <bool kVec>
__device__ inline void layer_part(const float* in, int ins, int nin, const float* wr, int i0, int nu, int m,
                                  int kg, f32x4& acc) {
    switch (nu) {                                          // uniform
        case 1: layer_chunks<1, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
        case 2: layer_chunks<2, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
        case 3: layer_chunks<3, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
        case 4: layer_chunks<4, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
        case 5: layer_chunks<5, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
        case 6: layer_chunks<6, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
        case 7: layer_chunks<7, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
        default: layer_chunks<8, kVec>(in, ins, nin, wr, i0, m, kg, acc); break;
    }
}

// One dense layer on the matrix cores: out[r][o] = act(bias[o] + sum_i W[o][i]
// in[r][i]) for the workgroup's 16 rows r and o < nout (a multiple of 16),
// with in and out in LDS (row strides ins, outs; in's rows hold zeros from
// nin up to a multiple of 16) and W [nout][nin] in memory (torch.nn.Linear's
// layout).  v_mfma_f32_16x16x4f32: A = 16 units x 4 inputs of W, B = 4 inputs
// x 16 rows; the result's lane (n, k) holds units o0 + 4k .. +3 of row n.
// Wave w takes the 16-unit tiles w, w + 8, ...; up to 8 chunks (128 inputs)
// of a tile are loaded together ahead of their products.
__device__ inline void mfma_layer(const float* in, int ins, int nin, const float* __restrict__ W,
                                  const float* __restrict__ bias, int nout, float* out, int outs,
                                  bool relu) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m = lane & 15, kg = lane >> 4;
    const int nch = (nin + 15) / 16;
    const bool vec = (nin & 3) == 0;                      // W rows are 16-byte aligned
    for (int ot = wave; ot * 16 < nout; ot += kDenseThreads / 64) {
        const int o0 = ot * 16;
        f32x4 acc = *(const f32x4*)(bias + o0 + 4 * kg);
        const float* wr = W + (int64_t)(o0 + m) * nin;
        for (int c0 = 0; c0 < nch; c0 += 8) {
            const int nu = min(8, nch - c0);
            if (vec) layer_part<true>(in, ins, nin, wr, 16 * c0, nu, m, kg, acc);
            else layer_part<false>(in, ins, nin, wr, 16 * c0, nu, m, kg, acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = acc[j];
            out[m * outs + o0 + 4 * kg + j] = relu ? fmaxf(v, 0.f) : v;
        }
    }
}

// One bag's pooled row, lane c of its eight holding float4 columns c, c + 8,
// ... (len 0 for a lane without a bag; the loop runs while any bag of the wave
// has ids left).  A round's id and row loads are issued under the execution
// mask, only for ids the bag still holds, so short bags issue no duplicate
// loads; the other slots add zeros.
template <int NF>
__device__ inline void bag_pool(const DlrmArgs& a, const TabDev& tab, int32_t mode, int64_t bag, int32_t len,
                                int c, float4 (&acc)[NF]) {
    const int d = a.dim;
    const int64_t off = a.offsets[bag];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; __ballot(j0 < len) != 0; j0 += kIdRound) {
        int64_t raw[kIdRound];
#pragma unroll
        for (int u = 0; u < kIdRound; ++u) {
            raw[u] = 0;
            if (j0 + u < len) raw[u] = a.values[off + j0 + u];
        }
        float4 v[kIdRound][NF];
#pragma unroll
        for (int u = 0; u < kIdRound; ++u) {
#pragma unroll
            for (int f = 0; f < NF; ++f) v[u][f] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j0 + u < len) {
                const int64_t row = floor_mod_magic(raw[u], tab.rows, tab.magic, tab.shift);
                const float4* src = (const float4*)(tab.values + row * d) + c;
#pragma unroll
                for (int f = 0; f < NF; ++f) v[u][f] = src[8 * f];
            }
        }
#pragma unroll
        for (int u = 0; u < kIdRound; ++u) {
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                acc[f].x += v[u][f].x;
                acc[f].y += v[u][f].y;
                acc[f].z += v[u][f].z;
                acc[f].w += v[u][f].w;
            }
        }
    }
    if (mode == REC_POOL_MEAN && len > 0) {
        const float inv = 1.f / (float)len;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            acc[f].x *= inv;
            acc[f].y *= inv;
            acc[f].z *= inv;
            acc[f].w *= inv;
        }
    }
}

// The bags of the workgroup's samples b0 .. b0 + rows - 1 into z in LDS
// (row stride zs, vector t + 1 = bag (t, b)).
template <int NF>
__device__ inline void bags_into_lds(const DlrmArgs& a, int64_t b0, int rows, float* s_z, int zs) {
    const int lane = threadIdx.x & 63, c = lane & 7;
    const int nq = kDenseSamples * a.S;                      // bags of the workgroup
    for (int q0 = (int)(threadIdx.x >> 6) * 8; q0 < nq; q0 += kDenseThreads / kBagLanes) {
        // q0 is a multiple of 8, so the wave's eight bags share their table
        const int q = q0 + (lane >> 3);
        const int r = q % kDenseSamples;
        const int t = __builtin_amdgcn_readfirstlane(q0 / kDenseSamples);
        const bool live = q < nq && r < rows;
        const int64_t bag = (int64_t)t * a.B + b0 + (live ? r : 0);
        const int32_t len = live ? a.lengths[bag] : 0;
        float4 acc[NF];
        bag_pool<NF>(a, a.tab[t], a.mode[t], bag, len, c, acc);
        if (!live) continue;
        float4* o = (float4*)(s_z + r * zs + (1 + t) * a.dim) + c;
#pragma unroll
        for (int f = 0; f < NF; ++f) o[8 * f] = acc[f];
    }
}

__host__ __device__ inline int round16(int x) { return (x + 15) & ~15; }

// Dynamic LDS of k_dlrm_fwd, in floats: z of the 16 samples (rows of F*d,
// as in memory; later the top MLP's two hidden layers), then the bottom MLP's
// input and hidden layer (later the interaction output), then the pair list
// (two uint16 per pair).
struct DenseLds {
    int zs, xs, hs, is, np, zfl, bfl, bytes;
};
__host__ __device__ inline DenseLds dense_lds(int S, int d, int n_dense) {
    DenseLds L;
    const int F = S + 1;
    L.zs = F * d;
    L.xs = round16(n_dense) + 4;
    L.hs = 128 + 4;
    L.np = F * (F + 1) / 2;
    L.is = round16(L.np) + 4;
    const int top = kDenseSamples * (L.hs + 64 + 4);
    L.zfl = max(kDenseSamples * L.zs, top);
    L.bfl = max(kDenseSamples * (L.xs + L.hs), kDenseSamples * L.is);
    L.bytes = 4 * (L.zfl + L.bfl) + 4 * L.np;
    return L;
}

template <int NF>
// At most 168 registers (three waves per SIMD): a workgroup of eight waves
// holds a CU either way, and widths up to 224 then need no scratch.
__global__ __launch_bounds__(kDenseThreads, 3) void k_dlrm_fwd(const DlrmArgs a) {
    extern __shared__ __attribute__((aligned(16))) float s_dyn[];
    const DenseLds Ld = dense_lds(a.S, a.dim, a.n_dense);
    const int F = a.S + 1, d = a.dim, zw = F * d, zs = Ld.zs;
    const int np = Ld.np, is = Ld.is, xs = Ld.xs, hs = Ld.hs;
    float* s_z = s_dyn;
    float* s_b = s_dyn + Ld.zfl;
    float* s_x = s_b;
    float* s_h = s_b + kDenseSamples * xs;
    float* s_i = s_b;
    float* s_t1 = s_z;
    float* s_t2 = s_z + kDenseSamples * hs;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m = lane & 15, kg = lane >> 4;
    const int64_t b0 = (int64_t)blockIdx.x * kDenseSamples;
    const int rows = (int)min((int64_t)kDenseSamples, a.B - b0);
    // dense inputs (rows past the batch and columns past n_dense read zeros)
    for (int idx = threadIdx.x; idx < kDenseSamples * xs; idx += kDenseThreads) {
        const int r = idx / xs, i = idx - r * xs;
        const bool ok = r < rows && i < a.n_dense;
        const float v = a.dense[ok ? (b0 + r) * a.n_dense + i : 0];
        s_x[idx] = ok ? v : 0.f;
    }
    bags_into_lds<NF>(a, b0, rows, s_z, zs);
    __syncthreads();
    mfma_layer(s_x, xs, a.n_dense, a.wb1, a.bb1, 128, s_h, hs, true);
    __syncthreads();
    mfma_layer(s_h, hs, 128, a.wb2, a.bb2, d, s_z, zs, true);       // vector 0 of z
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows * zw / 4; idx += kDenseThreads)
        ((float4*)(a.z + b0 * (int64_t)zw))[idx] = ((const float4*)s_z)[idx];
    // the interaction: G = Z Z^T per sample, lane (n, k) of the result holding
    // G[4k + j][n]; rows of Z past F read zeros
    for (int r = wave; r < kDenseSamples; r += kDenseThreads / 64) {
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
        const float* zr = s_z + r * zs + m * d + 4 * kg;
        for (int c = 0; c < d / 16; ++c) {
            const float4 v = m < F ? *(const float4*)(zr + 16 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
            g = __builtin_amdgcn_mfma_f32_16x16x4f32(v.x, v.x, g, 0, 0, 0);
            g = __builtin_amdgcn_mfma_f32_16x16x4f32(v.y, v.y, g, 0, 0, 0);
            g = __builtin_amdgcn_mfma_f32_16x16x4f32(v.z, v.z, g, 0, 0, 0);
            g = __builtin_amdgcn_mfma_f32_16x16x4f32(v.w, v.w, g, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = 4 * kg + j, n = m;
            if (i <= n && n < F) {
                const int p = i * F - i * (i - 1) / 2 + (n - i);
                s_i[r * is + p] = g[j];
                if (a.inter && r < rows) a.inter[(b0 + r) * np + p] = g[j];
            }
        }
    }
    for (int idx = threadIdx.x; idx < kDenseSamples * (is - np); idx += kDenseThreads) {
        const int r = idx / (is - np);
        s_i[r * is + np + idx - r * (is - np)] = 0.f;           // the pad columns read zeros
    }
    __syncthreads();
    mfma_layer(s_i, is, np, a.wt1, a.bt1, 128, s_t1, hs, true);
    __syncthreads();
    mfma_layer(s_t1, hs, 128, a.wt2, a.bt2, 64, s_t2, 64 + 4, true);
    __syncthreads();
    if (threadIdx.x < rows) {
        const int r = threadIdx.x;
        float l = a.bt3;
        for (int i = 0; i < 64; ++i) l = fmaf(a.wt3[i], s_t2[r * (64 + 4) + i], l);
        a.logit[b0 + r] = l;
        if (a.prob) a.prob[b0 + r] = 1.f / (1.f + expf(-l));
    }
}

}  // namespace

// Wide models (more than 31 tables, or (S + 1) * d above 1024 floats per
// sample): z and the interaction output go through memory.  Launches: the
// bags, up to 32 tables per launch (a table group's descriptors are
// a.tab[0 .. nt)); the bottom MLP; the interaction (rec_dlrm.hip); the top
// MLP, whose first layer reads its inputs from memory.
template <int NF>
__global__ __launch_bounds__(256) void k_dlrm_bags_wide(const DlrmArgs a, int t0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nbw = (a.B + 31) / 32;                  // 32-sample chunks per table
    const int t = (int)(blockIdx.x / nbw);                 // table of the group
    const int64_t b = (blockIdx.x % nbw) * 32 + wave * kBagLanes + (lane >> 3);
    const bool live = b < a.B;
    const int64_t bag = (int64_t)(t0 + t) * a.B + (live ? b : 0);
    const int32_t len = live ? a.lengths[bag] : 0;
    float4 acc[NF];
    bag_pool<NF>(a, a.tab[t], a.mode[t], bag, len, lane & 7, acc);
    if (!live) return;
    float4* o = (float4*)(a.z + (b * (int64_t)(a.S + 1) + 1 + t0 + t) * a.dim) + (lane & 7);
#pragma unroll
    for (int f = 0; f < NF; ++f) o[8 * f] = acc[f];
}

__global__ __launch_bounds__(kDenseThreads) void k_dlrm_bottom(const DlrmArgs a) {
    constexpr int kXs = kDlrmMaxDense + 4, kHs = 128 + 4, kOs = 256 + 4;
    __shared__ __attribute__((aligned(16))) float s_x[kDenseSamples * kXs];
    __shared__ __attribute__((aligned(16))) float s_h[kDenseSamples * kHs];
    __shared__ __attribute__((aligned(16))) float s_o[kDenseSamples * kOs];
    const int64_t b0 = (int64_t)blockIdx.x * kDenseSamples;
    const int rows = (int)min((int64_t)kDenseSamples, a.B - b0);
    const int xs = round16(a.n_dense) + 4;
    for (int idx = threadIdx.x; idx < kDenseSamples * xs; idx += kDenseThreads) {
        const int r = idx / xs, i = idx - r * xs;
        const bool ok = r < rows && i < a.n_dense;
        const float v = a.dense[ok ? (b0 + r) * a.n_dense + i : 0];
        s_x[idx] = ok ? v : 0.f;
    }
    __syncthreads();
    mfma_layer(s_x, xs, a.n_dense, a.wb1, a.bb1, 128, s_h, kHs, true);
    __syncthreads();
    mfma_layer(s_h, kHs, 128, a.wb2, a.bb2, a.dim, s_o, kOs, true);
    __syncthreads();
    const int d4 = a.dim / 4;
    for (int idx = threadIdx.x; idx < rows * d4; idx += kDenseThreads) {
        const int r = idx / d4, c = idx - r * d4;
        ((float4*)(a.z + (b0 + r) * (int64_t)(a.S + 1) * a.dim))[c] = *(const float4*)(s_o + r * kOs + 4 * c);
    }
}

// A float4 of memory that is only 4-byte aligned (rows of an odd number of
// floats); the hardware reads it with one 16-byte load.
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

// The wide first top layer runs in stages of kTopK inputs: W's 128 rows and
// the 16 samples' inputs over the stage, staged in LDS (row stride kTopS
// floats, two buffers).  Each of the 512 threads moves kTopLd float4s per
// stage; a wave's float4s are two rows' 512-byte runs, so one load touches
// few cache lines (reading the MFMA operands straight from memory, where one
// load spans 16 rows, kept the address units busy nine tenths of the time).
constexpr int kTopK = 128, kTopS = kTopK + 4;
constexpr int kTopRows = 128 + kDenseSamples;                     // W rows, then x rows
constexpr int kTopBuf = kTopRows * kTopS;                          // floats per buffer
constexpr int kTopLd = kTopRows * (kTopK / 4) / kDenseThreads;    // float4s per thread
static_assert(kTopRows * (kTopK / 4) % kDenseThreads == 0, "stage split");
constexpr int kTopLdsBytes = 2 * kTopBuf * 4;                      // 152 KiB

// Thread t's float4s of the stage at input k0: all of them exist (kEdge
// false), or those past np read zeros (the last stage).
template <bool kEdge>
__device__ inline void top_stage_load(const float* W, const float* xb, int64_t np, int rows, int64_t k0,
                                      f32x4u (&v)[kTopLd]) {
#pragma unroll
    for (int q = 0; q < kTopLd; ++q) {
        const int idx = q * kDenseThreads + threadIdx.x;
        const int r = idx / (kTopK / 4), c4 = idx % (kTopK / 4);
        // rows past the batch re-read the last sample (their results are dropped)
        const float* src = r < 128 ? W + (int64_t)r * np : xb + (int64_t)min(r - 128, rows - 1) * np;
        const int64_t i = k0 + 4 * c4;
        if (!kEdge) {
            v[q] = *(const f32x4u*)(src + i);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float t = src[min(i + j, np - 1)];
                v[q][j] = i + j < np ? t : 0.f;
            }
        }
    }
}

__device__ inline void top_stage_store(float* buf, const f32x4u (&v)[kTopLd]) {
#pragma unroll
    for (int q = 0; q < kTopLd; ++q) {
        const int idx = q * kDenseThreads + threadIdx.x;
        const int r = idx / (kTopK / 4), c4 = idx % (kTopK / 4);
        *(f32x4*)(buf + r * kTopS + 4 * c4) = f32x4{v[q][0], v[q][1], v[q][2], v[q][3]};
    }
}

// The top MLP of a wide model, 16 samples per workgroup.  Its first layer
// (np = F(F+1)/2 inputs read from memory, 23,653 for F = 217, to 128 units)
// is the bulk of the work.  Per stage, wave w takes inputs 16w .. 16w + 15 of
// the stage for all 128 units (eight 16-unit tiles: per lane eight W float4s
// and one x float4 from LDS, 32 products), so every staged value is read
// once; the next two stages' loads are in flight meanwhile (one stage ahead
// left the waves waiting on memory: 433 us against 383 us for the 217-feature
// model at B = 4096; one ahead from memory without LDS, 480 us; the first
// version, eight waves over the 128 units each reading every input from
// memory, 1.80 ms).  Each wave thus sums
// one eighth of the inputs; the eight partial sums are added in LDS in wave
// order, then bias and ReLU, and the 128 -> 64 -> 1 layers run as in the
// one-launch kernel.
__global__ __launch_bounds__(kDenseThreads) void k_dlrm_top_wide(const DlrmArgs a) {
    extern __shared__ __attribute__((aligned(16))) float s_dyn[];
    constexpr int kWaves = kDenseThreads / 64, kPs = 128, kT2s = 64 + 4;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, kg = lane >> 4;
    const int F = a.S + 1;
    const int64_t np = (int64_t)F * (F + 1) / 2;
    const int64_t b0 = (int64_t)blockIdx.x * kDenseSamples;
    const int rows = (int)min((int64_t)kDenseSamples, a.B - b0);
    const float* xb = a.inter + b0 * np;
    const int nst = (int)((np + kTopK - 1) / kTopK);
    f32x4 acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nfull = (int)(np / kTopK);                   // stages whose inputs all exist
    // Two stages' loads are in flight while a third is computed: stage st is
    // in LDS buffer st & 1, stage st + 1 in one register set, st + 2 in the
    // other.
    f32x4u va[kTopLd], vb[kTopLd];
    auto load = [&](int sidx, f32x4u (&v)[kTopLd]) {
        const int64_t k = (int64_t)sidx * kTopK;
        if (sidx < nfull) top_stage_load<false>(a.wt1, xb, np, rows, k, v);
        else if (sidx < nst) top_stage_load<true>(a.wt1, xb, np, rows, k, v);
    };
    auto compute = [&](const float* cur) {
        const float* wl = cur + m * kTopS + 16 * wave + 4 * kg;
        const f32x4 xv = *(const f32x4*)(cur + (128 + m) * kTopS + 16 * wave + 4 * kg);
        f32x4 wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) wv[u] = *(const f32x4*)(wl + 16 * u * kTopS);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int u = 0; u < 8; ++u)
                acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[u][j], xv[j], acc[u], 0, 0, 0);
    };
    float* buf0 = s_dyn;
    float* buf1 = s_dyn + kTopBuf;
    load(0, va);
    top_stage_store(buf0, va);
    load(1, va);
    load(2, vb);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        compute(buf0);                                     // stage st
        if (st + 1 < nst) top_stage_store(buf1, va);
        load(st + 3, va);
        __syncthreads();
        if (st + 1 >= nst) break;
        compute(buf1);                                     // stage st + 1
        if (st + 2 < nst) top_stage_store(buf0, vb);
        load(st + 4, vb);
        __syncthreads();
    }
    // lane (m, k) holds units 16u + 4k .. +3 of sample m; the partial sums
    // [wave][sample][unit] reuse the stage buffers, then t1 takes the first
    // slab and t2 the second
    float* s_part = s_dyn;
    float* s_t1 = s_part;
    float* s_t2 = s_part + kDenseSamples * kPs;
#pragma unroll
    for (int u = 0; u < 8; ++u)
        *(f32x4*)(s_part + (wave * kDenseSamples + m) * kPs + 16 * u + 4 * kg) = acc[u];
    __syncthreads();
    for (int idx = 4 * threadIdx.x; idx < kDenseSamples * kPs; idx += 4 * kDenseThreads) {
        f32x4 t = *(const f32x4*)(s_part + idx);
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += *(const f32x4*)(s_part + w * kDenseSamples * kPs + idx);
        const f32x4 bb = *(const f32x4*)(a.bt1 + idx % kPs);
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = fmaxf(t[j] + bb[j], 0.f);
        *(f32x4*)(s_t1 + idx) = t;                         // only this thread touches idx
    }
    __syncthreads();
    mfma_layer(s_t1, kPs, 128, a.wt2, a.bt2, 64, s_t2, kT2s, true);
    __syncthreads();
    if (threadIdx.x < rows) {
        const int r = threadIdx.x;
        float l = a.bt3;
        for (int i = 0; i < 64; ++i) l = fmaf(a.wt3[i], s_t2[r * kT2s + i], l);
        a.logit[b0 + r] = l;
        if (a.prob) a.prob[b0 + r] = 1.f / (1.f + expf(-l));
    }
}

template <int NF>
hipError_t launch_bags_wide(const DlrmArgs& a, const TabDev* tabs, const int32_t* modes, hipStream_t s) {
    const int64_t nbw = (a.B + 31) / 32;
    for (int t0 = 0; t0 < a.S; t0 += 32) {
        DlrmArgs g = a;
        const int nt = min(32, a.S - t0);
        for (int t = 0; t < nt; ++t) {
            g.tab[t] = tabs[t0 + t];
            g.mode[t] = modes[t0 + t];
        }
        hipLaunchKernelGGL(k_dlrm_bags_wide<NF>, dim3((unsigned)(nt * nbw)), dim3(256), 0, s, g, t0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int NF>
hipError_t launch_dlrm_nf(const DlrmArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.B + kDenseSamples - 1) / kDenseSamples)), blk(kDenseThreads);
    const DenseLds L = dense_lds(a.S, a.dim, a.n_dense);
    if (L.bytes > 64 * 1024) {
        // beyond the default limit of dynamic LDS (at most about 100 KiB within
        // rec_dlrm_fwd's limits)
        const hipError_t e = hipFuncSetAttribute((const void*)k_dlrm_fwd<NF>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, L.bytes);
        if (e != hipSuccess) return e;
    }
    REC_LAUNCH(REC_TIME_DLRM_FWD, k_dlrm_fwd<NF>, grid, blk, (size_t)L.bytes, s, a);
    return hipGetLastError();
}

hipError_t launch_dlrm_fwd_wide(const DlrmArgs& a, const TabDev* tabs, const int32_t* modes, int num_cus,
                                hipStream_t s) {
    hipError_t e;
    switch (a.dim / 32) {
        case 1: e = launch_bags_wide<1>(a, tabs, modes, s); break;
        case 2: e = launch_bags_wide<2>(a, tabs, modes, s); break;
        case 3: e = launch_bags_wide<3>(a, tabs, modes, s); break;
        case 4: e = launch_bags_wide<4>(a, tabs, modes, s); break;
        case 5: e = launch_bags_wide<5>(a, tabs, modes, s); break;
        case 6: e = launch_bags_wide<6>(a, tabs, modes, s); break;
        case 7: e = launch_bags_wide<7>(a, tabs, modes, s); break;
        default: e = launch_bags_wide<8>(a, tabs, modes, s); break;
    }
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.B + kDenseSamples - 1) / kDenseSamples)), blk(kDenseThreads);
    hipLaunchKernelGGL(k_dlrm_bottom, grid, blk, 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_dlrm_interact(a.z, a.B, a.S + 1, a.dim, a.inter, num_cus, s);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)k_dlrm_top_wide, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kTopLdsBytes);
    if (e != hipSuccess) return e;
    REC_LAUNCH(REC_TIME_DLRM_FWD, k_dlrm_top_wide, grid, blk, (size_t)kTopLdsBytes, s, a);
    return hipGetLastError();
}

hipError_t launch_dlrm_fwd(const DlrmArgs& a, hipStream_t s) {
    switch (a.dim / 32) {
        case 1: return launch_dlrm_nf<1>(a, s);
        case 2: return launch_dlrm_nf<2>(a, s);
        case 3: return launch_dlrm_nf<3>(a, s);
        case 4: return launch_dlrm_nf<4>(a, s);
        case 5: return launch_dlrm_nf<5>(a, s);
        case 6: return launch_dlrm_nf<6>(a, s);
        case 7: return launch_dlrm_nf<7>(a, s);
        default: return launch_dlrm_nf<8>(a, s);
    }
}

}  // namespace rec
