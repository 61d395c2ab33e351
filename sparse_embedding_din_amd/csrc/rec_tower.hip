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
// bf16 path: one workgroup of four waves carries 32 samples through all five
// layers and the activations never leave the chip.  Each layer's results go
// through bias, ReLU and bf16 rounding into an LDS array [32 samples][units]
// (rows padded by 16 bytes, so a wave's 16-byte operand reads and 8-byte
// result writes fall on distinct banks), which the next layer reads as its
// matrix-core B operand.  The waves split each layer's output units (wave w
// owns a quarter of the 16-unit tiles), so every weight is read once per
// workgroup, straight from global memory into registers as the A operand, a
// few K-steps ahead of its use; both 16-sample halves of the workgroup share
// each weight fragment.  The next layer's first fragments are in flight
// across each barrier.  The weights are the plain row-major bf16 matrices
// (torch.nn.Linear layout), or the image rec_tower_pack_mlp writes once, in
// which every fragment load is 1 KiB of consecutive memory: with the plain
// layout the 64 lanes of a load touch 16 rows, and the loads run several
// times slower.
//
// fp32 path: the same dataflow with fp32 activations in LDS and one output
// (sample, unit) per thread per pass, plain fp32 fused multiply-adds in
// column order; it exists for exactness checks at small sizes.
#include "rec_internal.h"
#include "rec_mfma.h"

namespace rec {
namespace {

constexpr int kM = kTowerSamples;        // 32 samples = two 16-sample halves
constexpr int kWaves = 4;
// LDS row strides in bf16 elements
constexpr int kStrX = 256 + 8;           // deep input; later the 256-wide second layer
constexpr int kStrH = 512 + 8;           // first hidden layer
constexpr int kStrZ = 192 + 8;           // [deep out (128), att (48), zeros (16)]
// K-steps of A fragments kept in flight, per layer
constexpr int kPf1 = 4, kPf2 = 4, kPf3 = 4, kPf4 = 3;

// Where a layer's A fragments come from.  Plain: rows [row0, row0 + 16 NT)
// of the row-major matrix W (ldw columns); lane (m, g) of K-step c reads
// 16 bytes of row row0 + 16t + m at column 32c + 8g, zero at or past kvalid.
// Packed (rec_tower_pack_mlp): the same 16 bytes, stored so that a wave's
// fragments for a layer are one contiguous run [c][t][lane] -- each fragment
// load is then 1 KiB of consecutive memory in lane order.
struct ASrc {
    const uint16_t* W;     // plain matrix, or the layer's run in the packed image
    int ldw, row0, kvalid;
};

template <bool kPacked, int NT>
__device__ inline void load_a(uint4 (&r)[NT], const ASrc& A, int c, int lane) {
    if (kPacked) {
        const uint4* P = (const uint4*)A.W;
#pragma unroll
        for (int t = 0; t < NT; ++t) r[t] = P[(c * NT + t) * 64 + lane];
        return;
    }
    const int m = lane & 15, col = 32 * c + 8 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (col < A.kvalid)
            r[t] = *(const uint4*)(A.W + (int64_t)(A.row0 + 16 * t + m) * A.ldw + col);
        else
            r[t] = make_uint4(0u, 0u, 0u, 0u);
    }
}

template <bool kPacked, int NT, int PF>
__device__ inline void prefetch_a(uint4 (&ring)[PF][NT], const ASrc& A, int lane) {
#pragma unroll
    for (int c = 0; c < PF; ++c) load_a<kPacked, NT>(ring[c], A, c, lane);
}

// Accumulators start from the bias of their rows (the first product's C).
template <int NT>
__device__ inline void bias_init(f32x4 (&acc)[NT][2], const float* __restrict__ bias, int row0,
                                 int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const f32x4 b = *(const f32x4*)(bias + row0 + 16 * t + 4 * (lane >> 4));
        acc[t][0] = b;
        acc[t][1] = b;
    }
}

// acc[t][s] += W(rows of tile t) x in(half s), over NK K-steps of 32.  The
// ring holds K-steps 0 .. PF-1 on entry; step c + PF is loaded into the slot
// step c has just used.
template <bool kPacked, int NT, int NK, int PF>
__device__ inline void layer_mma(f32x4 (&acc)[NT][2], uint4 (&ring)[PF][NT], const ASrc& A,
                                 const __bf16* in, int istr, int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int c = 0; c < NK; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        const int slot = c % PF;
        bf16x8 x[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) x[s] = *(const bf16x8*)(in + (16 * s + m) * istr + 32 * c + 8 * g);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, ring[slot][t]), x[s], acc[t][s], 0, 0, 0);
        if (c + PF < NK) load_a<kPacked, NT>(ring[slot], A, c + PF, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// ReLU + bf16 of tiles (unit0 + 16t ...) into the LDS rows of their samples.
template <int NT>
__device__ inline void store_act(const f32x4 (&acc)[NT][2], __bf16* out, int ostr, int unit0,
                                 int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint2 p;
            p.x = relu_pk_bf16(acc[t][s][0], acc[t][s][1]);
            p.y = relu_pk_bf16(acc[t][s][2], acc[t][s][3]);
            *(uint2*)(out + (16 * s + m) * ostr + unit0 + 16 * t + 4 * g) = p;
        }
}

__device__ inline uint2 pack_bf16x4(float4 v) {
    bf16x2 lo, hi;
    lo[0] = (__bf16)v.x;
    lo[1] = (__bf16)v.y;
    hi[0] = (__bf16)v.z;
    hi[1] = (__bf16)v.w;
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ inline float logistic(float l) { return 1.f / (1.f + expf(-l)); }

// The packed image: layer l's fragments for wave w start at
// pack_base(l) + w * NK_l * NT_l fragments (one fragment = 64 lanes x 16 B).
constexpr int kNT[4] = {8, 4, 2, 1}, kNK[4] = {8, 16, 8, 6};
__host__ __device__ constexpr int pack_frags(int l) { return kWaves * kNT[l] * kNK[l]; }
__host__ __device__ constexpr int pack_base(int l) {
    return l == 0 ? 0 : pack_base(l - 1) + pack_frags(l - 1);
}
static_assert((pack_base(3) + pack_frags(3)) * 1024 == REC_TOWER_PACKED_BYTES,
              "packed tower image size");
constexpr int kLdw[4] = {256, 512, 256, 176}, kRowsPerWave[4] = {128, 64, 32, 16};

template <bool kPacked>
__device__ inline ASrc a_src(const TowerArgs& a, int l, int w) {
    ASrc s;
    if (kPacked) {
        s.W = (const uint16_t*)a.w[0] + (int64_t)(pack_base(l) + w * kNK[l] * kNT[l]) * 512;
    } else {
        s.W = (const uint16_t*)a.w[l];
    }
    s.ldw = kLdw[l];
    s.row0 = kRowsPerWave[l] * w;
    s.kvalid = kLdw[l];
    return s;
}

template <bool kPacked>
__global__ __launch_bounds__(64 * kWaves) void k_towers_bf16(const TowerArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 s_x[kM * kStrX];   // deep input, then layer 2
    __shared__ __attribute__((aligned(16))) __bf16 s_h[kM * kStrH];   // layer 1
    __shared__ __attribute__((aligned(16))) __bf16 s_z[kM * kStrZ];   // concat input of layer 4
    __shared__ float s_part[kWaves][kM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t b0 = (int64_t)blockIdx.x * kM;
    const ASrc A1 = a_src<kPacked>(a, 0, w), A2 = a_src<kPacked>(a, 1, w);
    const ASrc A3 = a_src<kPacked>(a, 2, w), A4 = a_src<kPacked>(a, 3, w);

    uint4 r1[kPf1][8];
    prefetch_a<kPacked, 8, kPf1>(r1, A1, lane);
    // stage the deep input (first 256 pooled columns) and att as bf16.  Rows
    // of samples past B are read at row B-1 and zeroed, so that every load
    // of the staging is issued before the first wait.
    float4 xv[4][2], av[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int u = tid + 256 * j, row = u >> 5, col = (u & 31) * 8;
        const float4* p = (const float4*)(a.pooled + min(b0 + row, a.B - 1) * a.pooled_ld + col);
        xv[j][0] = p[0];
        xv[j][1] = p[1];
    }
    const int arow = tid >> 3, acol = (tid & 7) * 8;   // att columns 0..63, 48.. are zero
    {
        const float4* p = (const float4*)(a.att + min(b0 + arow, a.B - 1) * 48 + min(acol, 40));
        av[0] = p[0];
        av[1] = p[1];
    }
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int u = tid + 256 * j, row = u >> 5, col = (u & 31) * 8;
        const bool live = b0 + row < a.B;
        const uint2 lo = pack_bf16x4(live ? xv[j][0] : zero4), hi = pack_bf16x4(live ? xv[j][1] : zero4);
        *(uint4*)(s_x + row * kStrX + col) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    {
        const bool live = b0 + arow < a.B && acol < 48;
        const uint2 lo = pack_bf16x4(live ? av[0] : zero4), hi = pack_bf16x4(live ? av[1] : zero4);
        *(uint4*)(s_z + arow * kStrZ + 128 + acol) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    f32x4 acc1[8][2];
    bias_init<8>(acc1, a.b[0], 128 * w, lane);
    __syncthreads();

    // layer 1: 256 -> 512, wave w owns units 128w .. 128w+127
    layer_mma<kPacked, 8, 8, kPf1>(acc1, r1, A1, s_x, kStrX, lane);
    uint4 r2[kPf2][4];
    prefetch_a<kPacked, 4, kPf2>(r2, A2, lane);
    store_act<8>(acc1, s_h, kStrH, 128 * w, lane);
    f32x4 acc2[4][2];
    bias_init<4>(acc2, a.b[1], 64 * w, lane);
    __syncthreads();

    // layer 2: 512 -> 256, units 64w ..; its results replace the deep input
    layer_mma<kPacked, 4, 16, kPf2>(acc2, r2, A2, s_h, kStrH, lane);
    uint4 r3[kPf3][2];
    prefetch_a<kPacked, 2, kPf3>(r3, A3, lane);
    store_act<4>(acc2, s_x, kStrX, 64 * w, lane);
    f32x4 acc3[2][2];
    bias_init<2>(acc3, a.b[2], 32 * w, lane);
    __syncthreads();

    // layer 3: 256 -> 128, units 32w ..: the deep tower's output
    layer_mma<kPacked, 2, 8, kPf3>(acc3, r3, A3, s_x, kStrX, lane);
    uint4 r4[kPf4][1];
    prefetch_a<kPacked, 1, kPf4>(r4, A4, lane);
    if (a.deep_out) {
        const int m = lane & 15, g = lane >> 4;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int64_t b = b0 + 16 * s + m;
            if (b < a.B) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f32x4 v = acc3[t][s];
                    *(float4*)(a.deep_out + b * 128 + 32 * w + 16 * t + 4 * g) =
                        make_float4(fmaxf(v[0], 0.f), fmaxf(v[1], 0.f), fmaxf(v[2], 0.f), fmaxf(v[3], 0.f));
                }
            }
        }
    }
    store_act<2>(acc3, s_z, kStrZ, 32 * w, lane);
    f32x4 acc4[1][2];
    bias_init<1>(acc4, a.b[3], 16 * w, lane);
    __syncthreads();

    // layer 4: [deep, att] (176, zero-padded to 192) -> 64, units 16w ..
    layer_mma<kPacked, 1, 6, kPf4>(acc4, r4, A4, s_z, kStrZ, lane);
    // the logit: wo . relu(layer 4) + bo, a partial sum over each wave's units
    {
        const int m = lane & 15, g = lane >> 4;
        const f32x4 wo = *(const f32x4*)(a.wo + 16 * w + 4 * g);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) p += fmaxf(acc4[0][s][i], 0.f) * wo[i];
            p += __shfl_xor(p, 16, 64);
            p += __shfl_xor(p, 32, 64);
            if (g == 0) s_part[w][16 * s + m] = p;
        }
    }
    __syncthreads();
    if (tid < kM) {
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
    for (int idx = threadIdx.x; idx < kM * nout; idx += 64 * kWaves) {
        const int r = idx / nout, o = idx % nout;
        float acc = bias[o];
        const float* wr = W + (int64_t)o * nin;
        const float* x = in + r * nin;
        for (int i = 0; i < nin; ++i) acc = fmaf(wr[i], x[i], acc);
        out[r * ostr + o] = fmaxf(acc, 0.f);
    }
}

__global__ __launch_bounds__(64 * kWaves) void k_towers_f32(const TowerArgs a) {
    __shared__ float s_x[kM * 256];     // deep input, then layer 2
    __shared__ float s_h[kM * 512];     // layer 1, then layer 4
    __shared__ float s_z[kM * 176];     // [deep out, att]
    const int tid = threadIdx.x;
    const int64_t b0 = (int64_t)blockIdx.x * kM;
    for (int idx = tid; idx < kM * 256; idx += 64 * kWaves) {
        const int r = idx >> 8, c = idx & 255;
        const int64_t b = b0 + r;
        s_x[idx] = b < a.B ? a.pooled[b * a.pooled_ld + c] : 0.f;
    }
    for (int idx = tid; idx < kM * 48; idx += 64 * kWaves) {
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
        for (int idx = tid; idx < kM * 128; idx += 64 * kWaves) {
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

// One thread per 16-byte slot of the packed image: (layer, wave, K-step,
// tile, lane) -> 8 bf16 of one weight row, zeros past the row's end.
struct PackArgs {
    const uint16_t* w[4];
    uint4* out;
};

__global__ __launch_bounds__(256) void k_tower_pack(const PackArgs p) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= REC_TOWER_PACKED_BYTES / 16) return;
    const int f = d >> 6, lane = d & 63;
    int l = 0;
    while (l < 3 && f >= pack_base(l + 1)) ++l;
    const int r = f - pack_base(l);
    const int per_wave = kNK[l] * kNT[l];
    const int w = r / per_wave, ct = r % per_wave, c = ct / kNT[l], t = ct % kNT[l];
    const int row = kRowsPerWave[l] * w + 16 * t + (lane & 15), col = 32 * c + 8 * (lane >> 4);
    const uint16_t* W = l == 0 ? p.w[0] : l == 1 ? p.w[1] : l == 2 ? p.w[2] : p.w[3];
    p.out[d] = col < kLdw[l] ? *(const uint4*)(W + row * kLdw[l] + col) : make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t launch_towers(const TowerArgs& a, hipStream_t s) {
    const int64_t blocks = (a.B + kM - 1) / kM;
    if (a.dtype == REC_BF16_PACKED)
        hipLaunchKernelGGL(k_towers_bf16<true>, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, a);
    else if (a.dtype == REC_BF16)
        hipLaunchKernelGGL(k_towers_bf16<false>, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, a);
    else
        hipLaunchKernelGGL(k_towers_f32, dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tower_pack(const void* const w[4], void* packed, hipStream_t s) {
    PackArgs p;
    for (int l = 0; l < 4; ++l) p.w[l] = (const uint16_t*)w[l];
    p.out = (uint4*)packed;
    hipLaunchKernelGGL(k_tower_pack, dim3(REC_TOWER_PACKED_BYTES / 16 / 256), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace rec
