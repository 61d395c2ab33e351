// Matrix-core operand types and the bf16 epilogue shared by the attention
// MLP and the towers.
//
// v_mfma_f32_16x16x32_bf16 takes, per lane l = 16 g + m (g = 0..3):
//   A  8 bf16: row m of the 16 x 32 left tile, K elements 8g .. 8g+7
//   B  8 bf16: column m of the 32 x 16 right tile, K elements 8g .. 8g+7
//   C/D 4 fp32: column m of the 16 x 16 result, rows 4g .. 4g+3
// v_mfma_f32_16x16x16_bf16 takes the same layout with 4 bf16 per lane (K
// elements 4g .. 4g+3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));   // 4 bf16 bit patterns (16x16x16 operands)

// max(RNE(a), 0), max(RNE(b), 0) as a bf16 pair.  Rounding to nearest keeps
// the sign, so ReLU after rounding equals rounding after ReLU; on the bit
// patterns a negative bf16 (or -0) is a negative int16, so the ReLU is one
// packed integer max for two values.
__device__ inline uint32_t relu_pk_bf16(float a, float b) {
    bf16x2 p;
    p[0] = (__bf16)a;
    p[1] = (__bf16)b;
    s16x2 v = __builtin_bit_cast(s16x2, p);
    v = __builtin_elementwise_max(v, (s16x2){0, 0});
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace
}  // namespace rec
