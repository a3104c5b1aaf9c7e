// MFMA operand types and layout helpers shared by the attention kernels
// (CDNA4 / gfx950, v_mfma_f32_32x32x16_bf16).
#pragma once
#include "lf_internal.h"

namespace lf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;

// Row index held by accumulator register r of lane half h in a 32x32 MFMA
// output: 8*(r/4) + 4*h + r%4 (the column is the lane index mod 32).
__device__ inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

}  // namespace lf
