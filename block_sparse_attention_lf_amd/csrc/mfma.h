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

// LDS layout of 256-byte bf16 rows (d = 128) without padding: the 16-byte
// chunk c of row r is stored at chunk position c ^ lds_swizzle(r). Reads of
// 32 rows at one chunk (MFMA operand rows) and the transposing reads of 8
// rows at 16 consecutive columns then spread over all banks.
__device__ inline int lds_swizzle(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt == 0 only.
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);

// Buffer resource word 3 for raw (untyped) dword access on this GPU family.
constexpr int kRawBufferFlags = 0x00020000;

// A wave-uniform pointer moved to scalar registers (so address arithmetic on
// it stays scalar and loads can use the scalar-base form).
template <typename P>
__device__ inline P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// XCD-aware work order. The hardware deals consecutive workgroup ids
// round-robin to the 8 XCDs (each with its own L2); this maps workgroup id
// wg of nwg to a work item such that each XCD gets one contiguous range of
// items, so neighbouring items (the query blocks of one head, which read
// the same keys and values) share one L2.
__device__ inline int xcd_item(int wg, int nwg) {
  const int xcd = wg & 7, idx = wg >> 3, per = nwg >> 3, rem = nwg & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

}  // namespace lf
