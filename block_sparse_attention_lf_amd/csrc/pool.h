// Block mean pooling shared by the compression kernels and the fused
// pool-and-select kernel (Light Forcing, technical summary 2.2 "token
// compression": mean pooling per block). Sums are float64, the mean is
// rounded once to float32: mean = (float)(sum / count).
#pragma once
#include "lf_internal.h"

namespace lf {

template <typename T>
__device__ inline void unpack16(const uint4& v, float* f);

template <>
__device__ inline void unpack16<float>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

template <>
__device__ inline void unpack16<__bf16>(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Float64 column sums of `rows` rows, over the DS columns starting at src
// (rows D elements apart; DS = D for whole rows, less for a column slice),
// reduced across the wavefront: on return every lane holds, for its columns
// col .. col+EPL-1 of the slice, the sums over all rows.
template <typename T, int D, int DS = D>
struct BlockPool {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per 16-byte load
  static constexpr int LPR = DS / EPL;             // lanes per row (slice)
  static constexpr int RPL = 64 / LPR;             // rows per wave-wide load
  // loads in flight per lane: 16 (bf16) / 8 (f32) for whole rows, which
  // keeps the registers under 128; a slice takes at most a 64-row block's worth
  static constexpr int UNROLL_MAX = sizeof(T) == 2 ? 16 : 8;
  static constexpr int UNROLL_BLOCK = (64 + RPL - 1) / RPL;
  static constexpr int UNROLL = DS == D || UNROLL_BLOCK > UNROLL_MAX ? UNROLL_MAX : UNROLL_BLOCK;
  static_assert(64 % LPR == 0 && D % DS == 0, "row slice must map onto whole lanes");

  __device__ static void sums(const T* src, int rows, int lane, double (&acc)[EPL]) {
    const int sub = lane / LPR;
    const int col = (lane % LPR) * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
    for (int r0 = 0; r0 < rows; r0 += RPL * UNROLL) {
      uint4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int r = r0 + u * RPL + sub;
        if (r < rows)
          v[u] = *reinterpret_cast<const uint4*>(src + (int64_t)r * D + col);
        else
          v[u] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float f[EPL];
        unpack16<T>(v[u], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += (double)f[e];
      }
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
  }

  // mean = (float)(sum / count), written by the lanes of the first row group.
  __device__ static void store_mean(float* dst, const double (&acc)[EPL], int count, int lane) {
    if (lane >= LPR) return;
    const int col = lane * EPL;
    float m[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) m[e] = (float)(acc[e] / (double)count);
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(dst + col + e) = make_float4(m[e], m[e + 1], m[e + 2], m[e + 3]);
  }
};

}  // namespace lf
