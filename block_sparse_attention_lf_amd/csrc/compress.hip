// Token compression for hierarchical sparse attention (Light Forcing,
// technical summary 2.2 "token compression"; press summary section 3):
// mean pooling of the current chunk's queries per block, and of the history
// keys per block and per frame.
//
// Numerics: sums are accumulated in float64 and the mean is rounded once to
// float32, mean = (float)(sum / count). With bf16 (or fp32) inputs of the
// magnitudes used here the float64 sums are exact, so the result does not
// depend on summation order.
//
// Design (HBM-bound): one wavefront pools one block. Each lane loads 16 bytes
// per row group; a wave-wide load covers RPL full rows, and UNROLL loads are
// in flight before any arithmetic, so a wave keeps a whole 64-row block
// (16 KiB at D=128 bf16) in flight. A short xor-shuffle tree folds the row
// groups at the end of the block. The frame means come from a second, tiny
// pass over the float64 block sums (kept in the caller's workspace), so no
// workgroup ever needs another's partial result.
#include "lf_internal.h"

namespace lf {
namespace {

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

// Work items: first every history key block (b, h, f, j), then every query
// block (b, h, fc, j). Item order matches the output layouts, so an item's
// index is also its output row.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_blocks_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          float* __restrict__ q_blk, float* __restrict__ k_blk,
                                                          double* __restrict__ blk_sum, const KGeom g) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per 16-byte load
  constexpr int LPR = D / EPL;              // lanes per row
  constexpr int RPL = 64 / LPR;             // rows per wave-wide load
  constexpr int UNROLL = 16;
  static_assert(64 % LPR == 0, "row must map onto whole lanes");

  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t per_bh_k = (int64_t)g.Fh * g.nb;
  const int64_t n_k = (int64_t)g.B * g.H * per_bh_k;
  const int64_t n_q = (int64_t)g.B * g.H * g.nqb;
  if (item >= n_k + n_q) return;  // whole wave leaves; no barriers below

  const T* src;
  float* mean_dst;
  double* sum_dst = nullptr;
  int rows;
  if (item < n_k) {
    const int64_t bh = item / per_bh_k;
    const int rem = (int)(item - bh * per_bh_k);
    const int f = rem / g.nb, j = rem - (rem / g.nb) * g.nb;
    const int start = j * g.b;
    rows = min(g.b, g.T - start);
    src = k + ((bh * g.S + g.slot[f]) * (int64_t)g.T + start) * D;
    mean_dst = k_blk + item * D;
    sum_dst = blk_sum + item * D;
  } else {
    const int64_t it = item - n_k;
    const int64_t bh = it / g.nqb;
    const int qb = (int)(it - bh * g.nqb);
    const int fc = qb / g.nb, j = qb - fc * g.nb;
    rows = min(g.b, g.T - j * g.b);
    src = q + (bh * g.Lq + (int64_t)fc * g.T + (int64_t)j * g.b) * D;
    mean_dst = q_blk + it * D;
  }

  const int sub = lane / LPR;
  const int col = (lane % LPR) * EPL;
  double acc[EPL];
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
  if (lane < LPR) {
    const double count = (double)rows;
    float m[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) m[e] = (float)(acc[e] / count);
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(mean_dst + col + e) = make_float4(m[e], m[e + 1], m[e + 2], m[e + 3]);
    if (sum_dst) {
#pragma unroll
      for (int e = 0; e < EPL; e += 2)
        *reinterpret_cast<double2*>(sum_dst + col + e) = make_double2(acc[e], acc[e + 1]);
    }
  }
}

// Frame means from the float64 block sums: k_frm[f] = (sum_j blk_sum[f, j]) / T.
template <int D>
__global__ __launch_bounds__(64) void pool_frames_kernel(const double* __restrict__ blk_sum,
                                                         float* __restrict__ k_frm, const KGeom g) {
  const int64_t item = blockIdx.x;  // (b*H + h)*Fh + f
  const double* s = blk_sum + item * g.nb * D;
#pragma unroll
  for (int d = threadIdx.x; d < D; d += 64) {
    double acc = 0.0;
    for (int j = 0; j < g.nb; ++j) acc += s[(int64_t)j * D + d];
    k_frm[item * D + d] = (float)(acc / (double)g.T);
  }
}

template <typename T, int D>
hipError_t launch_typed(const KGeom& g, const void* q, const void* k, float* q_blk, float* k_blk, float* k_frm,
                        double* blk_sum, hipStream_t stream) {
  const int64_t items = (int64_t)g.B * g.H * (g.Fh + g.Fc) * g.nb;
  const int64_t wgs = (items + 3) / 4;
  hipLaunchKernelGGL((pool_blocks_kernel<T, D>), dim3((unsigned)wgs), dim3(256), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), q_blk, k_blk, blk_sum, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.Fh == 0) return e;
  hipLaunchKernelGGL((pool_frames_kernel<D>), dim3((unsigned)((int64_t)g.B * g.H * g.Fh)), dim3(64), 0, stream,
                     blk_sum, k_frm, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(const KGeom& g, int32_t dtype, const void* q, const void* k_cache, float* q_blk,
                           float* k_blk, float* k_frm, double* blk_sum, hipStream_t stream) {
  if (dtype == LF_BF16) {
    if (g.D == 128) return launch_typed<__bf16, 128>(g, q, k_cache, q_blk, k_blk, k_frm, blk_sum, stream);
    return launch_typed<__bf16, 64>(g, q, k_cache, q_blk, k_blk, k_frm, blk_sum, stream);
  }
  if (g.D == 128) return launch_typed<float, 128>(g, q, k_cache, q_blk, k_blk, k_frm, blk_sum, stream);
  return launch_typed<float, 64>(g, q, k_cache, q_blk, k_blk, k_frm, blk_sum, stream);
}

}  // namespace lf
