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
// Design (HBM-bound, one launch). A wavefront pools one block: each lane
// loads 16 bytes per row group, a wave-wide load covers RPL full rows, and
// UNROLL loads are in flight before any arithmetic, so a wave keeps a whole
// 64-row block (16 KiB at D=128 bf16) in flight; a short xor-shuffle tree
// folds the row groups at the end. Workgroups of the first kind each own one
// history frame of one (batch, head): their NWAVE wavefronts take every
// NWAVE-th block of the frame (a frame of 25-29 blocks is then at most two
// round trips to memory per wavefront), write its mean, and keep running
// float64 column sums, which the workgroup adds up through LDS, in wavefront
// order, into the frame mean. The remaining workgroups pool QWAVE query
// blocks each (their other wavefronts leave at once): fewer blocks per
// workgroup spread the queries over the CUs the frames leave idle. No partial
// result ever crosses workgroups, so there is no second pass and no
// workspace.
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

// Float64 column sums of `rows` rows of D elements starting at src, reduced
// across the wavefront: on return every lane holds, for its columns
// col .. col+EPL-1, the sums over all rows.
template <typename T, int D>
struct BlockPool {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per 16-byte load
  static constexpr int LPR = D / EPL;              // lanes per row
  static constexpr int RPL = 64 / LPR;             // rows per wave-wide load
  static constexpr int UNROLL = sizeof(T) == 2 ? 16 : 8;  // loads in flight per lane (fits 128 registers)
  static_assert(64 % LPR == 0, "row must map onto whole lanes");

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

constexpr int NWAVE = 16;  // wavefronts per workgroup
constexpr int QWAVE = 4;   // query blocks per query workgroup

// Workgroups [0, B*H*Fh) own one history frame each, (b*H + h)*Fh + f; the
// rest own QWAVE consecutive query blocks each. Output rows follow the
// layouts: k_blk row (bh*Fh + f)*nb + j, k_frm row bh*Fh + f, q_blk row
// bh*nqb + qb.
template <typename T, int D>
__global__ __launch_bounds__(64 * NWAVE) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   float* __restrict__ q_blk, float* __restrict__ k_blk,
                                                   float* __restrict__ k_frm, const KGeom g) {
  using P = BlockPool<T, D>;
  constexpr int EPL = P::EPL, LPR = P::LPR;
  __shared__ double part[NWAVE][D];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t n_frames = (int64_t)g.B * g.H * g.Fh;
  const int64_t wg = blockIdx.x;
  double acc[EPL];

  if (wg < n_frames) {
    const int64_t bh = wg / g.Fh;
    const int f = (int)(wg - bh * g.Fh);
    const T* frame = k + (bh * g.S + g.slot[f]) * (int64_t)g.T * D;
    double fsum[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) fsum[e] = 0.0;
    for (int j = wv; j < g.nb; j += NWAVE) {
      const int start = j * g.b, rows = min(g.b, g.T - start);
      P::sums(frame + (int64_t)start * D, rows, lane, acc);
      P::store_mean(k_blk + (wg * g.nb + j) * D, acc, rows, lane);
#pragma unroll
      for (int e = 0; e < EPL; ++e) fsum[e] += acc[e];
    }
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[wv][lane * EPL + e] = fsum[e];
    }
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += 64 * NWAVE) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) t += part[w][d];
      k_frm[wg * D + d] = (float)(t / (double)g.T);
    }
    return;
  }

  const int64_t it = (wg - n_frames) * QWAVE + wv;  // query block item, (b*H + h)*nqb + qb
  if (wv >= QWAVE || it >= (int64_t)g.B * g.H * g.nqb) return;  // whole wave leaves; no barriers on this path
  const int64_t bh = it / g.nqb;
  const int qb = (int)(it - bh * g.nqb);
  const int fc = qb / g.nb, j = qb - fc * g.nb;
  const int rows = min(g.b, g.T - j * g.b);
  P::sums(q + (bh * g.Lq + (int64_t)fc * g.T + (int64_t)j * g.b) * D, rows, lane, acc);
  P::store_mean(q_blk + it * D, acc, rows, lane);
}

template <typename T, int D>
hipError_t launch_typed(const KGeom& g, const void* q, const void* k, float* q_blk, float* k_blk, float* k_frm,
                        hipStream_t stream) {
  const int64_t n_frames = (int64_t)g.B * g.H * g.Fh;
  const int64_t n_q = ((int64_t)g.B * g.H * g.nqb + QWAVE - 1) / QWAVE;
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3((unsigned)(n_frames + n_q)), dim3(64 * NWAVE), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), q_blk, k_blk, k_frm, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(const KGeom& g, int32_t dtype, const void* q, const void* k_cache, float* q_blk,
                           float* k_blk, float* k_frm, hipStream_t stream) {
  if (dtype == LF_BF16) {
    if (g.D == 128) return launch_typed<__bf16, 128>(g, q, k_cache, q_blk, k_blk, k_frm, stream);
    return launch_typed<__bf16, 64>(g, q, k_cache, q_blk, k_blk, k_frm, stream);
  }
  if (g.D == 128) return launch_typed<float, 128>(g, q, k_cache, q_blk, k_blk, k_frm, stream);
  return launch_typed<float, 64>(g, q, k_cache, q_blk, k_blk, k_frm, stream);
}

}  // namespace lf
