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
#include "pool.h"

namespace lf {
namespace {

constexpr int NWAVE = 16;  // wavefronts per workgroup
constexpr int QWAVE = 4;   // query blocks per query workgroup

// One history frame (T rows of D from `frame`) pooled by a whole workgroup:
// block means to blk_dst[j], the frame mean to frm_dst.
template <typename T, int D>
__device__ inline void pool_frame(const T* frame, float* blk_dst, float* frm_dst, const KGeom& g,
                                  double (&part)[NWAVE][D], int lane, int wv) {
  using P = BlockPool<T, D>;
  constexpr int EPL = P::EPL, LPR = P::LPR;
  double acc[EPL], fsum[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) fsum[e] = 0.0;
  for (int j = wv; j < g.nb; j += NWAVE) {
    const int start = j * g.b, rows = min(g.b, g.T - start);
    P::sums(frame + (int64_t)start * D, rows, lane, acc);
    P::store_mean(blk_dst + (int64_t)j * D, acc, rows, lane);
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
    frm_dst[d] = (float)(t / (double)g.T);
  }
}

// Workgroups [0, B*H*Fh) own one history frame each, (b*H + h)*Fh + f; the
// rest own QWAVE consecutive query blocks each. Output rows follow the
// layouts: k_blk row (bh*Fh + f)*nb + j, k_frm row bh*Fh + f, q_blk row
// bh*nqb + qb.
template <typename T, int D>
__global__ __launch_bounds__(64 * NWAVE) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   float* __restrict__ q_blk, float* __restrict__ k_blk,
                                                   float* __restrict__ k_frm, const KGeom g) {
  using P = BlockPool<T, D>;
  __shared__ double part[NWAVE][D];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t n_frames = (int64_t)g.B * g.H * g.Fh;
  const int64_t wg = blockIdx.x;

  if (wg < n_frames) {
    const int64_t bh = wg / g.Fh;
    const int f = (int)(wg - bh * g.Fh);
    pool_frame<T, D>(k + (bh * g.S + g.slot[f]) * (int64_t)g.T * D, k_blk + wg * g.nb * D, k_frm + wg * D, g, part,
                     lane, wv);
    return;
  }

  const int64_t it = (wg - n_frames) * QWAVE + wv;  // query block item, (b*H + h)*nqb + qb
  if (wv >= QWAVE || it >= (int64_t)g.B * g.H * g.nqb) return;  // whole wave leaves; no barriers on this path
  const int64_t bh = it / g.nqb;
  const int qb = (int)(it - bh * g.nqb);
  const int fc = qb / g.nb, j = qb - fc * g.nb;
  const int rows = min(g.b, g.T - j * g.b);
  double acc[P::EPL];
  P::sums(q + (bh * g.Lq + (int64_t)fc * g.T + (int64_t)j * g.b) * D, rows, lane, acc);
  P::store_mean(q_blk + it * D, acc, rows, lane);
}

// Pool-on-commit: workgroup (bh, i) pools the frame in cache slot
// g.slot[i] (i < g.Fh, the number of slots named) into the slot-indexed
// pooled cache: kp_blk row (bh*S + slot)*nb + j, kp_frm row bh*S + slot.
template <typename T, int D>
__global__ __launch_bounds__(64 * NWAVE) void pool_slots_kernel(const T* __restrict__ k, float* __restrict__ kp_blk,
                                                         float* __restrict__ kp_frm, const KGeom g) {
  __shared__ double part[NWAVE][D];
  const int64_t bh = blockIdx.x / g.Fh;
  const int i = (int)(blockIdx.x - bh * g.Fh);
  const int64_t row = bh * g.S + g.slot[i];
  pool_frame<T, D>(k + row * (int64_t)g.T * D, kp_blk + row * g.nb * D, kp_frm + row * D, g, part,
                   threadIdx.x & 63, threadIdx.x >> 6);
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

template <typename T, int D>
hipError_t launch_slots_typed(const KGeom& g, const void* k, float* kp_blk, float* kp_frm, hipStream_t stream) {
  hipLaunchKernelGGL((pool_slots_kernel<T, D>), dim3((unsigned)((int64_t)g.B * g.H * g.Fh)), dim3(64 * NWAVE), 0,
                     stream, static_cast<const T*>(k), kp_blk, kp_frm, g);
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

hipError_t launch_pool_slots(const KGeom& g, int32_t dtype, const void* k_cache, float* kp_blk, float* kp_frm,
                             hipStream_t stream) {
  if (dtype == LF_BF16) {
    if (g.D == 128) return launch_slots_typed<__bf16, 128>(g, k_cache, kp_blk, kp_frm, stream);
    return launch_slots_typed<__bf16, 64>(g, k_cache, kp_blk, kp_frm, stream);
  }
  if (g.D == 128) return launch_slots_typed<float, 128>(g, k_cache, kp_blk, kp_frm, stream);
  return launch_slots_typed<float, 64>(g, k_cache, kp_blk, kp_frm, stream);
}

}  // namespace lf
