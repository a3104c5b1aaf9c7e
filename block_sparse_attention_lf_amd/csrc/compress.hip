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
// loads 16 bytes per row group, a wave-wide load covers RPL rows, and up to
// a whole 64-row block (16 KiB at D=128 bf16) is in flight before any
// arithmetic; a short xor-shuffle tree folds the row groups at the end.
// Workgroups of the first kind each own one history frame of one (batch,
// head), or one column slice of it: their NWAVE wavefronts take every
// NWAVE-th block of the frame, write its mean (or the slice of it), and keep
// running float64 column sums, which the workgroup adds up through LDS, in
// wavefront order, into the frame mean. The remaining workgroups pool QW
// query blocks each, one per wavefront. No partial result ever crosses
// workgroups, so there is no second pass and no workspace.
// Two launch shapes: a frame pooled whole spreads the queries thinly (four
// blocks per workgroup) over the CUs the frames leave idle; when the grid is
// small enough for every workgroup to get a CU of its own, each frame is
// split into 128-byte column slices (one cache line of every row) so its
// reads and float64 sums spread over several CUs, and the query workgroups
// take sixteen blocks each. Slicing by columns keeps every column's sum in
// one workgroup: both shapes give the same bits.
#include <atomic>

#include "pool.h"

namespace lf {
namespace {

constexpr int NWAVE = 16;  // wavefronts per workgroup

// Column slices per frame in the sliced shape: one 128-byte cache line of
// each row per slice.
template <typename T, int D>
constexpr int kSlices = D * (int)sizeof(T) / 128 > 1 ? D * (int)sizeof(T) / 128 : 1;

// One history frame, or the DS-column slice of it that `frame` points at
// (rows D elements apart), pooled by a whole workgroup: the (slice of the)
// mean of block j to blk_dst + j*D, of the frame mean to frm_dst.
template <typename T, int D, int DS>
__device__ inline void pool_frame(const T* frame, float* blk_dst, float* frm_dst, const KGeom& g,
                                  double (&part)[NWAVE][DS], int lane, int wv) {
  using P = BlockPool<T, D, DS>;
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
  for (int d = threadIdx.x; d < DS; d += 64 * NWAVE) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) t += part[w][d];
    frm_dst[d] = (float)(t / (double)g.T);
  }
}

// Workgroups [0, B*H*Fh*NS) own one history frame, or one of its NS column
// slices, each: (((b*H + h)*Fh + f)*NS + slice); the rest own QW consecutive
// query blocks each. Output rows follow the layouts: k_blk row
// (bh*Fh + f)*nb + j, k_frm row bh*Fh + f, q_blk row bh*nqb + qb.
template <typename T, int D, int NS, int QW>
__global__ __launch_bounds__(64 * NWAVE) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   float* __restrict__ q_blk, float* __restrict__ k_blk,
                                                   float* __restrict__ k_frm, const KGeom g) {
  static_assert(QW <= NWAVE && D % NS == 0, "launch shape");
  using P = BlockPool<T, D>;
  constexpr int DS = D / NS;
  __shared__ double part[NWAVE][DS];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t n_parts = (int64_t)g.B * g.H * g.Fh * NS;
  const int64_t wg = blockIdx.x;

  if (wg < n_parts) {
    const int64_t fw = wg / NS;  // (b*H + h)*Fh + f
    const int c0 = (int)(wg - fw * NS) * DS;
    const int64_t bh = fw / g.Fh;
    const int f = (int)(fw - bh * g.Fh);
    pool_frame<T, D, DS>(k + (bh * g.S + g.slot[f]) * (int64_t)g.T * D + c0, k_blk + fw * g.nb * D + c0,
                         k_frm + fw * D + c0, g, part, lane, wv);
    return;
  }

  const int64_t it = (wg - n_parts) * QW + wv;  // query block item, (b*H + h)*nqb + qb
  if (wv >= QW || it >= (int64_t)g.B * g.H * g.nqb) return;  // whole wave leaves; no barriers on this path
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
  pool_frame<T, D, D>(k + row * (int64_t)g.T * D, kp_blk + row * g.nb * D, kp_frm + row * D, g, part,
                      threadIdx.x & 63, threadIdx.x >> 6);
}

// Compute units of the current device (queried once per device).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    cached[dev].store(n, std::memory_order_relaxed);
  return n > 0 ? n : 0;
}

template <typename T, int D>
hipError_t launch_typed(const KGeom& g, const void* q, const void* k, float* q_blk, float* k_blk, float* k_frm,
                        hipStream_t stream) {
  constexpr int NS = kSlices<T, D>;
  const int64_t n_frames = (int64_t)g.B * g.H * g.Fh, n_qblk = (int64_t)g.B * g.H * g.nqb;
  // Sliced shape when every workgroup of it gets a CU of its own (one
  // 1024-thread workgroup fits a CU); otherwise whole frames.
  if constexpr (NS > 1) {
    const int64_t sliced = n_frames * NS + (n_qblk + NWAVE - 1) / NWAVE;
    if (sliced <= cu_count()) {
      hipLaunchKernelGGL((pool_kernel<T, D, NS, NWAVE>), dim3((unsigned)sliced), dim3(64 * NWAVE), 0, stream,
                         static_cast<const T*>(q), static_cast<const T*>(k), q_blk, k_blk, k_frm, g);
      return hipGetLastError();
    }
  }
  constexpr int QW = 4;
  hipLaunchKernelGGL((pool_kernel<T, D, 1, QW>), dim3((unsigned)(n_frames + (n_qblk + QW - 1) / QW)),
                     dim3(64 * NWAVE), 0, stream, static_cast<const T*>(q), static_cast<const T*>(k), q_blk, k_blk,
                     k_frm, g);
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
