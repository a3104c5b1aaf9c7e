// Two-stage mask selection for hierarchical sparse attention (Light Forcing,
// technical summary 2.2 "two-stage mask selection"; press summary section 3):
// per query block, rank the non-sink history frames by the inner product of
// the pooled query with the frame-level keys, keep the top kf; inside each
// kept frame rank its blocks by the block-level keys, keep the top kb. The
// sink frames are attended in full. Output: ascending logical block ids.
//
// Numerics: scores are float64 dot products of the float32 pooled vectors
// (every product is exact in float64). The two-stage selection sums each dot
// product as 8 partial sums over consecutive ranges of d (each ascending),
// combined by a pairwise butterfly that leaves the same bits in all 8 lanes;
// the single-level selection sums in ascending d. A candidate is kept when
// fewer than k others rank above it, where c ranks above c' if its score is
// larger, or equal with a lower index. That is exactly "stable sort
// descending, take the first k" without sorting.
//
// Design: one workgroup of two wavefronts per (batch, head, query block).
// Each dot product is shared by 8 lanes (each holds its D/8 channels of the
// pooled query in registers; the partial sums meet through DPP lane moves),
// so a workgroup scores 16 candidates per round with dependent chains of D/8
// fused multiply-adds, and the key slices of four rounds are loaded before
// any is summed. The frame candidates are scored, ranked against the scores
// kept in LDS, and then the blocks of all kept frames are scored as one batch
// (up to 1024 at a time) and ranked inside their frame; kept ids are
// compacted in ascending order with a ballot and a prefix popcount. The whole
// step reads O(kf*nb + Fh) pooled vectors per query block, independent of how
// long the history is beyond that.
#include "pool.h"

namespace lf {
namespace {

template <int D>
__device__ inline double dot_f64(const float* __restrict__ qv_lds, const float* __restrict__ k) {
  double acc = 0.0;
#pragma unroll 8
  for (int d = 0; d < D; d += 4) {
    const float4 kv = *reinterpret_cast<const float4*>(k + d);
    acc = fma((double)qv_lds[d], (double)kv.x, acc);
    acc = fma((double)qv_lds[d + 1], (double)kv.y, acc);
    acc = fma((double)qv_lds[d + 2], (double)kv.z, acc);
    acc = fma((double)qv_lds[d + 3], (double)kv.w, acc);
  }
  return acc;
}

// Lanes sharing one dot product, candidates per wavefront round, and the
// number of block candidates scored per batch.
constexpr int kDotLanes = 8;
constexpr int kPerRound = 64 / kDotLanes;
constexpr int kBlockBatch = 1024;
// Wavefronts per query block in the two-stage selection (two measured
// 4-11% faster than one; four leave too few workgroups resident per CU).
constexpr int kSelectWaves = 2;
static_assert(LF_MAX_BLOCKS_PER_FRAME <= kBlockBatch, "one frame's blocks must fit a batch");

// v of another lane of the same row of 16 lanes, moved by the DPP control
// CTRL (a register move between lanes, no LDS round trip), per 32-bit half.
template <int CTRL>
__device__ inline double dpp_move(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i of 8 <- lane 7-i

// Dot products of the pooled query with key rows, each shared by the
// kDotLanes lanes of one candidate: lane `part` sums d in [part*D/8,
// (part+1)*D/8) in ascending order, then a butterfly adds the partial sums:
// pairs (lane ^ 1), then (lane ^ 2), then the two quads of the group (after
// two steps all lanes of a quad hold the same value, so the mirrored lane
// stands for its quad). Every lane of the group returns the same value
// (a + b == b + a exactly). All 64 lanes must take part (lanes exchange
// values). The lane's slice of the query lives in registers (QSlice); the
// key slices of several candidates are loaded before any is summed, so one
// memory round trip serves several rounds.
template <int D>
struct QSlice {
  static constexpr int SPAN = D / kDotLanes;
  static_assert(SPAN % 4 == 0, "each lane reads whole float4s");
  double q[SPAN];
  __device__ void load(const float* __restrict__ qv_lds, int part) {
#pragma unroll
    for (int d = 0; d < SPAN; ++d) q[d] = (double)qv_lds[part * SPAN + d];
  }
  // this lane's slice of key row k
  __device__ static void load_key(const float* __restrict__ k, int part, float4 (&kv)[SPAN / 4]) {
#pragma unroll
    for (int t = 0; t < SPAN / 4; ++t) kv[t] = *reinterpret_cast<const float4*>(k + part * SPAN + 4 * t);
  }
  __device__ double dot(const float4 (&kv)[SPAN / 4]) const {
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < SPAN / 4; ++t) {
      acc = fma(q[4 * t], (double)kv[t].x, acc);
      acc = fma(q[4 * t + 1], (double)kv[t].y, acc);
      acc = fma(q[4 * t + 2], (double)kv[t].z, acc);
      acc = fma(q[4 * t + 3], (double)kv[t].w, acc);
    }
    static_assert(kDotLanes == 8, "the butterfly below covers groups of 8 lanes");
    acc += dpp_move<kDppXor1>(acc);
    acc += dpp_move<kDppXor2>(acc);
    acc += dpp_move<kDppHalfMirror>(acc);
    return acc;
  }
};
// Rounds of kPerRound candidates whose key slices are in flight together.
constexpr int kRoundsInFlight = 4;

// keep[c] = 1 iff fewer than k candidates rank above c (thread t of nt
// takes c = t, t + nt, ...).
__device__ inline void rank_keep(const double* score, int n, int k, unsigned char* keep, int t, int nt) {
  for (int c = t; c < n; c += nt) {
    const double s = score[c];
    int above = 0;
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
      const double v = score[i];
      above += (v > s) || (v == s && i < c);
    }
    keep[c] = above < k;
  }
}

// Pooled-key row of history frame f: per logical frame (bh*Fh + f) as
// lf_compress writes them, or per cache slot (bh*S + slot[f]) as the
// commit-time pooling keeps them.
__device__ inline int64_t key_row(bool by_slot, const KGeom& g, int64_t bh, int f) {
  return by_slot ? bh * g.S + g.slot[f] : bh * g.Fh + f;
}

// FUSED = false: pooled queries q_blk and pooled keys per logical history
// frame, as lf_compress writes them. FUSED = true: the query block is pooled
// here from q (and optionally written to q_blk_out), and the pooled keys come
// from the slot-indexed cache filled on commit. NWS wavefronts per query
// block: a round scores kPerRound candidates per wavefront, and the bf16
// query block's rows are split between the wavefronts (float64 partial sums
// of bf16 values are exact, so the split does not change the mean; float32
// queries are pooled by one wavefront, in lf_compress's order).
template <int D, bool FUSED, typename T, int NWS>
__global__ __launch_bounds__(64 * NWS) void select_kernel(const float* __restrict__ q_blk, const T* __restrict__ q,
                                                          const float* __restrict__ k_blk,
                                                          const float* __restrict__ k_frm, const KGeom g, int kf,
                                                          int kb, int kf_stride, int32_t* __restrict__ sel_frames,
                                                          int32_t* __restrict__ sel_blocks,
                                                          int32_t* __restrict__ n_sel, int max_sel,
                                                          float* __restrict__ q_blk_out) {
  constexpr int NT = 64 * NWS;
  constexpr int PR = kPerRound * NWS;  // candidates per round
  __shared__ __attribute__((aligned(16))) float qv[D];
  __shared__ double fscore[LF_MAX_FRAMES];
  __shared__ unsigned char fkeep[LF_MAX_FRAMES];
  __shared__ double bscore[kBlockBatch];
  __shared__ unsigned char bkeep[kBlockBatch];
  __shared__ int bframe[LF_MAX_FRAMES];
  __shared__ double qpart[FUSED && NWS > 1 ? NWS : 1][FUSED && NWS > 1 ? D : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = lane % kDotLanes, sub = wv * kPerRound + lane / kDotLanes;  // candidate slot in a round
  const int64_t item = blockIdx.x;  // (b*H + h)*nqb + qb
  const int64_t bh = item / g.nqb;
  const int nb = g.nb, ns = g.ns;
  constexpr int KV = QSlice<D>::SPAN / 4;

  // Stage 1 key slices, kRoundsInFlight rounds of PR frame candidates from
  // candidate r0 on (lanes past the last candidate load the last one and
  // drop it). The first batch is loaded before the query is read or pooled:
  // it does not depend on it, so the two memory round trips overlap.
  const int ncand = g.Fh - ns;
  float4 kv1[kRoundsInFlight][KV];
  const auto load_frames = [&](int r0) {
#pragma unroll
    for (int u = 0; u < kRoundsInFlight; ++u) {
      if (r0 + u * PR + wv * kPerRound >= ncand) break;  // uniform over the wavefront
      const int c = min(r0 + u * PR + sub, ncand - 1);
      QSlice<D>::load_key(k_frm + key_row(FUSED, g, bh, ns + c) * D, part, kv1[u]);
    }
  };
  load_frames(0);

  if constexpr (FUSED) {
    using P = BlockPool<T, D>;
    const int qb = (int)(item - bh * g.nqb);
    const int fc = qb / nb, jq = qb - fc * nb;
    const int rows = min(g.b, g.T - jq * g.b);
    const T* src = q + (bh * g.Lq + (int64_t)fc * g.T + (int64_t)jq * g.b) * D;
    if constexpr (NWS > 1 && sizeof(T) == 2) {
      // wavefront w sums rows [w*RW, w*RW + RW) (RW a multiple of a load's rows)
      const int per = (rows + NWS - 1) / NWS;
      const int RW = (per + P::RPL - 1) / P::RPL * P::RPL;
      const int r0 = wv * RW, nr = max(0, min(RW, rows - r0));
      double acc[P::EPL];
      P::sums(src + (int64_t)r0 * D, nr, lane, acc);
      if (lane < P::LPR) {
#pragma unroll
        for (int e = 0; e < P::EPL; ++e) qpart[wv][lane * P::EPL + e] = acc[e];
      }
      __syncthreads();
      for (int d = tid; d < D; d += NT) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < NWS; ++w) t += qpart[w][d];
        const float m = (float)(t / (double)rows);
        qv[d] = m;
        if (q_blk_out != nullptr) q_blk_out[item * D + d] = m;
      }
    } else {
      if (wv == 0) {
        double acc[P::EPL];
        P::sums(src, rows, lane, acc);
        if (lane < P::LPR) {
#pragma unroll
          for (int e = 0; e < P::EPL; ++e) qv[lane * P::EPL + e] = (float)(acc[e] / (double)rows);
        }
        if (q_blk_out != nullptr) P::store_mean(q_blk_out + item * D, acc, rows, lane);
      }
    }
  } else {
    for (int d = tid; d < D; d += NT) qv[d] = q_blk[item * D + d];
  }
  __syncthreads();

  int32_t* out = sel_blocks + item * max_sel;
  for (int i = tid; i < ns * nb; i += NT) out[i] = i;  // sink frames in full
  int pos = ns * nb;  // (kept by wavefront 0, which writes the kept ids)

  QSlice<D> qs;
  qs.load(qv, part);

  // Stage 1: frame scores, one batch of rounds at a time (the first batch
  // is already in flight).
  for (int r0 = 0; r0 < ncand; r0 += PR * kRoundsInFlight) {
    if (r0 > 0) load_frames(r0);
#pragma unroll
    for (int u = 0; u < kRoundsInFlight; ++u) {
      if (r0 + u * PR + wv * kPerRound >= ncand) break;
      const int c = r0 + u * PR + sub;
      const double sc = qs.dot(kv1[u]);
      if (c < ncand && part == 0) fscore[c] = sc;
    }
  }
  __syncthreads();
  rank_keep(fscore, ncand, kf, fkeep, tid, NT);
  __syncthreads();

  // Stage 2: the blocks of the kept frames, in batches of whole frames.
  int c = 0, nf = 0;
  for (;;) {
    int nbf = 0;  // kept frames in this batch (uniform across the workgroup)
    while (c < ncand && (nbf + 1) * nb <= kBlockBatch) {
      if (fkeep[c]) {
        const int f = ns + c;
        if (tid == 0) bframe[nbf] = f;
        if (sel_frames != nullptr && tid == 0 && nf < kf_stride) sel_frames[item * kf_stride + nf] = f;
        ++nbf;
        ++nf;
      }
      ++c;
    }
    if (nbf == 0) break;
    __syncthreads();  // bframe is visible
    const int nc = nbf * nb;
    for (int r0 = 0; r0 < nc; r0 += PR * kRoundsInFlight) {
      float4 kv[kRoundsInFlight][KV];
#pragma unroll
      for (int u = 0; u < kRoundsInFlight; ++u) {
        if (r0 + u * PR + wv * kPerRound >= nc) break;  // uniform over the wavefront
        const int xc = min(r0 + u * PR + sub, nc - 1);
        const int fi = xc / nb, j = xc - fi * nb;
        QSlice<D>::load_key(k_blk + (key_row(FUSED, g, bh, bframe[fi]) * nb + j) * (int64_t)D, part, kv[u]);
      }
#pragma unroll
      for (int u = 0; u < kRoundsInFlight; ++u) {
        if (r0 + u * PR + wv * kPerRound >= nc) break;
        const int x = r0 + u * PR + sub;
        const double sc = qs.dot(kv[u]);
        if (x < nc && part == 0) bscore[x] = sc;
      }
    }
    __syncthreads();
    for (int x = tid; x < nc; x += NT) {  // rank inside the candidate's frame
      const int fi = x / nb, j = x - fi * nb;
      const double* seg = bscore + fi * nb;
      const double sc = seg[j];
      int above = 0;
#pragma unroll 8
      for (int i = 0; i < nb; ++i) {
        const double t = seg[i];
        above += (t > sc) || (t == sc && i < j);
      }
      bkeep[x] = above < kb;
    }
    __syncthreads();
    if (wv == 0) {
      for (int x0 = 0; x0 < nc; x0 += 64) {
        const int x = x0 + lane;
        const bool take = x < nc && bkeep[x];
        const unsigned long long m = __ballot(take);
        const int at = pos + __popcll(m & ((1ull << lane) - 1ull));
        if (take && at < max_sel) {  // bound holds unless scores are NaN
          const int fi = x / nb;
          out[at] = bframe[fi] * nb + (x - fi * nb);
        }
        pos = min(pos + __popcll(m), max_sel);
      }
    }
    __syncthreads();  // bframe/bscore/bkeep are rewritten by the next batch
  }
  if (sel_frames != nullptr)
    for (int i = nf + tid; i < kf_stride; i += NT) sel_frames[item * kf_stride + i] = -1;
  if (wv == 0) {
    for (int i = pos + lane; i < max_sel; i += 64) out[i] = -1;
    if (lane == 0) n_sel[item] = pos;
  }
}

// Order-preserving map of a float64 score to an unsigned key (larger score,
// larger key; inputs are finite).
__device__ inline uint64_t score_key(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}

// Single-level ("1D") selection (press summary, section 4, the ablation
// baseline): one top-k over every non-sink history block, no frame stage.
// One wavefront per query block. Scores go to LDS as order-preserving keys;
// the k-th largest key T is found bit by bit from the top (is there at least
// k keys >= T | bit?), each count a sum of ballots; then keys > T are kept
// and keys == T fill the rest in ascending index, i.e. exactly "stable sort
// descending, take the first k". Ids ascend by construction.
template <int D>
__global__ __launch_bounds__(64) void select_blocks_kernel(const float* __restrict__ q_blk,
                                                           const float* __restrict__ k_blk, const KGeom g, int k,
                                                           int32_t* __restrict__ sel_blocks,
                                                           int32_t* __restrict__ n_sel, int max_sel) {
  __shared__ __attribute__((aligned(16))) float qv[D];
  __shared__ uint64_t key[LF_MAX_CANDIDATES_1D];

  const int lane = threadIdx.x;
  const int64_t item = blockIdx.x;  // (b*H + h)*nqb + qb
  const int64_t bh = item / g.nqb;
  const int nb = g.nb, ns = g.ns;
  for (int d = lane; d < D; d += 64) qv[d] = q_blk[item * D + d];
  __syncthreads();

  int32_t* out = sel_blocks + item * max_sel;
  for (int i = lane; i < ns * nb; i += 64) out[i] = i;  // sink frames in full
  const int base = ns * nb;
  const int ncand = (g.Fh - ns) * nb;
  const float* rows = k_blk + (bh * g.Fh + ns) * (int64_t)nb * D;
  for (int c = lane; c < ncand; c += 64) key[c] = score_key(dot_f64<D>(qv, rows + (int64_t)c * D));
  __syncthreads();

  // k-th largest key
  uint64_t t = 0;
  if (k > 0) {
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = t | (1ull << bit);
      int cnt = 0;
      for (int c0 = 0; c0 < ncand; c0 += 64) {
        const int c = c0 + lane;
        cnt += __popcll(__ballot(c < ncand && key[c] >= cand));
      }
      if (cnt >= k) t = cand;
    }
  }
  int above = 0;  // keys strictly above t
  for (int c0 = 0; c0 < ncand; c0 += 64) {
    const int c = c0 + lane;
    above += __popcll(__ballot(k > 0 && c < ncand && key[c] > t));
  }
  int pos = base, ties_left = k - above;
  for (int c0 = 0; c0 < ncand; c0 += 64) {
    const int c = c0 + lane;
    const bool valid = k > 0 && c < ncand;
    const bool tie = valid && key[c] == t;
    const unsigned long long lt = (1ull << lane) - 1ull;
    const unsigned long long tm = __ballot(tie);
    const bool take = valid && (key[c] > t || (tie && __popcll(tm & lt) < ties_left));
    const unsigned long long m = __ballot(take);
    const int at = pos + __popcll(m & lt);
    if (take && at < max_sel) out[at] = base + c;
    pos = min(pos + __popcll(m), max_sel);
    ties_left -= min(__popcll(tm), max(ties_left, 0));
  }
  for (int i = pos + lane; i < max_sel; i += 64) out[i] = -1;
  if (lane == 0) n_sel[item] = pos;
}

}  // namespace

hipError_t launch_select(const KGeom& g, const float* q_blk, const float* k_blk, const float* k_frm, int32_t kf,
                         int32_t kb, int32_t k_frames_stride, int32_t* sel_frames, int32_t* sel_blocks,
                         int32_t* n_sel, int32_t max_sel, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)g.B * g.H * g.nqb);
  const float* no_q = nullptr;
  if (g.D == 128)
    hipLaunchKernelGGL((select_kernel<128, false, float, kSelectWaves>), dim3(grid), dim3(64 * kSelectWaves), 0, stream, q_blk, no_q, k_blk, k_frm,
                       g, kf, kb, k_frames_stride, sel_frames, sel_blocks, n_sel, max_sel, nullptr);
  else
    hipLaunchKernelGGL((select_kernel<64, false, float, kSelectWaves>), dim3(grid), dim3(64 * kSelectWaves), 0, stream, q_blk, no_q, k_blk, k_frm,
                       g, kf, kb, k_frames_stride, sel_frames, sel_blocks, n_sel, max_sel, nullptr);
  return hipGetLastError();
}

namespace {
template <typename T, int D>
hipError_t launch_fused_typed(const KGeom& g, const void* q, const float* kp_blk, const float* kp_frm, int32_t kf,
                              int32_t kb, int32_t k_frames_stride, int32_t* sel_frames, int32_t* sel_blocks,
                              int32_t* n_sel, int32_t max_sel, float* q_blk, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)g.B * g.H * g.nqb);
  const float* no_qblk = nullptr;
  hipLaunchKernelGGL((select_kernel<D, true, T, kSelectWaves>), dim3(grid), dim3(64 * kSelectWaves), 0, stream, no_qblk, static_cast<const T*>(q),
                     kp_blk, kp_frm, g, kf, kb, k_frames_stride, sel_frames, sel_blocks, n_sel, max_sel, q_blk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_fused(const KGeom& g, int32_t dtype, const void* q, const float* kp_blk, const float* kp_frm,
                               int32_t kf, int32_t kb, int32_t k_frames_stride, int32_t* sel_frames,
                               int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, float* q_blk,
                               hipStream_t stream) {
  if (dtype == LF_BF16) {
    if (g.D == 128)
      return launch_fused_typed<__bf16, 128>(g, q, kp_blk, kp_frm, kf, kb, k_frames_stride, sel_frames, sel_blocks,
                                             n_sel, max_sel, q_blk, stream);
    return launch_fused_typed<__bf16, 64>(g, q, kp_blk, kp_frm, kf, kb, k_frames_stride, sel_frames, sel_blocks,
                                          n_sel, max_sel, q_blk, stream);
  }
  if (g.D == 128)
    return launch_fused_typed<float, 128>(g, q, kp_blk, kp_frm, kf, kb, k_frames_stride, sel_frames, sel_blocks,
                                          n_sel, max_sel, q_blk, stream);
  return launch_fused_typed<float, 64>(g, q, kp_blk, kp_frm, kf, kb, k_frames_stride, sel_frames, sel_blocks, n_sel,
                                       max_sel, q_blk, stream);
}

namespace {

// Selection-list check, one workgroup: wavefront w takes rows w, w + 16, ...
// A row (b*H + h)*nqb + qb is bad when n_sel is outside [0, max_sel], or one
// of its first n_sel ids is outside [0, Fh*nb), or an id is not greater than
// the one before it. The count of bad rows and the smallest bad row (or -1)
// are summed / taken in LDS and written by thread 0.
constexpr int kCheckWaves = 16;
__global__ __launch_bounds__(64 * kCheckWaves) void check_selection_kernel(const int32_t* __restrict__ sel,
                                                                            const int32_t* __restrict__ n_sel,
                                                                            int64_t rows, int max_sel, int n_ids,
                                                                            int32_t* __restrict__ result) {
  __shared__ int bad_count[kCheckWaves];
  __shared__ int64_t first_bad[kCheckWaves];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int count = 0;
  int64_t first = -1;
  for (int64_t r = wv; r < rows; r += kCheckWaves) {
    const int n = n_sel[r];
    bool bad = n < 0 || n > max_sel;
    if (!bad) {
      const int32_t* ids = sel + r * max_sel;
      for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        bool lane_bad = false;
        if (j < n) {
          const int x = ids[j];
          lane_bad = x < 0 || x >= n_ids || (j > 0 && ids[j - 1] >= x);
        }
        if (__builtin_amdgcn_ballot_w64(lane_bad) != 0) {
          bad = true;
          break;
        }
      }
    }
    if (bad) {
      ++count;
      if (first < 0) first = r;
    }
  }
  if (lane == 0) {
    bad_count[wv] = count;
    first_bad[wv] = first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int total = 0;
    int64_t lowest = -1;
    for (int w = 0; w < kCheckWaves; ++w) {
      total += bad_count[w];
      if (first_bad[w] >= 0 && (lowest < 0 || first_bad[w] < lowest)) lowest = first_bad[w];
    }
    result[0] = total;
    result[1] = (int32_t)lowest;
  }
}

}  // namespace

hipError_t launch_check_selection(const KGeom& g, const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel,
                                  int32_t* result, hipStream_t stream) {
  const int64_t rows = (int64_t)g.B * g.H * g.nqb;
  hipLaunchKernelGGL(check_selection_kernel, dim3(1), dim3(64 * kCheckWaves), 0, stream, sel_blocks, n_sel, rows,
                     max_sel, g.Fh * g.nb, result);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const KGeom& g, const float* q_blk, const float* k_blk, int32_t k,
                                int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)g.B * g.H * g.nqb);
  if (g.D == 128)
    hipLaunchKernelGGL((select_blocks_kernel<128>), dim3(grid), dim3(64), 0, stream, q_blk, k_blk, g, k, sel_blocks,
                       n_sel, max_sel);
  else
    hipLaunchKernelGGL((select_blocks_kernel<64>), dim3(grid), dim3(64), 0, stream, q_blk, k_blk, g, k, sel_blocks,
                       n_sel, max_sel);
  return hipGetLastError();
}

}  // namespace lf
