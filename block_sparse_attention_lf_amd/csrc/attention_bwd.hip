// Backward of the block-sparse attention (gradients of sum(out * dout)
// through the same block masks), for sparse fine-tuning: the ablation
// paragraph of the Light Forcing press summary (section 4) compares the
// sparse attention with and without fine-tuning the model around it. With
// S = scale q k^T over the keys a query
// block sees, P = softmax(S), O = P v:
//   dV = P^T dO,  dP = dO v^T,  D_i = dO_i . O_i,  dS = P * (dP - D),
//   dq = scale dS k,  dk = scale dS^T q.
// P is recomputed from the forward's log-sum-exp: P = exp2(scale*log2(e)*s
// - lse*log2(e)).
//
// gfx950 design (bf16 inputs, float32 gradients, MFMA 32x32x16 bf16 with
// float32 accumulation; P and dS are rounded to bf16 as MFMA operands):
//   * bwd_dq_kernel: one workgroup per query block (one wavefront per 32
//     rows), walking the keys the forward walks (the current chunk, then
//     the blocks of its selection) in 32-key tiles: S^T = K Q^T and
//     dP^T = V dO^T (Q^T, dO^T in registers), dS^T, then dQ^T += K^T dS^T
//     with K^T read from the row-major tile by the transposing LDS read. It
//     also writes D_i = dO_i . O_i for the key passes.
//   * bwd_dkv_kernel: one workgroup per key group (one wavefront per 32
//     keys; 256 keys of the current chunk, or one 64-key history tile),
//     walking the query blocks that see it (all of them for current-chunk
//     keys; those whose selection holds the block for a history tile) a
//     few query rows at a time. Per 32 query rows: S = Q K^T (K^T, V^T in
//     registers), P; dV^T += dO^T P; dP = dO V^T, dS, dK^T += Q^T dS.
//   Each key row's gradient is summed inside one workgroup: no atomics, and
//   every gradient row of a frame named by the slot table is written once
//   (zero where no query sees it). Rows of other slots are not written.
#include <mutex>

#include "mfma.h"

namespace lf {
namespace {

template <int D>
struct BwdShape {
  // LDS rows: at d = 128, 256 bytes with 16-byte chunks XOR-swizzled per row
  // (lds_swizzle); otherwise the bf16 row plus a 32-byte pad.
  static constexpr bool SWZ = D == 128;
  static constexpr int RS = SWZ ? 256 : D * 2 + 32;  // LDS row pitch (bytes)
  static constexpr int CPR = D * 2 / 16;  // 16-byte chunks per row
  static constexpr int QSTEPS = D / 16;   // MFMA reduction steps over d
  static constexpr int DB = D / 32;       // 32-column blocks of d
};

// Direct HBM -> LDS loads of a tile of ROWS rows (buffer loads that write
// LDS, 16 bytes per lane, no registers). Load instruction i of wavefront w
// fills 64 consecutive 16-byte LDS slots. Swizzled rows: slot s holds chunk
// (s mod 16) ^ lds_swizzle(row) of row s / 16. Padded rows: slot s holds
// chunk s mod SPR of row s / SPR, and the pad slots of a row re-read a chunk
// of the same row (same cache line). The buffer resource spans the tile's `count` valid rows,
// so rows past it come back as zeros and no load leaves the matrix.
template <int D, int ROWS, int NT>
struct TileDma {
  static constexpr int RS = BwdShape<D>::RS, CPR = BwdShape<D>::CPR, SPR = RS / 16;
  static constexpr int SLOTS = ROWS * SPR, NI = (SLOTS + NT - 1) / NT;
  static_assert(SLOTS % 64 == 0, "whole load instructions");
  uint32_t off[NI];
  __device__ inline void init(int tid) {
    const int wv = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = (i * (NT / 64) + wv) * 64 + lane;
      if constexpr (BwdShape<D>::SWZ) {  // slot (row, c') holds chunk c' ^ lds_swizzle(row)
        const int row = slot >> 4;
        off[i] = (uint32_t)(row * D * 2 + ((slot & 15) ^ lds_swizzle(row)) * 16);
      } else {
        const int row = min(slot / SPR, ROWS - 1);
        int c = slot - (slot / SPR) * SPR;
        while (c >= CPR) c -= CPR;
        off[i] = (uint32_t)(row * D * 2 + c * 16);
      }
    }
  }
  __device__ inline void issue(char* lds, const __bf16* src, int count, int tid) const {
#if defined(__HIP_DEVICE_COMPILE__)  // (the builtin exists only for the device pass)
    const int wv = tid >> 6;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(uniform_ptr(src)), (short)0, count * D * 2, kRawBufferFlags);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int L0 = (i * (NT / 64) + wv) * 64;
      if ((i + 1) * NT <= SLOTS || L0 < SLOTS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds + L0 * 16), 16, off[i], 0, 0, 0);
    }
#else
    (void)lds;
    (void)src;
    (void)count;
    (void)tid;
#endif
  }
};

// MFMA operand fragments (lane l, l32 = l % 32, h = l / 32):
// rows r0 + l32 of an LDS tile, d = 16t + 8h .. +7 (A operand, rows = M;
// r0 a multiple of 32).
template <int D>
__device__ inline bf16x8 row_frag(const char* tile, int r0, int t, int l32, int h) {
  if constexpr (BwdShape<D>::SWZ) {
    // chunk 2t+h of row r sits at (2t+h) ^ sw(r); with sw = 2*xh + x0 that is
    // byte 32*(t ^ xh) + 16*(h ^ x0): a per-lane base XOR 32t
    const int x = lds_swizzle(l32);
    const uint32_t base = (uint32_t)(l32 * 256 + 32 * (x >> 1) + 16 * (h ^ (x & 1)));
    return *reinterpret_cast<const bf16x8*>(tile + r0 * 256 + (base ^ (uint32_t)(32 * t)));
  } else {
    return *reinterpret_cast<const bf16x8*>(tile + (r0 + l32) * BwdShape<D>::RS + (16 * t + 8 * h) * 2);
  }
}
// The transposed fragment of 16 rows (step ps) and 32 columns (block db):
// A[d][row] with the rows in the order a 32x32 accumulator holds them, so
// the bf16 copy of an accumulator is the matching B operand.
template <int D>
__device__ inline bf16x8 tr_frag(const char* tile, int ps, int db, int lane) {
  constexpr int RS = BwdShape<D>::RS;
  const int s16 = lane & 15, h = lane >> 5;
  i16x4 part[2];
  if constexpr (BwdShape<D>::SWZ) {
    // row 4h + s16/4 + 16ps + 8j (sw = 4*(s16/4) + h + 2j), chunk 4db + cb
    // with cb = 2*((lane/16)&1) + (s16&3)/2, half s16&1: the chunk bits are
    // (4*(s16/4) + (cb ^ h)) ^ (4db + 2j), a per-lane base XOR a constant.
    const int cb = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
    const uint32_t base = (uint32_t)((4 * h + (s16 >> 2)) * 256 + 16 * (4 * (s16 >> 2) + (cb ^ h)) + 8 * (s16 & 1));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      part[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          LDS_PTR(i16x4, tile + (16 * ps + 8 * j) * 256 + (base ^ (uint32_t)(16 * (4 * db + 2 * j)))));
  } else {
    const char* base = tile + (4 * h + (s16 >> 2)) * RS + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      part[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, base + (16 * ps + 8 * j) * RS + 64 * db));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}
// This lane's own row of a global matrix, d = 16t + 8h .. +7 (B operand,
// column = the lane's row), zeros when the row does not exist.
__device__ inline bf16x8 own_frag(const __bf16* row, bool ok, int t, int h) {
  const uint4 v = ok ? *reinterpret_cast<const uint4*>(row + 16 * t + 8 * h) : make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(bf16x8, v);
}

// Writes a transposed 32x32 accumulator block (rows = d in [32db, 32db+32),
// column = this lane's row) times `mul` as float32 into row `dst`.
__device__ inline void store_acc_t(float* dst, const f32x16& acc, int db, int h, float mul) {
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4) {
    const int col = db * 32 + 8 * a4 + 4 * h;
    *reinterpret_cast<float4*>(dst + col) = make_float4(acc[4 * a4] * mul, acc[4 * a4 + 1] * mul,
                                                       acc[4 * a4 + 2] * mul, acc[4 * a4 + 3] * mul);
  }
}

// Position in a query block's walk: the current chunk's KT-key tiles
// (frame cf, tile ct of it), then the tiles of its selected history blocks
// (list entry e, tile half of the block; a block is hpb = ceil(b / KT)
// tiles). Counters rather than divisions: the walk advances one tile at a
// time.
struct DqWalk {
  int t = 0, cf = 0, ct = 0, e = 0, half = 0;
};

// The walk's next tile from position w.t on (ignored ids skipped): its
// address and valid key count; false when the walk is over. On return w.t
// is the tile found and the counters point past it.
template <int KT>
__device__ inline bool dq_tile(const KGeom& g, const int32_t* sel, int64_t item, int max_sel, int tpf, int n_cur,
                               int hpb, int64_t bh, DqWalk& w, int n_tiles, int64_t& base, int& count) {
  for (; w.t < n_tiles; ++w.t) {
    int slot, start;
    if (w.t < n_cur) {
      slot = g.slot[g.Fh + w.cf];
      start = w.ct * KT;
      count = min(KT, g.T - start);
      if (++w.ct == tpf) {
        w.ct = 0;
        ++w.cf;
      }
    } else {
      const int x = sel[item * max_sel + w.e];
      const int half = w.half;
      if (++w.half == hpb) {
        w.half = 0;
        ++w.e;
      }
      if (x < 0 || x >= g.Fh * g.nb) continue;  // ignored id
      const int f = x / g.nb, jb = x - f * g.nb;
      slot = g.slot[f];
      start = jb * g.b + half * KT;
      count = min(KT, min(jb * g.b + g.b, g.T) - start);
      if (count <= 0) continue;
    }
    base = ((bh * g.S + slot) * (int64_t)g.T + start) * g.D;
    return true;
  }
  return false;
}

// One tile of the dQ walk on the stage (ks, vs): KT keys, `count` valid.
template <int D, int KT>
__device__ inline void dq_tile_math(const char* ks, const char* vs, int count, const bf16x8* qf, const bf16x8* dof,
                                    f32x16* acc, float c2, float lse2, float dd, int lane) {
  using S = BwdShape<D>;
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kh = 0; kh < KT / 32; ++kh) {
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.0f;
      dp[r] = 0.0f;
    }
#pragma unroll
    for (int st = 0; st < S::QSTEPS; ++st) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(ks, 32 * kh, st, l32, h), qf[st], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(vs, 32 * kh, st, l32, h), dof[st], dp, 0, 0, 0);
    }
    bf16x8 b0, b1;
    if (count >= 32 * (kh + 1)) {  // every key of the half exists (wave-uniform): no mask
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -lse2));
        const __bf16 d = (__bf16)(p * (dp[r] - dd));
        if (r < 8) b0[r] = d; else b1[r - 8] = d;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool kv = 32 * kh + acc_row(r, h) < count;
        const float p = kv ? __builtin_amdgcn_exp2f(fmaf(s[r], c2, -lse2)) : 0.0f;
        const __bf16 d = (__bf16)(p * (dp[r] - dd));
        if (r < 8) b0[r] = d; else b1[r - 8] = d;
      }
    }
#pragma unroll
    for (int db = 0; db < S::DB; ++db) {
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(ks, 2 * kh, db, lane), b0, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(ks, 2 * kh + 1, db, lane), b1, acc[db], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ (and D_i): one workgroup of WPQ wavefronts per (batch, head, query
// block), walking key tiles of KT keys. With KT = 32 the four stage buffers
// take 37 KB of LDS (D = 128), so workgroups share a CU two wavefronts per
// SIMD (registers capped at 256 to match).
template <int D, int WPQ, int KT>
__global__ __launch_bounds__(64 * WPQ, (KT == 32 && WPQ >= 2 ? 2 : 1)) void bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ kc,
                                                          const __bf16* __restrict__ vc, const __bf16* __restrict__ out,
                                                          const __bf16* __restrict__ dout, const float* __restrict__ lse,
                                                          const int32_t* __restrict__ sel,
                                                          const int32_t* __restrict__ nsel, int max_sel, float scale,
                                                          const KGeom g, float* __restrict__ delta,
                                                          float* __restrict__ dq) {
  using S = BwdShape<D>;
  constexpr int NT = 64 * WPQ;
  // Double-buffered K/V stages, separate arrays so the compiler sees that the
  // fragment reads of one stage never wait on the loads filling the other.
  __shared__ __attribute__((aligned(1024))) char ks0[KT * S::RS];
  __shared__ __attribute__((aligned(1024))) char vs0[KT * S::RS];
  __shared__ __attribute__((aligned(1024))) char ks1[KT * S::RS];
  __shared__ __attribute__((aligned(1024))) char vs1[KT * S::RS];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t item = xcd_item(blockIdx.x, gridDim.x);  // (b*H + h)*nqb + qb
  const int64_t bh = item / g.nqb;
  const int qb = (int)(item - bh * g.nqb);
  const int fc = qb / g.nb, jq = qb - fc * g.nb;
  const int nrows = min(g.b, g.T - jq * g.b);
  const int64_t row0 = bh * g.Lq + (int64_t)fc * g.T + (int64_t)jq * g.b;
  const int qr = 32 * wv + l32;
  const bool ok = qr < nrows;
  const float c2 = scale * kLog2e;

  bf16x8 qf[S::QSTEPS], dof[S::QSTEPS];
  float dd = 0.0f;
  {
    const __bf16* qp = q + (row0 + (ok ? qr : 0)) * D;
    const __bf16* gp = dout + (row0 + (ok ? qr : 0)) * D;
    const __bf16* op = out + (row0 + (ok ? qr : 0)) * D;
#pragma unroll
    for (int t = 0; t < S::QSTEPS; ++t) {
      qf[t] = own_frag(qp, ok, t, h);
      dof[t] = own_frag(gp, ok, t, h);
      const bf16x8 of = own_frag(op, ok, t, h);
#pragma unroll
      for (int e = 0; e < 8; ++e) dd = fmaf((float)dof[t][e], (float)of[e], dd);
    }
  }
  dd += __shfl_xor(dd, 32);  // the other half of the row's d
  if (ok && h == 0) delta[row0 + qr] = dd;
  const float lse2 = ok ? lse[row0 + qr] * kLog2e : 0.0f;

  f32x16 acc[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  const int tpf = (g.T + KT - 1) / KT;
  const int n_cur = g.Fc * tpf;
  const int hpb = (g.b + KT - 1) / KT;
  const int len = max_sel > 0 ? min(max(nsel[item], 0), max_sel) : 0;
  const int n_tiles = n_cur + len * hpb;
  TileDma<D, KT, NT> dma;
  dma.init(tid);
  DqWalk walk;
  int count = 0, ncount = 0;
  int64_t nbase = 0;
  bool have = dq_tile<KT>(g, sel, item, max_sel, tpf, n_cur, hpb, bh, walk, n_tiles, nbase, ncount);
  if (have) {
    dma.issue(ks0, kc + nbase, ncount, tid);
    dma.issue(vs0, vc + nbase, ncount, tid);
  }
  // Per tile: wait for its loads, barrier (everyone's landed; everyone is done
  // with the other stage), start the next tile's loads into the other stage,
  // compute. Unrolled by two so each half names its stage buffers.
#define LF_DQ_STEP(KA, VA, KB, VB)                                                         \
  {                                                                                      \
    count = ncount;                                                                      \
    ++walk.t;                                                                            \
    const bool more = dq_tile<KT>(g, sel, item, max_sel, tpf, n_cur, hpb, bh, walk, n_tiles, nbase, ncount); \
    __builtin_amdgcn_s_waitcnt(kWaitVm0);                                                \
    __syncthreads();                                                                     \
    if (more) {                                                                          \
      dma.issue(KB, kc + nbase, ncount, tid);                                            \
      dma.issue(VB, vc + nbase, ncount, tid);                                            \
    }                                                                                    \
    dq_tile_math<D, KT>(KA, VA, count, qf, dof, acc, c2, lse2, dd, lane);                \
    have = more;                                                                         \
  }
  while (have) {
    LF_DQ_STEP(ks0, vs0, ks1, vs1)
    if (!have) break;
    LF_DQ_STEP(ks1, vs1, ks0, vs0)
  }
#undef LF_DQ_STEP
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no load may still be writing LDS when the workgroup ends
  if (!ok) return;
  float* dst = dq + (row0 + qr) * D;
#pragma unroll
  for (int db = 0; db < S::DB; ++db) store_acc_t(dst, acc[db], db, h, scale);
}

// Element i of rows [row0, row0 + n) of a float array (0 past n), read
// through a buffer resource: the base stays in scalar registers and the lane
// holds a 32-bit offset, not a 64-bit address.
__device__ inline float row_value(const float* base, int64_t row0, int n, int i) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(uniform_ptr(base + row0)), (short)0, n * 4, kRawBufferFlags);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
#else
  (void)base;
  (void)row0;
  (void)n;
  (void)i;
  return 0.0f;
#endif
}

// Element e of a packed bf16x8 as a float, from the 32-bit word holding it.
__device__ inline float bf16_word_elt(const bf16x8& v, int e) {
  const uint4 w = __builtin_bit_cast(uint4, v);
  const uint32_t x = (e >> 1) == 0 ? w.x : (e >> 1) == 1 ? w.y : (e >> 1) == 2 ? w.z : w.w;
  return __builtin_bit_cast(float, (e & 1) ? (x & 0xffff0000u) : (x << 16));
}

// One query block against this wavefront's 32 keys (K^T, V^T in registers):
// per 32 query rows, S = Q K^T and P; dV^T += dO^T P, or dP = dO V^T,
// dS = P (dP - D) and dK^T += Q^T dS. The row terms enter as the starting
// values of the accumulators, so no per-row value stays live across the
// MFMA chains: ls holds -lse/scale per row (-inf on missing rows, so their P
// is 0), and the score accumulator starts there, giving
// P = 2^(scale*log2(e) * (s - lse/scale)); nd holds -D per row, and the dP
// accumulator starts there, giving dP - D. IL: the S and dP chains (and the
// dV and dK ones) interleaved, which needs sixteen more registers; the
// history pass, which holds more state, runs them one after the other.
//
// issue_next() starts the next step's tile loads into the other stage. The
// interleaved form calls it first; the other after the first score chain,
// so that the K fragments that chain reads, if the compiler has spilled
// them, are reloaded before the tile loads are in flight (a reload issued
// after them would wait for them too).
template <int D, bool IL, typename Issue>  // adv: dV^T accumulators, adk: dK^T accumulators
__device__ inline void dkv_block_math(const char* qs, const char* gs, const float* ls, const float* nd, int nrows,
                                      const bf16x8* kf, const bf16x8* vf, f32x16* adv, f32x16* adk, float c2,
                                      bool kok, int lane, const Issue& issue_next) {
  using S = BwdShape<D>;
  // The lane index is made opaque here, so the fragment addresses derived
  // from it (one XOR per swizzled read) are recomputed at each step instead
  // of being hoisted out of the walk and held in registers across it.
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, h = lane >> 5;
  const int halves = (nrows + 31) / 32;
  if constexpr (IL) {
    issue_next();
    for (int qh = 0; qh < halves; ++qh) {
      // S - lse/scale and dP - D as two interleaved MFMA chains (each one's
      // fragment reads overlap the other's products).
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = ls[32 * qh + acc_row(r, h)];
        dp[r] = nd[32 * qh + acc_row(r, h)];
      }
#pragma unroll
      for (int st = 0; st < S::QSTEPS; ++st) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(qs, 32 * qh, st, l32, h), kf[st], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(gs, 32 * qh, st, l32, h), vf[st], dp, 0, 0, 0);
      }
      // P and dS = P (dP - D), rounded to bf16 (dS from the rounded P, the
      // values the dV product uses).
      bf16x8 p0, p1, b0, b1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const __bf16 pr = (__bf16)(kok ? __builtin_amdgcn_exp2f(s[r] * c2) : 0.0f);
        const __bf16 d = (__bf16)((float)pr * dp[r]);
        if (r < 8) {
          p0[r] = pr;
          b0[r] = d;
        } else {
          p1[r - 8] = pr;
          b1[r - 8] = d;
        }
      }
#pragma unroll
      for (int db = 0; db < S::DB; ++db) {  // dV^T += dO^T P, dK^T += Q^T dS
        adv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(gs, 2 * qh, db, lane), p0, adv[db], 0, 0, 0);
        adk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qs, 2 * qh, db, lane), b0, adk[db], 0, 0, 0);
        adv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(gs, 2 * qh + 1, db, lane), p1, adv[db], 0, 0, 0);
        adk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qs, 2 * qh + 1, db, lane), b1, adk[db], 0, 0, 0);
      }
    }
  } else {
    if (halves == 0) issue_next();
    for (int qh = 0; qh < halves; ++qh) {
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = ls[32 * qh + acc_row(r, h)];
#pragma unroll
      for (int st = 0; st < S::QSTEPS; ++st)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(qs, 32 * qh, st, l32, h), kf[st], s, 0, 0, 0);
      if (qh == 0) issue_next();
      // P, rounded to bf16 once: the dV product and dS both use these values.
      // They stay packed (eight registers) across the dP product: the empty asm
      // makes the packed words opaque, so the compiler cannot keep the sixteen
      // unpacked values alive instead, and dS unpacks them from the words.
      bf16x8 p0, p1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const __bf16 pr = (__bf16)(kok ? __builtin_amdgcn_exp2f(s[r] * c2) : 0.0f);
        if (r < 8) p0[r] = pr; else p1[r - 8] = pr;
      }
      asm volatile("" : "+v"(p0), "+v"(p1));
#pragma unroll
      for (int db = 0; db < S::DB; ++db) {  // dV^T += dO^T P
        adv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(gs, 2 * qh, db, lane), p0, adv[db], 0, 0, 0);
        adv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(gs, 2 * qh + 1, db, lane), p1, adv[db], 0, 0, 0);
      }
      {  // dP - D = dO V^T - D, dS = P (dP - D), dK^T += Q^T dS
        f32x16 dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = nd[32 * qh + acc_row(r, h)];
#pragma unroll
        for (int st = 0; st < S::QSTEPS; ++st)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(gs, 32 * qh, st, l32, h), vf[st], dp, 0, 0, 0);
        bf16x8 b0, b1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = r < 8 ? bf16_word_elt(p0, r) : bf16_word_elt(p1, r - 8);
          const __bf16 d = (__bf16)(pr * dp[r]);
          if (r < 8) b0[r] = d; else b1[r - 8] = d;
        }
#pragma unroll
        for (int db = 0; db < S::DB; ++db) {
          adk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qs, 2 * qh, db, lane), b0, adk[db], 0, 0, 0);
          adk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qs, 2 * qh + 1, db, lane), b1, adk[db], 0, 0, 0);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dV and dK of the keys of one workgroup, NW wavefronts of 32 keys each, walking the query blocks that see them
// MAXQ rows at a time. CUR: key groups of the current chunk (Fc *
// ceil(T / (32 NW)) per (batch, head)); otherwise one 64-key tile of a
// history block (blocks of more than 64 keys are two).
template <int D, int MAXQ, int NW, bool CUR>
__global__ __launch_bounds__(64 * NW, (NW >= 8 || MAXQ <= 32 ? 2 : 1)) void bwd_dkv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ kc,
                                                      const __bf16* __restrict__ vc, const __bf16* __restrict__ dout,
                                                      const float* __restrict__ lse, const float* __restrict__ delta,
                                                      const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ nsel, int max_sel, float scale,
                                                      const KGeom g, const int* __restrict__ order,
                                                      float* __restrict__ dv, float* __restrict__ dk) {
  using S = BwdShape<D>;
  constexpr int NT = 64 * NW;
  constexpr int KEYS = 32 * NW;  // keys per workgroup
  constexpr int QCAP = MAXQ <= 32 ? 512 : 1024;  // query blocks listed per batch
  __shared__ __attribute__((aligned(1024))) char qs0[MAXQ * S::RS];
  __shared__ __attribute__((aligned(1024))) char gs0[MAXQ * S::RS];
  __shared__ __attribute__((aligned(1024))) char qs1[MAXQ * S::RS];
  __shared__ __attribute__((aligned(1024))) char gs1[MAXQ * S::RS];
  __shared__ float ls0[MAXQ], ls1[MAXQ], ds0[MAXQ], ds1[MAXQ];
  __shared__ int qlist[QCAP];
  __shared__ uint32_t qmask[QCAP / 32];
  __shared__ int qcount;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hpb = g.b > 64 ? 2 : 1;
  const int gpf = (g.T + KEYS - 1) / KEYS;  // key groups per current frame
  const int per_bh = CUR ? g.Fc * gpf : g.Fh * g.nb * hpb;
  const int wgx = xcd_item(blockIdx.x, gridDim.x);
  const int wgi = !CUR && order != nullptr ? order[wgx] : wgx;  // history: longest first (hist_order_kernel)
  const int64_t bh = wgi / per_bh;
  const int ti = (int)(wgi - bh * per_bh);
  int f, start, count, hist_id = -1;
  if constexpr (CUR) {
    const int f2 = ti / gpf;
    f = g.Fh + f2;
    start = (ti - f2 * gpf) * KEYS;
    count = min(KEYS, g.T - start);
  } else {
    static_assert(KEYS == 64, "a history workgroup holds one 64-key tile");
    const int hi = ti;
    f = hi / (g.nb * hpb);
    const int rem = hi - f * g.nb * hpb;
    const int jb = rem / hpb, half = rem - jb * hpb;
    start = jb * g.b + half * 64;
    count = min(64, min(jb * g.b + g.b, g.T) - start);
    hist_id = f * g.nb + jb;
  }
  if (count <= 0) return;  // second half of a short last block: no keys (uniform over the workgroup)
  const int64_t krow0 = (bh * g.S + g.slot[f]) * (int64_t)g.T + start;
  const int key = 32 * wv + l32;
  const bool kok = key < count;
  const float c2 = scale * kLog2e, inv_scale = 1.0f / scale;

  bf16x8 kf[S::QSTEPS], vf[S::QSTEPS];
#pragma unroll
  for (int t = 0; t < S::QSTEPS; ++t) {
    kf[t] = own_frag(kc + (krow0 + (kok ? key : 0)) * D, kok, t, h);
    vf[t] = own_frag(vc + (krow0 + (kok ? key : 0)) * D, kok, t, h);
  }
  f32x16 adv[S::DB], adk[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      adv[db][r] = 0.0f;
      adk[db][r] = 0.0f;
    }
  TileDma<D, MAXQ, NT> dma;
  dma.init(tid);

  for (int c0 = 0; c0 < g.nqb; c0 += QCAP) {
    // The query blocks in [c0, c0 + QCAP) that see this tile, ascending.
    const int nqc = min(QCAP, g.nqb - c0);
    __syncthreads();  // the previous batch's list is consumed
    if (hist_id >= 0) {
      // A history tile is seen by the query blocks whose lists name its
      // block. The batch's rows of sel are one contiguous array: every
      // thread scans a strided share of it with U loads in flight at a time
      // and marks a query block's bit in qmask where its block id appears
      // at a position below the block's list length (staged in qlist).
      for (int i = tid; i < QCAP / 32; i += NT) qmask[i] = 0u;
      for (int i = tid; i < nqc; i += NT) qlist[i] = max_sel > 0 ? min(max(nsel[bh * g.nqb + c0 + i], 0), max_sel) : 0;
      __syncthreads();
      const int32_t* rows = sel + (bh * g.nqb + c0) * (int64_t)max_sel;
      const int n_ent = nqc * max_sel;
      constexpr int U = 8;
      for (int e0 = tid; e0 < n_ent; e0 += NT * U) {
        int x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = e0 + u * NT < n_ent ? rows[e0 + u * NT] : -1;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (x[u] == hist_id) {
            const int e = e0 + u * NT, qi = e / max_sel;
            if (e - qi * max_sel < qlist[qi]) atomicOr(&qmask[qi >> 5], 1u << (qi & 31));
          }
      }
      __syncthreads();
    }
    if (wv == 0) {
      int n = 0;
      for (int k0 = 0; k0 < nqc; k0 += 64) {
        const int qi = k0 + lane;
        const bool sees = qi < nqc && (hist_id < 0 || ((qmask[qi >> 5] >> (qi & 31)) & 1u) != 0);
        const uint64_t m = __builtin_amdgcn_ballot_w64(sees);
        if (sees) qlist[n + __builtin_popcountll(m & ((1ull << lane) - 1ull))] = c0 + qi;
        n += __builtin_popcountll(m);
      }
      if (lane == 0) qcount = n;
    }
    __syncthreads();
    const int nq = qcount;
    if (nq == 0) continue;
    // Steps of at most MAXQ query rows: a query block of more rows is taken
    // in several steps. Stage the first step; then per step: wait, barrier,
    // start the next step's lse / delta row loads (into registers) and its
    // tile loads into the other stage, compute, and write those rows to LDS.
    // The row loads go out after the barrier, ahead of the tiles, so the
    // computation covers their latency and the wait before the write leaves
    // the tile loads in flight.
    // Rows [r0, r0 + rows) of step (ii, hh): part hh of query block qlist[ii],
    // which has qrows rows in all.
    auto locate = [&](int ii, int hh, int64_t& r0, int& rows, int& qrows) {
      const int qb = qlist[ii];
      const int fc = qb / g.nb, jq = qb - fc * g.nb;
      qrows = min(g.b, g.T - jq * g.b);
      r0 = bh * g.Lq + (int64_t)fc * g.T + (int64_t)jq * g.b + (int64_t)hh * MAXQ;
      rows = min(MAXQ, qrows - hh * MAXQ);
    };
    int i = 0, hq = 0, nrows = 0, qrows = 0;
    int64_t row0 = 0;
    locate(0, 0, row0, nrows, qrows);
    if (tid < MAXQ) {
      ls0[tid] = tid < nrows ? -row_value(lse, row0, nrows, tid) * inv_scale : -INFINITY;  // -inf: P = 0 on missing rows
      ds0[tid] = -row_value(delta, row0, nrows, tid);
    }
    dma.issue(qs0, q + row0 * D, nrows, tid);
    dma.issue(gs0, dout + row0 * D, nrows, tid);
    bool have = true;
#define LF_DKV_STEP(QA, GA, LA, DA, QB, GB, LB, DB_)                                          \
  {                                                                                         \
    const int cur_rows = nrows;                                                             \
    bool more = true;                                                                       \
    if ((hq + 1) * MAXQ < qrows) {                                                          \
      ++hq;                                                                                 \
    } else if (i + 1 < nq) {                                                                \
      ++i;                                                                                  \
      hq = 0;                                                                               \
    } else {                                                                                \
      more = false;                                                                         \
    }                                                                                       \
    if (more) locate(i, hq, row0, nrows, qrows);                                            \
    __builtin_amdgcn_s_waitcnt(kWaitVm0);                                                   \
    __syncthreads();                                                                        \
    float nl = 0.0f, nd = 0.0f;                                                             \
    if (more) {                                                                             \
      if (tid < MAXQ) {                                                                     \
        nl = row_value(lse, row0, nrows, tid);                                              \
        nd = row_value(delta, row0, nrows, tid);                                            \
      }                                                                                     \
    }                                                                                       \
    const auto issue_next = [&]() {                                                         \
      if (more) {                                                                           \
        dma.issue(QB, q + row0 * D, nrows, tid);                                            \
        dma.issue(GB, dout + row0 * D, nrows, tid);                                         \
      }                                                                                     \
    };                                                                                      \
    dkv_block_math<D, CUR>(QA, GA, LA, DA, cur_rows, kf, vf, adv, adk, c2, kok, lane, issue_next); \
    if (more && tid < MAXQ) {                                                               \
      LB[tid] = tid < nrows ? -nl * inv_scale : -INFINITY;                                  \
      DB_[tid] = -nd;                                                                       \
    }                                                                                       \
    have = more;                                                                            \
  }
    while (have) {
      LF_DKV_STEP(qs0, gs0, ls0, ds0, qs1, gs1, ls1, ds1)
      if (!have) break;
      LF_DKV_STEP(qs1, gs1, ls1, ds1, qs0, gs0, ls0, ds0)
    }
#undef LF_DKV_STEP
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no load may still be writing LDS when the workgroup ends
  if (!kok) return;
  float* vrow = dv + (krow0 + key) * D;
  float* krow = dk + (krow0 + key) * D;
#pragma unroll
  for (int db = 0; db < S::DB; ++db) {
    store_acc_t(vrow, adv[db], db, h, 1.0f);
    store_acc_t(krow, adk[db], db, h, scale);
  }
}

// Launch order of the history dK/dV pass, longest first. A history tile's
// workgroup walks the query blocks whose selections name its block, so its
// time grows with their number (1 to 28 at the 480p workload). Workgroups
// are dealt round-robin to the 8 XCDs and each XCD works through one
// contiguous range of items (xcd_item); this kernel permutes each range so
// that its items come in descending order of that number, and the pass
// takes item order[xcd_item(wg)]. The longest workgroups then start first
// and the pass does not end on a few long ones started late (list
// scheduling, longest first). It decides only when each workgroup runs,
// not what any of them computes. One workgroup per range: count in LDS,
// then a counting sort by count.
constexpr int kOrderMaxItems = 12288;  // items per range (LDS); larger passes keep the plain order
constexpr int kOrderBuckets = 1024;    // counts are clamped to kOrderBuckets - 1

__global__ __launch_bounds__(1024) void hist_order_kernel(const int32_t* __restrict__ sel,
                                                          const int32_t* __restrict__ nsel, int max_sel, const KGeom g,
                                                          int nitems, int* __restrict__ order) {
  __shared__ int cnt[kOrderMaxItems];
  __shared__ int base[kOrderBuckets];
  const int x = blockIdx.x, tid = threadIdx.x;
  const int per = nitems >> 3, rem = nitems & 7;
  const int lo = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  const int n = per + (x < rem ? 1 : 0);
  if (n <= 0) return;
  for (int i = tid; i < n; i += 1024) cnt[i] = 0;
  for (int i = tid; i < kOrderBuckets; i += 1024) base[i] = 0;
  __syncthreads();
  const int hpb = g.b > 64 ? 2 : 1, nblk = g.Fh * g.nb, per_bh = nblk * hpb;
  const int n_ent = g.nqb * max_sel;
  for (int bh = lo / per_bh; bh <= (lo + n - 1) / per_bh; ++bh) {
    const int32_t* rows = sel + (int64_t)bh * n_ent;
    for (int e = tid; e < n_ent; e += 1024) {
      const int qi = e / max_sel;
      const int len = min(max(nsel[(int64_t)bh * g.nqb + qi], 0), max_sel);
      const int id = rows[e];
      if (e - qi * max_sel < len && id >= 0 && id < nblk)
        for (int hf = 0; hf < hpb; ++hf) {
          const int it = bh * per_bh + id * hpb + hf - lo;
          if (it >= 0 && it < n) atomicAdd(&cnt[it], 1);
        }
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) atomicAdd(&base[min(cnt[i], kOrderBuckets - 1)], 1);
  __syncthreads();
  if (tid < 64) {
    // bucket starts in descending count order: lane l takes the 16 buckets
    // below kOrderBuckets - 16 l, then an exclusive scan over the lanes
    const int top = kOrderBuckets - 16 * tid;
    int sum = 0;
    for (int c = top - 1; c >= top - 16; --c) sum += base[c];
    int incl = sum;
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (tid >= off) incl += t;
    }
    int run = incl - sum;
    for (int c = top - 1; c >= top - 16; --c) {
      const int t = base[c];
      base[c] = run;
      run += t;
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) order[lo + atomicAdd(&base[min(cnt[i], kOrderBuckets - 1)], 1)] = lo + i;
}

// Key tile width of the dQ walk (32: two wavefronts per SIMD; 64: one, with
// half the tiles).
constexpr int kDqKeys = 32;

template <int D>
hipError_t launch_bwd_d(const KGeom& g, const void* q, const void* k, const void* v, const int32_t* sel,
                        const int32_t* nsel, int max_sel, float scale, const void* out, const float* lse,
                        const void* dout, float* delta, float* dq, float* dk, float* dv, hipStream_t stream) {
  const __bf16* Q = static_cast<const __bf16*>(q);
  const __bf16* K = static_cast<const __bf16*>(k);
  const __bf16* V = static_cast<const __bf16*>(v);
  const __bf16* O = static_cast<const __bf16*>(out);
  const __bf16* G = static_cast<const __bf16*>(dout);
  const unsigned nq = (unsigned)((int64_t)g.B * g.H * g.nqb);
  switch ((g.b + 31) / 32) {
    case 1:
      hipLaunchKernelGGL((bwd_dq_kernel<D, 1, kDqKeys>), dim3(nq), dim3(64), 0, stream, Q, K, V, O, G, lse, sel, nsel, max_sel,
                         scale, g, delta, dq);
      break;
    case 2:
      hipLaunchKernelGGL((bwd_dq_kernel<D, 2, kDqKeys>), dim3(nq), dim3(128), 0, stream, Q, K, V, O, G, lse, sel, nsel,
                         max_sel, scale, g, delta, dq);
      break;
    case 3:
      hipLaunchKernelGGL((bwd_dq_kernel<D, 3, kDqKeys>), dim3(nq), dim3(192), 0, stream, Q, K, V, O, G, lse, sel, nsel,
                         max_sel, scale, g, delta, dq);
      break;
    default:
      hipLaunchKernelGGL((bwd_dq_kernel<D, 4, kDqKeys>), dim3(nq), dim3(256), 0, stream, Q, K, V, O, G, lse, sel, nsel,
                         max_sel, scale, g, delta, dq);
      break;
  }
  // Current-chunk keys are seen by every query block of the head: 256 keys
  // per workgroup (eight wavefronts) so each staged query block feeds eight
  // wavefronts' MFMA work. History blocks have their own query blocks: one
  // 64-key tile per workgroup. Both take dK and dV in one pass (S and P are
  // formed once for both), with two wavefronts per SIMD (256 registers).
  // The eight-wavefront current workgroups fill a CU on their own and
  // stage up to 64 query rows per step (78 KB of LDS); the two-wavefront
  // history workgroups stage 32 rows per step (35 KB), so four share a CU.
  // The history pass runs first, in the order hist_order_kernel writes into
  // the dk rows of the first chunk frame of (batch 0, head 0): T * D floats
  // that the current-chunk pass overwrites with their gradients afterwards,
  // so the call needs no scratch for it.
  const unsigned ncur = (unsigned)((int64_t)g.B * g.H * g.Fc * ((g.T + 255) / 256));
  const unsigned nhist = (unsigned)((int64_t)g.B * g.H * g.Fh * g.nb * (g.b > 64 ? 2 : 1));
  if (nhist > 0) {
    int* order = nullptr;
    if (max_sel > 0 && (nhist + 7) / 8 <= (unsigned)kOrderMaxItems && (int64_t)nhist <= (int64_t)g.T * D) {
      order = reinterpret_cast<int*>(dk + (int64_t)g.slot[g.Fh] * g.T * D);
      hipLaunchKernelGGL(hist_order_kernel, dim3(8), dim3(1024), 0, stream, sel, nsel, max_sel, g, (int)nhist, order);
    }
    hipLaunchKernelGGL((bwd_dkv_kernel<D, 32, 2, false>), dim3(nhist), dim3(128), 0, stream, Q, K, V, G, lse, delta,
                       sel, nsel, max_sel, scale, g, order, dv, dk);
  }
  hipLaunchKernelGGL((bwd_dkv_kernel<D, 64, 8, true>), dim3(ncur), dim3(512), 0, stream, Q, K, V, G, lse, delta, sel,
                     nsel, max_sel, scale, g, nullptr, dv, dk);
  return hipGetLastError();
}

}  // namespace

// Row scratch (delta) of lf_block_sparse_attn_bwd_noalloc: a fixed array in
// each GPU's copy of the library, LF_NOALLOC_MAX_ROWS floats. Host code never
// uses its name as an address (on the host the name is a stand-in, not the
// device address): the address comes from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) float scratch[LF_NOALLOC_MAX_ROWS];

hipError_t noalloc_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static float* addr[kMaxDevices];
  static hipError_t status[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev]() {
    void* p = nullptr;
    status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = static_cast<float*>(p);
  });
  if (status[dev] != hipSuccess) return status[dev];
  if (addr[dev] == nullptr) return hipErrorInvalidSymbol;
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attention_bwd(const KGeom& g, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel, float scale,
                                const void* out, const float* lse, const void* dout, float* delta, float* dq,
                                float* dk_cache, float* dv_cache, hipStream_t stream) {
  if (g.D == 128)
    return launch_bwd_d<128>(g, q, k_cache, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, dout, delta, dq,
                             dk_cache, dv_cache, stream);
  return launch_bwd_d<64>(g, q, k_cache, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, dout, delta, dq,
                          dk_cache, dv_cache, stream);
}

}  // namespace lf
