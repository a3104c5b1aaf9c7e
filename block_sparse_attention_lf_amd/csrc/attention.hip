// Block-sparse attention over a rolling/anchored KV cache (Light Forcing,
// technical summary 2.2 "execution"; press summary section 3): every query
// of a query block attends to its selected history blocks and to the whole
// current chunk, softmax(scale q k^T) v, with an fp32 online softmax.
//
// gfx950 design
//   * One workgroup per (batch, head, query block); NW = ceil(block/32)
//     wavefronts, each owning 32 query rows. Work is assigned XCD-aware: the
//     hardware deals workgroups round-robin over the 8 XCDs, so workgroup w
//     is remapped to work item p such that each XCD gets one contiguous range
//     of (batch, head, query block) items. Query blocks of one head then run
//     on one XCD and share the head's keys/values in that XCD's L2.
//   * The key walk is a list of BN-key tiles: the current chunk frame by
//     frame, then each selected history block (through the slot table).
//     Tiles are staged in LDS, K row-major and V transposed, from registers
//     that were prefetched from HBM while the previous tile was computed.
//   * MFMA 32x32x16 bf16 (32x32x2 f32 for fp32 inputs). Scores are formed
//     transposed, S^T = K Q^T (A = K from LDS, B = Q kept in registers for
//     the whole kernel), so that each lane ends up holding one query's
//     scores; softmax statistics need only one cross-lane exchange (lane
//     l and l^32), and the probabilities feed the next MFMA, O^T = V^T P^T,
//     straight from registers as its B operand. V^T is written to LDS with
//     the keys of each 16-key group permuted so that the A operand of every
//     lane is one contiguous 16-byte LDS read.
//   * exp2 with the scale folded into log2(e) units; masked (ragged) keys
//     are -inf; rows past the end of a ragged query block are computed on
//     zero queries and never stored.
#include "lf_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

// Per-dtype MFMA traits.
template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int KSTEP = 16;  // reduction length per MFMA
  using frag = bf16x8;
  static __device__ inline f32x16 mfma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // LDS position of key `key` in a transposed V row: inside each group of
  // 16 keys, key 8*a + 4*h + c goes to 8*h + 4*a + c, so that lane half h
  // reads its 8 keys {8a + 4h + c} of one MFMA step as one 16-byte run.
  static __device__ inline int vpos(int key) {
    return (key & ~15) | ((key & 4) << 1) | ((key & 8) >> 1) | (key & 3);
  }
};

template <>
struct Mma<float> {
  static constexpr int KSTEP = 2;
  using frag = float;
  static __device__ inline f32x16 mfma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ inline int vpos(int key) { return key; }
};

// Key index held by accumulator register r of lane half h in a 32x32 MFMA
// output (rows = keys): 8*(r/4) + 4*h + r%4.
__device__ inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

struct TileRef {
  int64_t off;  // element offset of the tile's first key row in the cache
  int count;    // valid keys in the tile (0: skip)
};

template <typename T, int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                                                       const T* __restrict__ vc, const int32_t* __restrict__ sel,
                                                       const int32_t* __restrict__ nsel, int max_sel, float scale,
                                                       const KGeom g, T* __restrict__ out, float* __restrict__ lse) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int NT = NW * 64;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;              // chunks per key row
  constexpr int KST = D + EPC;              // padded LDS row of K (elements)
  constexpr int VST = BN + EPC;             // padded LDS row of V^T (elements)
  constexpr int KTOT = BN * CPR;            // 16-byte K chunks per tile
  constexpr int VTOT = (BN / 4) * CPR;      // V units (4 keys x 1 chunk) per tile
  constexpr int KCH = (KTOT + NT - 1) / NT; // per thread
  constexpr int VUN = (VTOT + NT - 1) / NT;
  constexpr int QSTEPS = D / M::KSTEP;
  constexpr int KH = BN / 32;               // 32-key halves per tile
  constexpr int PSTEPS = BN / M::KSTEP;     // PV reduction steps per tile
  constexpr int DB = D / 32;                // 32-wide output column blocks
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) T Ks[BN * KST];
  __shared__ __attribute__((aligned(16))) T Vt[D * VST];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;

  // XCD-aware remap of the workgroup id to a work item.
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int xcd = wg & 7, idx = wg >> 3, per = nwg >> 3, rem = nwg & 7;
  const int item = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int64_t bh = item / g.nqb;
  const int qb = item - (int)bh * g.nqb;
  const int fc = qb / g.nb, jq = qb - fc * g.nb;
  const int64_t qrow0 = (int64_t)fc * g.T + (int64_t)jq * g.b;
  const int nrows = min(g.b, g.T - jq * g.b);

  // Queries of this wave (B operand of S^T = K Q^T), kept for the whole walk.
  const int qr = wv * 32 + l32;
  const bool wave_active = wv * 32 < nrows;
  frag qf[QSTEPS];
  {
    const T* qp = q + (bh * g.Lq + qrow0 + min(qr, nrows - 1)) * D;
    const bool ok = qr < nrows;
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) {
      if constexpr (sizeof(T) == 2) {
        const uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + s * 16 + 8 * h) : make_uint4(0u, 0u, 0u, 0u);
        qf[s] = __builtin_bit_cast(bf16x8, v);
      } else {
        qf[s] = ok ? qp[s * 2 + h] : 0.0f;
      }
    }
  }

  // Key walk: Fc frames of the current chunk (tiles of BN keys), then the
  // selected history blocks (tiles of up to BN keys inside each block).
  const int tpf = (g.T + BN - 1) / BN;
  const int tpb = (g.b + BN - 1) / BN;
  const int n_cur = g.Fc * tpf;
  const int64_t sel_row = bh * g.nqb + qb;
  const int nsel_q = max_sel > 0 ? min(max(nsel[sel_row], 0), max_sel) : 0;
  const int32_t* my_sel = sel + sel_row * max_sel;
  const int n_tiles = n_cur + nsel_q * tpb;
  const int n_hist_blocks = g.Fh * g.nb;
  const int64_t frame_elems = (int64_t)g.T * D;
  const int64_t bh_base = bh * g.S * frame_elems;

  auto tile_ref = [&](int t) -> TileRef {
    TileRef r;
    if (t < n_cur) {
      const int f = t / tpf, tt = t - f * tpf;
      const int start = tt * BN;
      r.count = min(BN, g.T - start);
      r.off = bh_base + g.slot[g.Fh + f] * frame_elems + (int64_t)start * D;
    } else {
      const int u = t - n_cur, s = u / tpb, sub = u - s * tpb;
      const int id = my_sel[s];
      if (id < 0 || id >= n_hist_blocks) {
        r.count = 0;
        r.off = 0;
      } else {
        const int f = id / g.nb, j = id - f * g.nb;
        const int bstart = j * g.b, bend = min(bstart + g.b, g.T);
        const int start = bstart + sub * BN;
        r.count = max(0, min(BN, bend - start));
        r.off = bh_base + g.slot[f] * frame_elems + (int64_t)start * D;
      }
    }
    return r;
  };
  auto next_tile = [&](int t) {
    while (t < n_tiles && tile_ref(t).count == 0) ++t;
    return t;
  };

  uint4 kreg[KCH];
  uint4 vreg[VUN][4];
  auto load_tile = [&](const TileRef& r) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * NT, row = c / CPR, cc = c - row * CPR;
      kreg[i] = (KTOT % NT == 0 || c < KTOT) && row < r.count
                    ? *reinterpret_cast<const uint4*>(kc + r.off + (int64_t)row * D + cc * EPC)
                    : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + i * NT, quad = u / CPR, cc = u - quad * CPR;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int row = quad * 4 + k4;
        vreg[i][k4] = (VTOT % NT == 0 || u < VTOT) && row < r.count
                          ? *reinterpret_cast<const uint4*>(vc + r.off + (int64_t)row * D + cc * EPC)
                          : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * NT, row = c / CPR, cc = c - row * CPR;
      if (KTOT % NT == 0 || c < KTOT) *reinterpret_cast<uint4*>(&Ks[row * KST + cc * EPC]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + i * NT, quad = u / CPR, cc = u - quad * CPR;
      if (VTOT % NT != 0 && u >= VTOT) continue;
      const int p0 = M::vpos(quad * 4);  // 4 consecutive keys stay consecutive
      if constexpr (sizeof(T) == 2) {
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[i][3]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int wi = e >> 1;
          uint32_t lo, hi;
          if (e & 1) {
            lo = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
            hi = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
          } else {
            lo = (w0[wi] & 0xffffu) | (w1[wi] << 16);
            hi = (w2[wi] & 0xffffu) | (w3[wi] << 16);
          }
          *reinterpret_cast<uint2*>(&Vt[(cc * EPC + e) * VST + p0]) = make_uint2(lo, hi);
        }
      } else {
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[i][2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[i][3]);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          *reinterpret_cast<uint4*>(&Vt[(cc * EPC + e) * VST + p0]) = make_uint4(w0[e], w1[e], w2[e], w3[e]);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const float c2 = scale * kLog2e;

  int t = next_tile(0);
  TileRef cur = tile_ref(t < n_tiles ? t : 0);
  if (t < n_tiles) load_tile(cur);
  while (t < n_tiles) {
    __syncthreads();  // every wave is done with the previous tile in LDS
    store_tile();
    __syncthreads();
    const int tn = next_tile(t + 1);
    TileRef nxt = cur;
    if (tn < n_tiles) {
      nxt = tile_ref(tn);
      load_tile(nxt);  // in flight while this tile is computed
    }
    if (wave_active) {
      // S^T = K Q^T, 32 keys x 32 queries per accumulator.
      f32x16 s[KH];
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kh][r] = 0.0f;
        const T* krow = &Ks[(kh * 32 + l32) * KST];
#pragma unroll
        for (int st = 0; st < QSTEPS; ++st) {
          frag a;
          if constexpr (sizeof(T) == 2)
            a = *reinterpret_cast<const bf16x8*>(krow + st * 16 + 8 * h);
          else
            a = krow[st * 2 + h];
          s[kh] = M::mfma(a, qf[st], s[kh]);
        }
      }
      if (cur.count < BN) {
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kh * 32 + acc_row(r, h) >= cur.count) s[kh][r] = -INFINITY;
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kh][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      const float mc = m_new * c2;
      float psum = 0.0f;
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kh][r], c2, -mc));
          s[kh][r] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      // O^T += V^T P^T.
#pragma unroll
      for (int ps = 0; ps < PSTEPS; ++ps) {
        frag b;
        if constexpr (sizeof(T) == 2) {
          const int kh = ps >> 1, r0 = (ps & 1) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = (__bf16)s[kh][r0 + e];
        } else {
          b = s[ps >> 4][ps & 15];
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const T* vrow = &Vt[(db * 32 + l32) * VST];
          frag a;
          if constexpr (sizeof(T) == 2)
            a = *reinterpret_cast<const bf16x8*>(vrow + ps * 16 + 8 * h);
          else
            a = vrow[M::vpos((ps >> 4) * 32 + acc_row(ps & 15, h))];
          o[db] = M::mfma(a, b, o[db]);
        }
      }
    }
    t = tn;
    cur = nxt;
  }

  if (!wave_active || qr >= nrows) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  T* orow = out + (bh * g.Lq + qrow0 + qr) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int col = db * 32 + 8 * a4 + 4 * h;
      if constexpr (sizeof(T) == 2) {
        bf16x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (__bf16)(o[db][a4 * 4 + c] * inv);
        *reinterpret_cast<bf16x4*>(orow + col) = v;
      } else {
        *reinterpret_cast<float4*>(orow + col) =
            make_float4(o[db][a4 * 4] * inv, o[db][a4 * 4 + 1] * inv, o[db][a4 * 4 + 2] * inv, o[db][a4 * 4 + 3] * inv);
      }
    }
  if (lse != nullptr && h == 0) lse[bh * g.Lq + qrow0 + qr] = m_run * scale + logf(l_tot);
}

template <typename T, int D, int NW, int BN>
hipError_t launch_typed(const KGeom& g, const void* q, const void* k, const void* v, const int32_t* sel,
                        const int32_t* nsel, int max_sel, float scale, void* out, float* lse, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)g.B * g.H * g.nqb);
  hipLaunchKernelGGL((attn_kernel<T, D, NW, BN>), dim3(grid), dim3(NW * 64), 0, stream, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v), sel, nsel, max_sel, scale, g,
                     static_cast<T*>(out), lse);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const KGeom& g, const void* q, const void* k, const void* v, const int32_t* sel,
                    const int32_t* nsel, int max_sel, float scale, void* out, float* lse, hipStream_t stream) {
  if (g.b <= 32) return launch_typed<T, D, 1, 32>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
  if (g.b <= 64) return launch_typed<T, D, 2, 64>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
  return launch_typed<T, D, 4, 64>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
}

}  // namespace

hipError_t launch_attention(const KGeom& g, int32_t dtype, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel, float scale, void* out,
                            float* lse, hipStream_t stream) {
  if (dtype == LF_BF16) {
    if (g.D == 128) return launch_d<__bf16, 128>(g, q, k_cache, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
    return launch_d<__bf16, 64>(g, q, k_cache, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
  }
  if (g.D == 128) return launch_d<float, 128>(g, q, k_cache, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
  return launch_d<float, 64>(g, q, k_cache, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
}

}  // namespace lf
