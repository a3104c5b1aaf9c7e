// Block-sparse attention over a rolling/anchored KV cache (Light Forcing,
// technical summary 2.2 "execution"; press summary section 3): every query
// of a query block attends to its selected history blocks and to the whole
// current chunk, softmax(scale q k^T) v, with an fp32 online softmax.
//
// gfx950 design
//   * WPQ = ceil(block/32) wavefronts per query block, 32 query rows each.
//     Two walks share the tile math:
//       - single-stage (bf16, 32 < block <= 64): a workgroup is one query
//         block; LDS holds one K and one V tile (four workgroups per CU).
//         Per tile, the V tile streams in under the score MFMAs and the
//         next K tile under the PV MFMAs, with a barrier between the phases.
//       - double-buffered (every other case): a workgroup owns 128 query
//         rows (4/WPQ query blocks of one head) and walks the ascending,
//         de-duplicated union of their selected history blocks; a tile is
//         loaded once and only the wavefronts whose query block selected it
//         compute on it. One barrier per tile.
//     Either walk starts with the current chunk's tiles, then the history
//     tiles of a table built in LDS at the start of the workgroup.
//   * Work is dealt XCD-aware: the hardware hands workgroups round-robin to
//     the 8 XCDs, so workgroup w is remapped such that each XCD gets one
//     contiguous range of (batch, head, query-block group) items; query
//     blocks of one head then share that head's keys/values in one L2.
//   * Key/value tiles of BN = 64 keys go HBM -> LDS with buffer loads that
//     write LDS directly (16 bytes per lane, no registers). Each tile's
//     buffer resource covers only its valid rows, so rows past the end of a
//     ragged block read as zeros (then masked) and no load leaves the tile.
//     LDS rows of bf16 keys and values at d = 128 are 256 bytes with their
//     16-byte chunks XOR-swizzled per row (lds_swizzle), other rows are
//     padded; either way the fragment reads spread over the banks and every
//     fragment address is one per-lane base XOR (or plus) a constant.
//   * MFMA 32x32x16 bf16 (32x32x2 f32 for fp32 inputs). Scores are formed
//     transposed, S^T = K Q^T (A = K from LDS, B = this wavefront's 32
//     queries, kept in registers for the whole walk), so each lane holds one
//     query's scores: the softmax needs one cross-lane exchange (lane l and
//     l^32) and the probabilities are the B operand of O^T = V^T P^T straight
//     from registers. The A operand V^T comes from the row-major V tile with
//     ds_read_tr16_b64: inside each 16-lane group it hands lane i element
//     i&3 of source lane 4e+(i>>2), i.e. four consecutive keys of one column.
//   * Online softmax in fp32 with exp2 (scale folded into log2(e) units)
//     against the running maximum, without a per-tile maximum; a rarely
//     taken exact branch rescales when a half's probabilities could grow too
//     large. The normaliser sums the probabilities in float32, before they
//     are rounded to bf16 for the PV product.
//   * Wave priorities by stage of a tile (s_setprio): the MFMA-only chains
//     lowest, the loops that carry the exponentials highest, so that the
//     two wavefronts sharing a SIMD overlap softmax and matrix work.
//   * FP8 variant (press summary section 5: FP8 with per-token activation
//     scales; either walk, D = 128): queries and keys as E4M3 codes
//     with E8M0 scales per 32 channels of a token, scores on the scaled FP8
//     MFMA (32x32x64); V, P and the rest as in the bf16 walk.
//   * Rows past the end of a ragged query block are computed on zero
//     queries and never stored.
#include "mfma.h"

namespace lf {
namespace {

constexpr int BN = 64;     // keys per tile
// bf16 blocks of 33..64 keys use the single-stage kernel (one query block
// per workgroup) instead of the double-buffered one.
constexpr bool kSingleStage = true;

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int KSTEP = 16;  // reduction length per MFMA
  using frag = bf16x8;
  static __device__ inline f32x16 mfma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int KSTEP = 2;
  using frag = float;
  static __device__ inline f32x16 mfma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Pins a computed value at this point of the program: an empty asm that
// claims to modify the register, so no optimisation pass moves the
// computation past it (the scheduling fences alone bind only the final
// instruction scheduler). Emits no instruction.
__device__ inline float pin(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Wavefronts per SIMD to plan registers for (the second launch bound). With
// bf16, LDS holds two workgroups' stage buffers, i.e. two wavefronts per
// SIMD (256 registers each), which pair up so that one's softmax hides under
// the other's MFMAs. Blocks of at most 32 keys (four query blocks per
// workgroup, a larger walk table) fit one workgroup per CU, and fp32 inputs
// (small, correctness-oriented shapes) run one wavefront per SIMD with the
// whole register file.
template <typename T, int WPQ>
constexpr int WAVES_PER_SIMD = sizeof(T) == 2 && WPQ > 1 ? 2 : 1;


// One workgroup's walk: per-wavefront query fragments and accumulators, the
// scalar tile producer, the LDS loader and the per-tile math.
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Q8 (bf16 walks only): queries and keys arrive as E4M3 codes with one E8M0
// scale per 32 channels of a token; the scores are formed with the scaled
// FP8 MFMA (32x32x64), everything after them as in the bf16 walk.
template <typename T, int D, int WPQ, int QPWT = 4 / WPQ, bool Q8 = false>
struct Walk {
  using M = Mma<T>;
  using frag = typename M::frag;
  static constexpr int QPW = QPWT;                 // query blocks per workgroup
  static constexpr int NW = WPQ * QPW;             // wavefronts
  static constexpr int NT = 64 * NW;
  static constexpr int ES = (int)sizeof(T);
  static constexpr int CPR = D * ES / 16;          // 16-byte chunks per key row
  // LDS row layout. K and V tiles are read differently (16-byte reads of 32
  // rows for K; transposing 8-byte reads that gather 4 row pieces of 32
  // bytes per 16 lanes for V). Rows other than those below are padded by 32
  // bytes, which spreads both reads over the banks well enough at those
  // sizes, and every fragment address is one per-lane base plus a constant.
  static constexpr int KES = Q8 ? 1 : ES;                       // bytes per key element
  static constexpr int CPRK = D * KES / 16;                     // 16-byte chunks per key row
  // bf16 rows of 256 bytes (D = 128) are stored unpadded with the 16-byte
  // chunks of row r permuted: LDS chunk c' of row r holds chunk c' ^ sw(r),
  // sw(r) = 4*(r%4) + (r/4)%4. Both read patterns are then free of bank
  // conflicts: the K reads (16 consecutive rows, one chunk each: sw takes all
  // 16 values) and the transposing V reads (4 consecutive rows from a
  // multiple of 4, 4 consecutive chunks each: (4a + m) ^ (4k + q) takes 16
  // values over rows k and chunks m). The DMA writes stay contiguous, no
  // pad bytes are loaded, and a read address is a per-lane base XOR a
  // constant.
  static constexpr bool kSwzK = ES == 2 && D == 128 && !Q8;
  static constexpr bool kSwzV = ES == 2 && D == 128;
  // (FP8 key rows: 16-byte pad, the two 16-byte reads per lane of a row
  // then fall in distinct bank groups)
  static constexpr int RSK = kSwzK ? 256 : D * KES + (Q8 ? 16 : 32);  // K row pitch in bytes
  static constexpr int RSV = kSwzV ? 256 : D * ES + 32;                // V row pitch in bytes
  static constexpr int SPRK = RSK / 16, SPRV = RSV / 16;       // 16-byte slots per row (CPR data + pad)
  static constexpr int SLOTS_K = BN * SPRK, SLOTS_V = BN * SPRV;
  static constexpr int LIK = (SLOTS_K + NT - 1) / NT;          // load instructions per wavefront per K tile
  static constexpr int LIV = (SLOTS_V + NT - 1) / NT;          // ... per V tile
  static constexpr int LI = LIK > LIV ? LIK : LIV;
  static constexpr int TILE_BYTES_K = BN * RSK, TILE_BYTES_V = BN * RSV;
  static constexpr int TILE_ALLOC_K = TILE_BYTES_K + (Q8 ? 4 * BN : 0);  // Q8: + one scale word per key
  static constexpr int QSTEPS = D / M::KSTEP;
  static constexpr int DB = D / 32;
  static_assert(SLOTS_K % 64 == 0 && SLOTS_V % 64 == 0, "whole load instructions");

  __device__ __forceinline__ explicit Walk(const KGeom& geom) : g(geom) {}

  // geometry (a reference to the kernel argument: copying it would put the
  // slot table in scratch memory) and identity
  const KGeom& g;
  const T* kc;
  const T* vc;
  const uint8_t* kc8;   // Q8: key codes [B,H,S,T,D]
  const uint8_t* ksc8;  // Q8: key scales [B,H,S,T,D/32]
  int lane, wv, h, l32, lq, nrows, qr, qb0;
  bool wave_active;
  int64_t bh, qrow0;
  // per-wavefront state
  frag qf[Q8 ? 1 : QSTEPS];
  i32x8 qf8[Q8 ? D / 64 : 1];  // Q8: this lane's query codes for each 64-channel step
  uint32_t qsw;                // Q8: its four block scales, shifted so byte 2t serves step t
  f32x16 o[DB];
  float m_run, l_run, c2;
  // producer state (uniform)
  const uint32_t* walk;  // LDS table of history tiles, see the kernel
  int tpf, n_cur, n_tiles, all_mask, t_next, cf, ct;
  int64_t frame_elems, bh_base, cur_base;

  // Fills (off, count, mask) of the next tile: the current chunk's tiles in
  // order (counters, no divisions), then the history tiles of the table;
  // false when the walk is over.
  __device__ __forceinline__ bool produce(int64_t& off, int& count, int& mask) {
    if (t_next >= n_tiles) return false;
    if (t_next < n_cur) {
      const int start = ct * BN;
      off = cur_base + (int64_t)start * D;
      count = min(BN, g.T - start);
      mask = all_mask;
      if (++ct == tpf) {
        ct = 0;
        ++cf;
        cur_base = bh_base + (int64_t)g.slot[g.Fh + min(cf, g.Fc - 1)] * frame_elems;
      }
    } else {
      const uint32_t e = __builtin_amdgcn_readfirstlane(walk[t_next - n_cur]);
      const int slot = (int)(e & 16383u), j = (int)((e >> 14) & 511u), half = (int)((e >> 23) & 1u);
      const int start = j * g.b + half * BN;
      off = bh_base + (int64_t)slot * frame_elems + (int64_t)start * D;
      count = min(BN, min(j * g.b + g.b, g.T) - start);
      mask = (int)(e >> 24);
    }
    ++t_next;
    return true;
  }

  // All wavefronts stream one tile (K and V) into a stage buffer.
  // Load instruction i of a wavefront fills 64 consecutive 16-byte LDS slots
  // (lane l the l-th); this lane's slot holds chunk c of key row `row`, i.e.
  // byte offset row*D*ES + c*16 from the tile's first key.
  uint32_t doffk[LIK], doffv[LIV];
  static __device__ __forceinline__ int swz(int row) { return lds_swizzle(row); }
  static __device__ __forceinline__ uint32_t slot_offset(int slot, int spr, int cpr, int row_bytes, bool swizzled) {
    if (swizzled) {  // 16 slots per row, no pad: slot (row, c') holds chunk c' ^ sw(row)
      const int row = slot >> 4;
      return (uint32_t)(row * row_bytes + (((slot & 15) ^ swz(row)) * 16));
    }
    const int row = min(slot / spr, BN - 1);
    int c = slot - (slot / spr) * spr;
    while (c >= cpr) c -= cpr;  // a pad slot re-reads a chunk its row already loads (same cache line)
    return (uint32_t)(row * row_bytes + c * 16);
  }
  __device__ __forceinline__ void init_loads() {
#pragma unroll
    for (int i = 0; i < LIK; ++i) doffk[i] = slot_offset((i * NW + wv) * 64 + lane, SPRK, CPRK, D * KES, kSwzK);
#pragma unroll
    for (int i = 0; i < LIV; ++i) doffv[i] = slot_offset((i * NW + wv) * 64 + lane, SPRV, CPR, D * ES, kSwzV);
  }

  // The next tile's loads, described at the top of an iteration and issued
  // from inside the current tile's math so the memory pipeline sees a steady
  // trickle instead of a burst. Each tensor's tile is addressed through a
  // buffer resource whose size is the tile's valid rows: the hardware returns
  // zeros for rows past `count`, so a ragged tile needs no per-lane clamping
  // and no load leaves the tile.
  struct Next {
    __amdgpu_buffer_rsrc_t rk, rv, rks;  // rks: Q8 key scales of the tile
    char* kd;
    char* vd;
  };
  // When the walk has no next tile the caller passes the last one again: it
  // is re-read into the idle buffer, which nothing reads any more (cheaper
  // than a branch around every load).
  __device__ __forceinline__ Next next_tile(char* kd, char* vd, int64_t off, int count) const {
    Next n;
    const int bytes = count * D * ES;
    if constexpr (Q8) {  // key codes (one byte each) and their scales (D/32 bytes per key)
      n.rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(uniform_ptr(kc8 + off)), (short)0, count * D,
                                               kRawBufferFlags);
      n.rks = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(uniform_ptr(ksc8 + off / 32)), (short)0,
                                                count * (D / 32), kRawBufferFlags);
    } else {
      n.rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(uniform_ptr(kc + off)), (short)0, bytes, kRawBufferFlags);
    }
    n.rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(uniform_ptr(vc + off)), (short)0, bytes, kRawBufferFlags);
    n.kd = kd;
    n.vd = vd;
    return n;
  }
  // Load instruction i (of LI) of the K (V == false) or V tile.
  // (Called with i a constant of an unrolled loop.)
  template <bool V>
  __device__ __forceinline__ void issue_one(const Next& n, int i) const {
    constexpr int NL = V ? LIV : LIK, SLOTS = V ? SLOTS_V : SLOTS_K;
    if (i < NL) {
      const int L0 = (i * NW + wv) * 64;
      // (the buffer-to-LDS builtin exists only for the device compilation
      // pass; the host pass never runs this function)
#if defined(__HIP_DEVICE_COMPILE__)
      if ((i + 1) * NT <= SLOTS || L0 < SLOTS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(V ? n.rv : n.rk, LDS_PTR(void, (V ? n.vd : n.kd) + L0 * 16), 16,
                                                 V ? doffv[i] : doffk[i], 0, 0, 0);
      if constexpr (Q8 && !V) {  // the 64 keys' scale words, 4 bytes per lane, behind the key tile
        static_assert(D == 128, "one 4-byte scale word per key");
        if (i == 0 && wv == 0)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(n.rks, LDS_PTR(void, n.kd + TILE_BYTES_K), 4, lane * 4, 0, 0, 0);
      }
#else
      (void)n;
      (void)L0;
      (void)SLOTS;
#endif
    }
  }
  template <bool V>
  __device__ __forceinline__ void issue_all(const Next& n) const {
#pragma unroll
    for (int i = 0; i < LI; ++i) issue_one<V>(n, i);
  }
  __device__ __forceinline__ void issue(const Next& n) const {
#pragma unroll
    for (int i = 0; i < LI; ++i) {
      issue_one<false>(n, i);
      issue_one<true>(n, i);
    }
  }

  // Wave priorities. A tile's first score chain and its last PV chain are
  // MFMAs and fragment reads only (priority 0); the two loops that
  // interleave the other chains with a half's exponentials come first
  // (priority 2); the rest (bf16 packing, sums, checks, the producer) sits
  // between (1). Two wavefronts share a SIMD: when one is in an MFMA-only
  // chain, the other's softmax instructions win the issue slot and run
  // under that chain instead of waiting behind it. (480p, one process,
  // launches interleaved with the build without priorities: 5% faster; with
  // two levels, 0 for the MFMA-only chains and 1 for the rest, 3%.)
  static __device__ __forceinline__ void mfma_only_begin() { __builtin_amdgcn_s_setprio(0); }
  static __device__ __forceinline__ void mfma_only_end() { __builtin_amdgcn_s_setprio(1); }
  static __device__ __forceinline__ void softmax_begin() { __builtin_amdgcn_s_setprio(2); }
  static __device__ __forceinline__ void softmax_end() { __builtin_amdgcn_s_setprio(1); }

  // ---- bf16 tile math ----------------------------------------------------
  // K fragments of key half kh (keys 32kh .. 32kh+31) for S^T = K Q^T.
  __device__ __forceinline__ void load_k(const char* ks, int kh, frag (&kf)[QSTEPS]) const {
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) kf[t] = load_k1(ks, kh, t);
  }
  __device__ __forceinline__ frag load_k1(const char* ks, int kh, int t) const {
    if constexpr (kSwzK) {
      // chunk 2t+h of row r sits at chunk (2t+h) ^ sw(r): with sw = 2*xh + x0,
      // byte offset 32*(t ^ xh) + 16*(h ^ x0), i.e. a per-lane base XOR 32t
      const int x = swz(l32);
      const uint32_t base = (uint32_t)(l32 * 256 + 32 * (x >> 1) + 16 * (h ^ (x & 1)));
      return *reinterpret_cast<const bf16x8*>(ks + kh * 32 * 256 + (base ^ (uint32_t)(32 * t)));
    } else {
      return *reinterpret_cast<const bf16x8*>(ks + (kh * 32 + l32) * RSK + h * 16 + t * 32);
    }
  }
  // V^T fragments (A operand) of the 16-key step ps for every 32-column block.
  __device__ __forceinline__ void load_v(const char* vs, int ps, bf16x8 (&a)[DB]) const {
#pragma unroll
    for (int db = 0; db < DB; ++db) a[db] = load_v1(vs, ps, db);
  }
  __device__ __forceinline__ bf16x8 load_v1(const char* vs, int ps, int db) const {
    const int s16 = lane & 15;
    i16x4 part[2];
    if constexpr (kSwzV) {
      // row 4h + s16/4 + 16ps + 8j (sw = 4*(s16/4) + h + 2j), chunk
      // 4db + cb with cb = 2*((lane/16)&1) + (s16&3)/2, half s16&1: the chunk
      // bits are (4*(s16/4) + (cb ^ h)) ^ (4db + 2j), a per-lane base XOR a
      // constant; the row offset 16ps + 8j is added after.
      const int cb = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
      const uint32_t base = (uint32_t)((4 * h + (s16 >> 2)) * 256 + 16 * (4 * (s16 >> 2) + (cb ^ h)) + 8 * (s16 & 1));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        part[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            LDS_PTR(i16x4, vs + (16 * ps + 8 * j) * 256 + (base ^ (uint32_t)(16 * (4 * db + 2 * j)))));
    } else {
      // lane's key inside an 8-key group and its first column inside a 32-column block
      const char* vbase = vs + (4 * h + (s16 >> 2)) * RSV + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        part[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vbase + (16 * ps + 8 * j) * RSV + 64 * db));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
  }
  __device__ __forceinline__ void mask_half(f32x16& s, int kh, int count) const {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kh * 32 + acc_row(r, h) >= count) s[r] = -INFINITY;
  }
  __device__ __forceinline__ void to_bf16(const f32x16& p, bf16x8& b0, bf16x8& b1) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b0[e] = (__bf16)p[e];
      b1[e] = (__bf16)p[8 + e];
    }
  }
  // Sum of a lane's 16 float32 probabilities (a tree of adds), taken before
  // they are rounded to bf16 for the PV product. Plain float adds rather than
  // the bf16 dot instruction: on gfx950 a dot product waits for the matrix
  // core while another wavefront's MFMAs run (3.5x slower beside them in an
  // issue probe; float adds 1.4x).
  static __device__ __forceinline__ float psum(const f32x16& p) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return (t[0] + t[1]) + (t[2] + t[3]);
  }
  // The exact path for one half, taken when the fast path's probabilities
  // could be too large (or the walk has no reference yet): recompute the
  // half's scores, move the reference to the true running max (both lanes of
  // a query row agree on it), rescale O and l, and redo the exponentials.
  // Returns this lane's sum of the half's probabilities.
  __device__ __forceinline__ float exact_half(const char* ks, int kh, int count, f32x16& s) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    // one fragment at a time (fenced): this path is rare and must not raise
    // the register high-water mark of the kernel
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      s = M::mfma(load_k1(ks, kh, t), qf[t], s);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (count < (kh + 1) * 32) mask_half(s, kh, count);
    return exact_from_scores(s);
  }
  // O *= alpha in place. Each multiply is a tied asm operand so the scaled
  // accumulators keep their registers: with a plain multiply the register
  // allocator may put the result elsewhere and then copy all of O back on the
  // common path, where the rescale branch is not taken.
  __device__ __forceinline__ void rescale_o(float alpha) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
  // The exact path from a half's masked raw scores (in s; probabilities out).
  __device__ __forceinline__ float exact_from_scores(f32x16& s) {
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    l_run *= alpha;
    m_run = m_new;
    rescale_o(alpha);
    const float mc = m_run * c2;
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc));
      ps += s[r];
    }
    return ps;  // (the bf16 path re-sums after rounding; the fp32 path uses this)
  }

  // One bf16 tile. Online softmax without a per-tile max: probabilities are
  // taken against the running reference m_run as they are, and only if some
  // lane's sum of a half exceeds 2^16 (or is not finite: no reference yet)
  // does the exact path run. Softmax is invariant to the reference, so this
  // is exact in real arithmetic; values stay far from float32 overflow.
  // Four groups, fenced so the MFMAs of one stage run while the exponentials
  // of the previous one are computed: S0 | S1 + softmax(S0) | PV0 +
  // softmax(S1) | PV1. The next tile's loads ride along in the first two.
  static constexpr float kFastLimit = 65536.0f;
  __device__ __forceinline__ void compute_bf16(const char* ks, const char* vs, int count, const Next& nx) {
#define LF_FENCE __builtin_amdgcn_sched_barrier(0)
    frag kf[QSTEPS];
    bf16x8 va[DB];
    f32x16 s0, s1;
    // A: S0 = K[0:32] Q^T; each K fragment register is refilled with the
    // matching K[32:64] fragment as soon as its MFMA has been issued, and the
    // next K tile's DMA goes out.
    load_k(ks, 0, kf);
    LF_FENCE;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = 0.0f;
    mfma_only_begin();
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      s0 = M::mfma(kf[t], qf[t], s0);
      kf[t] = load_k1(ks, 1, t);
      if (t & 1) issue_one<false>(nx, t / 2);
      LF_FENCE;
    }
    mfma_only_end();
#pragma unroll
    for (int i = QSTEPS / 2; i < LI; ++i) issue_one<false>(nx, i);
    if (count < 32) mask_half(s0, 0, count);
    LF_FENCE;
    // B: S1 = K[32:64] Q^T with the softmax of S0 between its MFMAs; the
    // first V fragments are read and the next V tile's DMA goes out.
    float mc = m_run * c2;
    float ps0 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s1[r] = 0.0f;
    softmax_begin();
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      s1 = M::mfma(kf[t], qf[t], s1);
      LF_FENCE;
#pragma unroll
      for (int u = 0; u < 16 / QSTEPS; ++u) {
        const int r = t * (16 / QSTEPS) + u;
        s0[r] = pin(__builtin_amdgcn_exp2f(fmaf(s0[r], c2, -mc)));
      }
      if (t >= QSTEPS - DB) va[t - (QSTEPS - DB)] = load_v1(vs, 0, t - (QSTEPS - DB));
      if (t & 1) issue_one<true>(nx, t / 2);
      LF_FENCE;
    }
    softmax_end();
#pragma unroll
    for (int i = QSTEPS / 2; i < LI; ++i) issue_one<true>(nx, i);
    bf16x8 b0, b1;
    to_bf16(s0, b0, b1);
    ps0 = psum(s0);
    if (__builtin_amdgcn_ballot_w64(!(ps0 <= kFastLimit)) != 0) {
      exact_half(ks, 0, count, s0);
      to_bf16(s0, b0, b1);
      ps0 = psum(s0);
    }
    l_run += ps0;
    if (count < BN) mask_half(s1, 1, count);
    LF_FENCE;
    // C: O^T += V[0:32]^T P0^T with the softmax of S1 between its MFMAs. V
    // fragments roll: after the MFMA of 16-key step ps, column block db, the
    // register is refilled with step ps+1's fragment of the same block.
    mc = m_run * c2;
    float ps1 = 0.0f;
    softmax_begin();
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int ps = j / DB, db = j % DB;
      o[db] = M::mfma(va[db], ps == 0 ? b0 : b1, o[db]);
      va[db] = load_v1(vs, ps + 1, db);
      LF_FENCE;
#pragma unroll
      for (int u = 0; u < 16 / (2 * DB); ++u) {
        const int r = j * (16 / (2 * DB)) + u;
        s1[r] = pin(__builtin_amdgcn_exp2f(fmaf(s1[r], c2, -mc)));
      }
      LF_FENCE;
    }
    softmax_end();
    to_bf16(s1, b0, b1);
    ps1 = psum(s1);
    if (__builtin_amdgcn_ballot_w64(!(ps1 <= kFastLimit)) != 0) {
      exact_half(ks, 1, count, s1);
      to_bf16(s1, b0, b1);
      ps1 = psum(s1);
    }
    l_run += ps1;
    LF_FENCE;
    // D: O^T += V[32:64]^T P1^T.
    mfma_only_begin();
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int ps = 2 + j / DB, db = j % DB;
      o[db] = M::mfma(va[db], ps == 2 ? b0 : b1, o[db]);
      if (ps == 2) va[db] = load_v1(vs, 3, db);
      LF_FENCE;
    }
    mfma_only_end();
#undef LF_FENCE
  }

  // ---- FP8 scores (Q8) ----------------------------------------------------
  // Fragment of key half kh for the 64-channel step t of the scaled FP8 MFMA
  // (32x32x64): lane half h holds channels 64t+16h .. +15 in bytes 0..15 and
  // 64t+32+16h .. +15 in bytes 16..31. With this split the MFMA's two scale
  // blocks per step are the contiguous channels 64t .. 64t+31 (its scale
  // from lane half 0) and 64t+32 .. 64t+63 (lane half 1), i.e. the tensors'
  // own 32-channel MX blocks. Queries are loaded the same way.
  __device__ __forceinline__ i32x8 load_k8(const char* ks, int kh, int t) const {
    const char* row = ks + (kh * 32 + l32) * RSK + 64 * t + 16 * h;
    const uint4 a = *reinterpret_cast<const uint4*>(row);
    const uint4 b = *reinterpret_cast<const uint4*>(row + 32);
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
  // This lane's key's scale word, shifted so that byte 2t holds the scale of
  // the block the lane half serves in step t (the MFMA picks byte 2t).
  __device__ __forceinline__ uint32_t kscale_word(const char* ks, int kh) const {
    return *reinterpret_cast<const uint32_t*>(ks + TILE_BYTES_K + (kh * 32 + l32) * 4) >> (8 * h);
  }
  template <int TT>
  static __device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c, uint32_t sa,
                                                 uint32_t sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 2 * TT, (int)sa, 2 * TT, (int)sb);
  }
  static __device__ __forceinline__ f32x16 mfma8_step(int t, const i32x8& a, const i32x8& b, const f32x16& c,
                                                      uint32_t sa, uint32_t sb) {
    return t == 0 ? mfma8<0>(a, b, c, sa, sb) : mfma8<1>(a, b, c, sa, sb);  // (t is a constant after unrolling)
  }
  __device__ __forceinline__ float exact_half_q8(const char* ks, int kh, int count, f32x16& s) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    const uint32_t sw = kscale_word(ks, kh);
#pragma unroll
    for (int t = 0; t < D / 64; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      s = mfma8_step(t, load_k8(ks, kh, t), qf8[t], s, sw, qsw);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (count < (kh + 1) * 32) mask_half(s, kh, count);
    return exact_from_scores(s);
  }

  // ---- single-stage tile (one K and one V buffer per workgroup) ----------
  // Phase 1 reads only the K tile: S0, then S1 with the softmax of S0
  // between its MFMAs; this tile's V DMA goes out meanwhile (the V buffer was
  // freed by the barrier before). Leaves P0 in b0/b1 and the raw S1.
  __device__ __forceinline__ void ss_phase1(const char* ks, int count, const Next& nv, f32x16& s1, bf16x8& b0,
                                            bf16x8& b1) {
#define LF_FENCE __builtin_amdgcn_sched_barrier(0)
    frag kf[QSTEPS];
    f32x16 s0;
    load_k(ks, 0, kf);
    LF_FENCE;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = 0.0f;
    mfma_only_begin();
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      s0 = M::mfma(kf[t], qf[t], s0);
      kf[t] = load_k1(ks, 1, t);
      issue_one<true>(nv, t);
      LF_FENCE;
    }
    mfma_only_end();
#pragma unroll
    for (int i = QSTEPS; i < LI; ++i) issue_one<true>(nv, i);
    if (count < 32) mask_half(s0, 0, count);
    LF_FENCE;
    const float mc = m_run * c2;
#pragma unroll
    for (int r = 0; r < 16; ++r) s1[r] = 0.0f;
    softmax_begin();
#pragma unroll
    for (int t = 0; t < QSTEPS; ++t) {
      s1 = M::mfma(kf[t], qf[t], s1);
      LF_FENCE;
#pragma unroll
      for (int u = 0; u < 16 / QSTEPS; ++u) {
        const int r = t * (16 / QSTEPS) + u;
        s0[r] = pin(__builtin_amdgcn_exp2f(fmaf(s0[r], c2, -mc)));
      }
      LF_FENCE;
    }
    softmax_end();
    to_bf16(s0, b0, b1);
    float ps0 = psum(s0);
    if (__builtin_amdgcn_ballot_w64(!(ps0 <= kFastLimit)) != 0) {
      exact_half(ks, 0, count, s0);
      to_bf16(s0, b0, b1);
      ps0 = psum(s0);
    }
    l_run += ps0;
    if (count < BN) mask_half(s1, 1, count);
#undef LF_FENCE
  }
  // Phase 1 of the FP8 walk: the same as ss_phase1 with the scores of each
  // half from D/64 scaled FP8 MFMAs (the V tile's loads spread over them).
  __device__ __forceinline__ void ss_phase1_q8(const char* ks, int count, const Next& nv, f32x16& s1, bf16x8& b0,
                                               bf16x8& b1) {
#define LF_FENCE __builtin_amdgcn_sched_barrier(0)
    constexpr int T8 = D / 64;
    i32x8 kf[T8];
    f32x16 s0;
    const uint32_t sw0 = kscale_word(ks, 0), sw1 = kscale_word(ks, 1);
#pragma unroll
    for (int t = 0; t < T8; ++t) kf[t] = load_k8(ks, 0, t);
    LF_FENCE;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = 0.0f;
    constexpr int PER = (LI + 2 * T8 - 1) / (2 * T8);  // V loads per MFMA
    mfma_only_begin();
#pragma unroll
    for (int t = 0; t < T8; ++t) {
      s0 = mfma8_step(t, kf[t], qf8[t], s0, sw0, qsw);
      kf[t] = load_k8(ks, 1, t);
#pragma unroll
      for (int u = 0; u < PER; ++u) issue_one<true>(nv, t * PER + u);
      LF_FENCE;
    }
    mfma_only_end();
    if (count < 32) mask_half(s0, 0, count);
    LF_FENCE;
    const float mc = m_run * c2;
#pragma unroll
    for (int r = 0; r < 16; ++r) s1[r] = 0.0f;
    softmax_begin();
#pragma unroll
    for (int t = 0; t < T8; ++t) {
      s1 = mfma8_step(t, kf[t], qf8[t], s1, sw1, qsw);
#pragma unroll
      for (int u = 0; u < PER; ++u) issue_one<true>(nv, (T8 + t) * PER + u);
      LF_FENCE;
#pragma unroll
      for (int u = 0; u < 16 / T8; ++u) {
        const int r = t * (16 / T8) + u;
        s0[r] = pin(__builtin_amdgcn_exp2f(fmaf(s0[r], c2, -mc)));
      }
      LF_FENCE;
    }
    softmax_end();
    to_bf16(s0, b0, b1);
    float ps0 = psum(s0);
    if (__builtin_amdgcn_ballot_w64(!(ps0 <= kFastLimit)) != 0) {
      exact_half_q8(ks, 0, count, s0);
      to_bf16(s0, b0, b1);
      ps0 = psum(s0);
    }
    l_run += ps0;
    if (count < BN) mask_half(s1, 1, count);
#undef LF_FENCE
  }
  // Phase 2 reads only the V tile (the next tile's K DMA goes out
  // meanwhile, so the rare exact path of S1 works from the saved raw
  // scores, not from K): PV0 with the softmax of S1 between its MFMAs, then
  // PV1.
  __device__ __forceinline__ void ss_phase2(const char* vs, const Next& nk, f32x16& s1, bf16x8& b0, bf16x8& b1) {
#define LF_FENCE __builtin_amdgcn_sched_barrier(0)
    bf16x8 va[DB];
    const f32x16 s1raw = s1;
    load_v(vs, 0, va);
    LF_FENCE;
    const float mc = m_run * c2;
    softmax_begin();
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int ps = j / DB, db = j % DB;
      o[db] = M::mfma(va[db], ps == 0 ? b0 : b1, o[db]);
      va[db] = load_v1(vs, ps + 1, db);
      issue_one<false>(nk, j);
      LF_FENCE;
#pragma unroll
      for (int u = 0; u < 16 / (2 * DB); ++u) {
        const int r = j * (16 / (2 * DB)) + u;
        s1[r] = pin(__builtin_amdgcn_exp2f(fmaf(s1[r], c2, -mc)));
      }
      LF_FENCE;
    }
#pragma unroll
    for (int i = 2 * DB; i < LI; ++i) issue_one<false>(nk, i);
    softmax_end();
    to_bf16(s1, b0, b1);
    float ps1 = psum(s1);
    if (__builtin_amdgcn_ballot_w64(!(ps1 <= kFastLimit)) != 0) {
      s1 = s1raw;
      exact_from_scores(s1);
      to_bf16(s1, b0, b1);
      ps1 = psum(s1);
    }
    l_run += ps1;
    LF_FENCE;
    mfma_only_begin();
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int ps = 2 + j / DB, db = j % DB;
      o[db] = M::mfma(va[db], ps == 2 ? b0 : b1, o[db]);
      if (ps == 2) va[db] = load_v1(vs, 3, db);
      LF_FENCE;
    }
    mfma_only_end();
#undef LF_FENCE
  }

  // One tile of the double-buffered walk with FP8 scores: compute_bf16 with
  // each half's scores from D/64 scaled FP8 MFMAs; the next tile's K loads
  // ride along the first half's, its V loads along the second half's.
  __device__ __forceinline__ void compute_q8(const char* ks, const char* vs, int count, const Next& nx) {
#define LF_FENCE __builtin_amdgcn_sched_barrier(0)
    constexpr int T8 = D / 64;
    constexpr int PK = (LIK + T8 - 1) / T8, PV = (LIV + T8 - 1) / T8;  // loads per MFMA
    i32x8 kf[T8];
    bf16x8 va[DB];
    f32x16 s0, s1;
    const uint32_t sw0 = kscale_word(ks, 0), sw1 = kscale_word(ks, 1);
#pragma unroll
    for (int t = 0; t < T8; ++t) kf[t] = load_k8(ks, 0, t);
    LF_FENCE;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = 0.0f;
    mfma_only_begin();
#pragma unroll
    for (int t = 0; t < T8; ++t) {
      s0 = mfma8_step(t, kf[t], qf8[t], s0, sw0, qsw);
      kf[t] = load_k8(ks, 1, t);
#pragma unroll
      for (int u = 0; u < PK; ++u) issue_one<false>(nx, t * PK + u);
      LF_FENCE;
    }
    mfma_only_end();
    if (count < 32) mask_half(s0, 0, count);
    LF_FENCE;
    float mc = m_run * c2;
#pragma unroll
    for (int r = 0; r < 16; ++r) s1[r] = 0.0f;
    softmax_begin();
#pragma unroll
    for (int t = 0; t < T8; ++t) {
      s1 = mfma8_step(t, kf[t], qf8[t], s1, sw1, qsw);
      LF_FENCE;
#pragma unroll
      for (int u = 0; u < 16 / T8; ++u) {
        const int r = t * (16 / T8) + u;
        s0[r] = pin(__builtin_amdgcn_exp2f(fmaf(s0[r], c2, -mc)));
      }
#pragma unroll
      for (int u = 0; u < PV; ++u) issue_one<true>(nx, t * PV + u);
      LF_FENCE;
    }
    softmax_end();
    load_v(vs, 0, va);
    bf16x8 b0, b1;
    to_bf16(s0, b0, b1);
    float ps0 = psum(s0);
    if (__builtin_amdgcn_ballot_w64(!(ps0 <= kFastLimit)) != 0) {
      exact_half_q8(ks, 0, count, s0);
      to_bf16(s0, b0, b1);
      ps0 = psum(s0);
    }
    l_run += ps0;
    if (count < BN) mask_half(s1, 1, count);
    LF_FENCE;
    mc = m_run * c2;
    softmax_begin();
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int ps = j / DB, db = j % DB;
      o[db] = M::mfma(va[db], ps == 0 ? b0 : b1, o[db]);
      va[db] = load_v1(vs, ps + 1, db);
      LF_FENCE;
#pragma unroll
      for (int u = 0; u < 16 / (2 * DB); ++u) {
        const int r = j * (16 / (2 * DB)) + u;
        s1[r] = pin(__builtin_amdgcn_exp2f(fmaf(s1[r], c2, -mc)));
      }
      LF_FENCE;
    }
    softmax_end();
    to_bf16(s1, b0, b1);
    float ps1 = psum(s1);
    if (__builtin_amdgcn_ballot_w64(!(ps1 <= kFastLimit)) != 0) {
      exact_half_q8(ks, 1, count, s1);
      to_bf16(s1, b0, b1);
      ps1 = psum(s1);
    }
    l_run += ps1;
    LF_FENCE;
    mfma_only_begin();
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int ps = 2 + j / DB, db = j % DB;
      o[db] = M::mfma(va[db], ps == 2 ? b0 : b1, o[db]);
      if (ps == 2) va[db] = load_v1(vs, 3, db);
      LF_FENCE;
    }
    mfma_only_end();
#undef LF_FENCE
  }

  __device__ __forceinline__ void compute(const char* ks, const char* vs, int count, const Next& nx) {
    if constexpr (Q8) {
      compute_q8(ks, vs, count, nx);
    } else if constexpr (ES == 2) {
      compute_bf16(ks, vs, count, nx);
    } else {
      issue(nx);
      compute_f32(ks, vs, count);
    }
  }

  // ---- fp32 tile math (small, correctness-oriented shapes) ----------------
  // One tile on the stage (ks, vs): S^T, online softmax, O^T += V^T P^T.
  __device__ __forceinline__ void compute_f32(const char* ks, const char* vs, int count) {
    f32x16 s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const char* krow = ks + (kh * 32 + l32) * RSK + h * 4;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kh][r] = 0.0f;
#pragma unroll
      for (int t = 0; t < QSTEPS; ++t) s[kh] = M::mfma(*reinterpret_cast<const frag*>(krow + t * 8), qf[t], s[kh]);
    }
    if (count < BN) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) mask_half(s[kh], kh, count);
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kh][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    l_run *= alpha;
    m_run = m_new;
    rescale_o(alpha);
    const float mc = m_run * c2;
    float psum = 0.0f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kh][r], c2, -mc));
        s[kh][r] = p;
        psum += p;
      }
    l_run += psum;
#pragma unroll
    for (int ps = 0; ps < BN / 2; ++ps) {
      const int kh = ps >> 4, r = ps & 15;
      const char* vrow = vs + (kh * 32 + acc_row(r, h)) * RSV + l32 * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = M::mfma(*reinterpret_cast<const frag*>(vrow + db * 128), s[kh][r], o[db]);
    }
  }
};

// SS = false: a workgroup owns 4/WPQ query blocks (128 rows) and
// double-buffers K/V tiles (one barrier per tile). SS = true (bf16): a
// workgroup owns one query block, holds one K and one V tile (34 KB of LDS
// with its walk table at d = 128, so four workgroups share a CU) and alternates them around two
// barriers per tile: V of tile t streams in while tile t's scores are formed,
// K of tile t+1 while its PV products run.
// Q8 (bf16 values, D = 128): q and k_cache are not read; the scores come
// from the MX-FP8 codes and scales in f8.
struct Fp8Operands {
  const uint8_t* q;   // [B,H,Lq,D] E4M3 codes
  const uint8_t* qs;  // [B,H,Lq,D/32] E8M0 scales
  const uint8_t* k;   // [B,H,S,T,D]
  const uint8_t* ks;  // [B,H,S,T,D/32]
};

template <typename T, int D, int WPQ, bool SS, bool Q8 = false>
__global__ __launch_bounds__((64 * WPQ * (SS ? 1 : 4 / WPQ)), (WAVES_PER_SIMD<T, WPQ>)) void attn_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ nsel, int max_sel, float scale, const KGeom g, T* __restrict__ out,
    float* __restrict__ lse, const Fp8Operands f8) {
  static_assert(!Q8 || (D == 128 && sizeof(T) == 2), "FP8 scores: bf16 values, D = 128");
  using W = Walk<T, D, WPQ, SS ? 1 : 4 / WPQ, Q8>;
  constexpr int QPW = W::QPW, ES = W::ES, QSTEPS = W::QSTEPS, DB = W::DB;

  // Two named stage buffers (not one indexed array): the loop below is
  // unrolled by two so every LDS read names its buffer at compile time, which
  // lets the compiler see that reading one stage never waits on the DMA that
  // is filling the other.
  __shared__ __attribute__((aligned(1024))) char k0[W::TILE_ALLOC_K];
  __shared__ __attribute__((aligned(1024))) char v0[W::TILE_BYTES_V];
  // History tiles of the walk, one entry each (see below); a block of more
  // than BN keys is two tiles.
  constexpr int WALK_CAP = QPW * LF_MAX_SEL * (WPQ > 2 ? 2 : 1);
  __shared__ uint32_t walk[WALK_CAP];

  W w(g);
  w.kc = kc;
  w.vc = vc;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.h = w.lane >> 5;
  w.l32 = w.lane & 31;

  // XCD-aware remap of the workgroup id to a work item (bh, query-block group).
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int groups = (g.nqb + QPW - 1) / QPW;
  w.bh = item / groups;
  w.qb0 = (item - (int)w.bh * groups) * QPW;

  // This wavefront's query block and rows.
  w.lq = w.wv / WPQ;
  const int rg = w.wv - w.lq * WPQ;
  const int qb = w.qb0 + w.lq;
  const int fc = qb / g.nb, jq = qb - fc * g.nb;
  w.nrows = qb < g.nqb ? min(g.b, g.T - jq * g.b) : 0;
  w.qr = rg * 32 + w.l32;
  w.wave_active = rg * 32 < w.nrows;
  w.qrow0 = (int64_t)fc * g.T + (int64_t)jq * g.b;
  if constexpr (Q8) {
    w.kc8 = f8.k;
    w.ksc8 = f8.ks;
    const bool ok = w.qr < w.nrows;
    const int64_t row = w.bh * g.Lq + w.qrow0 + (ok ? w.qr : 0);
    const uint8_t* qp = f8.q + row * D;
#pragma unroll
    for (int t = 0; t < D / 64; ++t) {
      const uint4 a = ok ? *reinterpret_cast<const uint4*>(qp + 64 * t + 16 * w.h) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 b = ok ? *reinterpret_cast<const uint4*>(qp + 64 * t + 32 + 16 * w.h) : make_uint4(0u, 0u, 0u, 0u);
      w.qf8[t] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
    w.qsw = (ok ? *reinterpret_cast<const uint32_t*>(f8.qs + row * (D / 32)) : 0u) >> (8 * w.h);
  } else {
    const bool ok = w.qr < w.nrows;
    const T* qp = q + (w.bh * g.Lq + w.qrow0 + (ok ? w.qr : 0)) * D;
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) {
      if constexpr (ES == 2) {
        const uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + s * 16 + 8 * w.h) : make_uint4(0u, 0u, 0u, 0u);
        w.qf[s] = __builtin_bit_cast(bf16x8, v);
      } else {
        w.qf[s] = ok ? qp[s * 2 + w.h] : 0.0f;
      }
    }
  }

  // Producer state.
  w.tpf = (g.T + BN - 1) / BN;
  w.n_cur = g.Fc * w.tpf;
  w.frame_elems = (int64_t)g.T * D;
  w.bh_base = w.bh * g.S * w.frame_elems;
  w.all_mask = (1 << min(QPW, g.nqb - w.qb0)) - 1;
  w.t_next = 0;
  w.cf = 0;
  w.ct = 0;
  w.cur_base = w.bh_base + (int64_t)g.slot[g.Fh] * w.frame_elems;
  w.walk = walk;

  // History walk table. Each query block's selected ids are first compacted
  // (ids outside [0, Fh*nb) dropped) into the still unused first K buffer,
  // one wavefront per list. Then every wavefront computes the same table
  // positions (wavefront 0 writes): the blocks of list 0, then those of
  // list 1 that list 0 lacks, and so on, each with the mask of all query
  // blocks that selected it, so a shared block is loaded once. Membership is
  // a binary search, valid when every list ascends; if one does not, no
  // block is shared (each list walks its own blocks with only its own bit),
  // which is still exact. Entry (32 bits): cache slot (bits 0-13, slots are
  // below LF_MAX_CACHE_SLOTS), block index in its frame (14-22), second
  // BN-key tile of a longer block (23), query-block mask (24-27).
  {
    int32_t* stage = reinterpret_cast<int32_t*>(k0);
    int32_t* stage_len = stage + QPW * LF_MAX_SEL;
    static_assert((QPW * LF_MAX_SEL + QPW) * 4 <= W::TILE_BYTES_K, "lists must fit in one K buffer");
    const int n_hist_blocks = g.Fh * g.nb;
    const uint64_t lt = (1ull << w.lane) - 1;  // lanes below this one
    if (w.wv < QPW) {
      const int i = w.wv, qbi = w.qb0 + i;
      const int64_t row = w.bh * g.nqb + qbi;
      const int len = (qbi < g.nqb && max_sel > 0) ? __builtin_amdgcn_readfirstlane(min(max(nsel[row], 0), max_sel)) : 0;
      int n = 0;
      for (int j0 = 0; j0 < len; j0 += 64) {
        const int j = j0 + w.lane;
        const int x = j < len ? sel[row * max_sel + j] : -1;
        const bool valid = x >= 0 && x < n_hist_blocks;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(valid);
        if (valid) stage[i * LF_MAX_SEL + n + __builtin_popcountll(bal & lt)] = x;
        n += __builtin_popcountll(bal);
      }
      if (w.lane == 0) stage_len[i] = n;
    }
    __syncthreads();
    int clen[QPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) clen[i] = __builtin_amdgcn_readfirstlane(stage_len[i]);
    bool sorted = true;
#pragma unroll
    for (int i = 0; i < QPW; ++i)
      for (int k0s = 0; k0s < clen[i]; k0s += 64) {
        const int k = k0s + w.lane;
        const bool bad = k + 1 < clen[i] && stage[i * LF_MAX_SEL + k] >= stage[i * LF_MAX_SEL + k + 1];
        sorted = sorted && __builtin_amdgcn_ballot_w64(bad) == 0;
      }
    int n_hist_tiles = 0;
#pragma unroll
    for (int i = 0; i < QPW; ++i)
      for (int k0s = 0; k0s < clen[i]; k0s += 64) {
        const int k = k0s + w.lane;
        const bool valid = k < clen[i];
        const int x = valid ? stage[i * LF_MAX_SEL + k] : 0;
        int mask = 1 << i;
        bool owned = valid;
        if (sorted && QPW > 1) {
#pragma unroll
          for (int i2 = 0; i2 < QPW; ++i2) {
            if (i2 == i) continue;
            const int32_t* l2 = stage + i2 * LF_MAX_SEL;
            int lo = 0, hi = clen[i2];
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if (l2[mid] < x) lo = mid + 1; else hi = mid;
            }
            if (lo < clen[i2] && l2[lo] == x) {
              mask |= 1 << i2;
              if (i2 < i) owned = false;
            }
          }
        }
        const int f = x / g.nb, j = x - f * g.nb;
        const bool two = min(g.b, g.T - j * g.b) > BN;
        const uint64_t b1 = __builtin_amdgcn_ballot_w64(owned), b2 = __builtin_amdgcn_ballot_w64(owned && two);
        const int pos = n_hist_tiles + __builtin_popcountll(b1 & lt) + __builtin_popcountll(b2 & lt);
        if (w.wv == 0 && owned) {
          const uint32_t e = (uint32_t)g.slot[f] | ((uint32_t)j << 14) | ((uint32_t)mask << 24);
          walk[pos] = e;
          if (two) walk[pos + 1] = e | (1u << 23);
        }
        n_hist_tiles += __builtin_popcountll(b1) + __builtin_popcountll(b2);
      }
    w.n_tiles = w.n_cur + n_hist_tiles;
    __syncthreads();  // the table is written and the first K buffer is free again
  }
  w.init_loads();

#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) w.o[db][r] = 0.0f;
  w.m_run = -INFINITY;
  w.l_run = 0.0f;
  w.c2 = scale * kLog2e;

  if constexpr (SS) {
    // Single-stage walk. K of the first tile is loaded up front; then per
    // tile: phase 1 on K (this tile's V DMA in flight), barrier, phase 2 on V
    // (next tile's K DMA in flight), barrier. At the end of the walk the
    // last tile's K is re-read into the buffer nobody reads any more.
    // Every wavefront runs both phases: each tile belongs to the one query
    // block, and a wavefront past the block's last row holds zero query
    // fragments (finite scores, discarded) and stores nothing. Skipping the
    // math there would branch around O and cost register copies of O on
    // every tile.
    int64_t c_off = 0;
    int c_cnt = 0, c_msk = 0;
    w.produce(c_off, c_cnt, c_msk);  // the current chunk always has a tile
    w.template issue_all<false>(w.next_tile(k0, v0, c_off, c_cnt));
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (;;) {
      const typename W::Next nv = w.next_tile(k0, v0, c_off, c_cnt);
      f32x16 s1;
      bf16x8 b0, b1;
      if constexpr (Q8)
        w.ss_phase1_q8(k0, c_cnt, nv, s1, b0, b1);
      else
        w.ss_phase1(k0, c_cnt, nv, s1, b0, b1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this tile's V has landed (own share)
      __syncthreads();                       // ... everyone's, and nobody reads K any more
      int64_t n_off = c_off;
      int n_cnt = c_cnt, n_msk = c_msk;
      const bool more = w.produce(n_off, n_cnt, n_msk);
      const typename W::Next nk = w.next_tile(k0, v0, n_off, n_cnt);
      w.ss_phase2(v0, nk, s1, b0, b1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // next tile's K has landed (own share)
      __syncthreads();                       // ... everyone's, and nobody reads V any more
      if (!more) break;
      c_off = n_off;
      c_cnt = n_cnt;
      c_msk = n_msk;
    }
  } else {
  __shared__ __attribute__((aligned(1024))) char k1[W::TILE_ALLOC_K];
  __shared__ __attribute__((aligned(1024))) char v1[W::TILE_BYTES_V];
  // Double-buffered walk, unrolled by two so each half names its buffers.
  // A wavefront computes a tile only if its query block selected it; with a
  // single query block per workgroup that holds for every tile (see the
  // single-stage walk for the rows past the block's end).
  int64_t noff = 0;
  int ncount = 0, nmask = 0;
  bool have = w.produce(noff, ncount, nmask);
  if (have) w.issue(w.next_tile(k0, v0, noff, ncount));
  while (have) {
    {
      const int count = ncount, mask = nmask;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wavefront's share of the tile has landed
      __syncthreads();                       // ... everyone's, and the other buffer is free
      have = w.produce(noff, ncount, nmask);
      const typename W::Next nx = w.next_tile(k1, v1, noff, ncount);
      if (W::QPW == 1 || (w.wave_active && ((mask >> w.lq) & 1)))
        w.compute(k0, v0, count, nx);
      else
        w.issue(nx);
    }
    if (!have) break;
    {
      const int count = ncount, mask = nmask;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      have = w.produce(noff, ncount, nmask);
      const typename W::Next nx = w.next_tile(k0, v0, noff, ncount);
      if (W::QPW == 1 || (w.wave_active && ((mask >> w.lq) & 1)))
        w.compute(k1, v1, count, nx);
      else
        w.issue(nx);
    }
  }

  }

  // No load may still be writing LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (!w.wave_active || w.qr >= w.nrows) return;
  const float l_tot = w.l_run + __shfl_xor(w.l_run, 32);
  const float inv = 1.0f / l_tot;
  T* orow = out + (w.bh * g.Lq + w.qrow0 + w.qr) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int col = db * 32 + 8 * a4 + 4 * w.h;
      if constexpr (ES == 2) {
        bf16x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (__bf16)(w.o[db][a4 * 4 + c] * inv);
        *reinterpret_cast<bf16x4*>(orow + col) = v;
      } else {
        *reinterpret_cast<float4*>(orow + col) = make_float4(w.o[db][a4 * 4] * inv, w.o[db][a4 * 4 + 1] * inv,
                                                             w.o[db][a4 * 4 + 2] * inv, w.o[db][a4 * 4 + 3] * inv);
      }
    }
  if (lse != nullptr && w.h == 0) lse[w.bh * g.Lq + w.qrow0 + w.qr] = w.m_run * scale + logf(l_tot);
}

template <typename T, int D, int WPQ, bool SS = false>
hipError_t launch_typed(const KGeom& g, const void* q, const void* k, const void* v, const int32_t* sel,
                        const int32_t* nsel, int max_sel, float scale, void* out, float* lse, hipStream_t stream) {
  constexpr int QPW = SS ? 1 : 4 / WPQ;
  const unsigned grid = (unsigned)((int64_t)g.B * g.H * ((g.nqb + QPW - 1) / QPW));
  hipLaunchKernelGGL((attn_kernel<T, D, WPQ, SS>), dim3(grid), dim3(64 * WPQ * QPW), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), sel, nsel, max_sel,
                     scale, g, static_cast<T*>(out), lse, Fp8Operands{});
  return hipGetLastError();
}

template <int WPQ, bool SS>
hipError_t launch_fp8_typed(const KGeom& g, const Fp8Operands& f8, const void* v, const int32_t* sel,
                            const int32_t* nsel, int max_sel, float scale, void* out, float* lse, hipStream_t stream) {
  constexpr int QPW = SS ? 1 : 4 / WPQ;
  const unsigned grid = (unsigned)((int64_t)g.B * g.H * ((g.nqb + QPW - 1) / QPW));
  hipLaunchKernelGGL((attn_kernel<__bf16, 128, WPQ, SS, true>), dim3(grid), dim3(64 * WPQ * QPW), 0, stream, nullptr,
                     nullptr, static_cast<const __bf16*>(v), sel, nsel, max_sel, scale, g, static_cast<__bf16*>(out),
                     lse, f8);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const KGeom& g, const void* q, const void* k, const void* v, const int32_t* sel,
                    const int32_t* nsel, int max_sel, float scale, void* out, float* lse, hipStream_t stream) {
  switch ((g.b + 31) / 32) {
    case 1: return launch_typed<T, D, 1>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
    case 2:
      if constexpr (sizeof(T) == 2) {
        if (kSingleStage) return launch_typed<T, D, 2, true>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
      }
      return launch_typed<T, D, 2>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
    case 3: return launch_typed<T, D, 3>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
    default: return launch_typed<T, D, 4>(g, q, k, v, sel, nsel, max_sel, scale, out, lse, stream);
  }
}

}  // namespace

hipError_t launch_attention_fp8(const KGeom& g, const uint8_t* q8, const uint8_t* q_scale, const uint8_t* k8_cache,
                                const uint8_t* k_scale, const void* v_cache, const int32_t* sel_blocks,
                                const int32_t* n_sel, int32_t max_sel, float scale, void* out, float* lse,
                                hipStream_t stream) {
  if (g.D != 128) return hipErrorInvalidValue;
  const Fp8Operands f8{q8, q_scale, k8_cache, k_scale};
  switch ((g.b + 31) / 32) {
    case 1: return launch_fp8_typed<1, false>(g, f8, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
    case 2: return launch_fp8_typed<2, true>(g, f8, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
    case 3: return launch_fp8_typed<3, false>(g, f8, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
    default: return launch_fp8_typed<4, false>(g, f8, v_cache, sel_blocks, n_sel, max_sel, scale, out, lse, stream);
  }
}

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
