// C-ABI entry points of liblf.so: argument validation, launch, and the two
// host-only pieces of the method (chunk-aware budget, cache slot table).
// Declarations and contracts: include/lf.h.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "lf_internal.h"

namespace {

thread_local char g_err[256] = "";

lf_status fail(lf_status s, const char* msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return s;
}

lf_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return LF_OK;
  snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
  return LF_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the geometry and (when given) the host slot table; fills kg.
lf_status make_geom(const lf_geom* g, const int32_t* frame_slot, lf::KGeom* kg) {
  if (g == nullptr) return fail(LF_ERR_NULL, "geometry is NULL");
  if (g->dtype != LF_F32 && g->dtype != LF_BF16) return fail(LF_ERR_DTYPE, "dtype must be LF_F32 or LF_BF16");
  if (g->batch < 1 || g->heads < 1) return fail(LF_ERR_GEOM, "batch and heads must be >= 1");
  if (g->head_dim != 64 && g->head_dim != 128) return fail(LF_ERR_GEOM, "head_dim must be 64 or 128");
  if (g->tokens_per_frame < 1) return fail(LF_ERR_GEOM, "tokens_per_frame must be >= 1");
  if (g->block < 1 || g->block > LF_MAX_BLOCK) return fail(LF_ERR_GEOM, "block must be in [1, LF_MAX_BLOCK]");
  if (g->chunk_frames < 1 || g->hist_frames < 0) return fail(LF_ERR_GEOM, "chunk_frames >= 1, hist_frames >= 0");
  if (g->hist_frames + g->chunk_frames > LF_MAX_FRAMES) return fail(LF_ERR_GEOM, "too many frames");
  if (g->n_sink < 0 || g->n_sink > g->hist_frames) return fail(LF_ERR_GEOM, "n_sink must be in [0, hist_frames]");
  if (g->cache_slots < g->hist_frames + g->chunk_frames) return fail(LF_ERR_GEOM, "cache_slots < frames named");
  if (g->cache_slots > LF_MAX_CACHE_SLOTS) return fail(LF_ERR_GEOM, "cache_slots > LF_MAX_CACHE_SLOTS");
  const int64_t nb = (g->tokens_per_frame + (int64_t)g->block - 1) / g->block;
  if (nb > LF_MAX_BLOCKS_PER_FRAME) return fail(LF_ERR_GEOM, "too many blocks per frame");
  const int64_t lq = (int64_t)g->chunk_frames * g->tokens_per_frame;
  const int64_t bh = (int64_t)g->batch * g->heads;
  if (lq > INT32_MAX / 2 || bh * g->chunk_frames * nb > INT32_MAX / 8 ||
      bh * g->cache_slots * (int64_t)g->tokens_per_frame >= ((int64_t)1 << 32))
    return fail(LF_ERR_GEOM, "problem too large for one call");
  kg->B = g->batch;
  kg->H = g->heads;
  kg->D = g->head_dim;
  kg->T = g->tokens_per_frame;
  kg->b = g->block;
  kg->Fc = g->chunk_frames;
  kg->Fh = g->hist_frames;
  kg->ns = g->n_sink;
  kg->S = g->cache_slots;
  kg->nb = (int32_t)nb;
  kg->nqb = (int32_t)(g->chunk_frames * nb);
  kg->Lq = (int32_t)lq;
  memset(kg->slot, 0, sizeof(kg->slot));
  if (frame_slot != nullptr) {
    const int n = g->hist_frames + g->chunk_frames;
    for (int i = 0; i < n; ++i) {
      const int s = frame_slot[i];
      if (s < 0 || s >= g->cache_slots) return fail(LF_ERR_SLOT, "frame_slot entry outside [0, cache_slots)");
      for (int j = 0; j < i; ++j)
        if (frame_slot[j] == s) return fail(LF_ERR_SLOT, "frame_slot names a slot twice");
      kg->slot[i] = s;
    }
  }
  return LF_OK;
}

int64_t max_sel_of(const lf::KGeom& g, int32_t k_frames, int32_t k_blocks) {
  const int kf = k_frames < g.Fh - g.ns ? k_frames : g.Fh - g.ns;
  const int kb = k_blocks < g.nb ? k_blocks : g.nb;
  return (int64_t)g.ns * g.nb + (int64_t)(kf > 0 ? kf : 0) * (kb > 0 ? kb : 0);
}

}  // namespace

extern "C" {

// Hash of the sources this library was built from (set by the build).
#ifndef LF_BUILD_ID
#define LF_BUILD_ID "unversioned"
#endif
const char* lf_build_id(void) { return LF_BUILD_ID; }

const char* lf_status_str(lf_status s) {
  switch (s) {
    case LF_OK: return "LF_OK";
    case LF_ERR_NULL: return "LF_ERR_NULL";
    case LF_ERR_GEOM: return "LF_ERR_GEOM";
    case LF_ERR_DTYPE: return "LF_ERR_DTYPE";
    case LF_ERR_K: return "LF_ERR_K";
    case LF_ERR_ALIGN: return "LF_ERR_ALIGN";
    case LF_ERR_HIP: return "LF_ERR_HIP";
    case LF_ERR_SLOT: return "LF_ERR_SLOT";
    case LF_ERR_ARG: return "LF_ERR_ARG";
  }
  return "LF_UNKNOWN_STATUS";
}

const char* lf_last_error(void) { return g_err; }

lf_status lf_compress(const lf_geom* g, const void* q, const void* k_cache, const int32_t* frame_slot, float* q_blk,
                      float* k_blk, float* k_frm, lf_stream stream) {
  if (frame_slot == nullptr) return fail(LF_ERR_NULL, "frame_slot is NULL");
  lf::KGeom kg;
  lf_status st = make_geom(g, frame_slot, &kg);
  if (st != LF_OK) return st;
  if (q == nullptr || q_blk == nullptr) return fail(LF_ERR_NULL, "q / q_blk is NULL");
  if (kg.Fh > 0 && (k_cache == nullptr || k_blk == nullptr || k_frm == nullptr))
    return fail(LF_ERR_NULL, "k_cache / k_blk / k_frm is NULL");
  if (!aligned16(q) || !aligned16(q_blk) ||
      (kg.Fh > 0 && (!aligned16(k_cache) || !aligned16(k_blk) || !aligned16(k_frm))))
    return fail(LF_ERR_ALIGN, "pointers must be 16-byte aligned");
  return hip_status(lf::launch_compress(kg, g->dtype, q, k_cache, q_blk, k_blk, k_frm, static_cast<hipStream_t>(stream)),
                    "lf_compress launch");
}

int32_t lf_max_sel(const lf_geom* g, int32_t k_frames, int32_t k_blocks) {
  lf::KGeom kg;
  if (make_geom(g, nullptr, &kg) != LF_OK || k_frames < 0 || k_blocks < 0) return -1;
  return (int32_t)max_sel_of(kg, k_frames, k_blocks);
}

lf_status lf_pool_keys(const lf_geom* g, const void* k_cache, const int32_t* slots, int32_t n_slots, float* kp_blk,
                       float* kp_frm, lf_stream stream) {
  lf::KGeom kg;
  lf_status st = make_geom(g, nullptr, &kg);
  if (st != LF_OK) return st;
  if (n_slots < 0 || n_slots > LF_MAX_FRAMES) return fail(LF_ERR_ARG, "n_slots must be in [0, LF_MAX_FRAMES]");
  if (n_slots == 0) return LF_OK;
  if (slots == nullptr || k_cache == nullptr || kp_blk == nullptr || kp_frm == nullptr)
    return fail(LF_ERR_NULL, "slots / k_cache / kp_blk / kp_frm is NULL");
  for (int i = 0; i < n_slots; ++i) {
    if (slots[i] < 0 || slots[i] >= kg.S) return fail(LF_ERR_SLOT, "slot outside [0, cache_slots)");
    for (int j = 0; j < i; ++j)
      if (slots[j] == slots[i]) return fail(LF_ERR_SLOT, "slot named twice");
    kg.slot[i] = slots[i];
  }
  kg.Fh = n_slots;
  if (!aligned16(k_cache) || !aligned16(kp_blk) || !aligned16(kp_frm))
    return fail(LF_ERR_ALIGN, "pointers must be 16-byte aligned");
  return hip_status(lf::launch_pool_slots(kg, g->dtype, k_cache, kp_blk, kp_frm, static_cast<hipStream_t>(stream)),
                    "lf_pool_keys launch");
}

lf_status lf_select_fused(const lf_geom* g, const void* q, const float* kp_blk, const float* kp_frm,
                          const int32_t* frame_slot, int32_t k_frames, int32_t k_blocks, int32_t* sel_frames,
                          int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, float* q_blk, lf_stream stream) {
  if (frame_slot == nullptr) return fail(LF_ERR_NULL, "frame_slot is NULL");
  lf::KGeom kg;
  lf_status st = make_geom(g, frame_slot, &kg);
  if (st != LF_OK) return st;
  if (k_frames < 0 || k_blocks < 0) return fail(LF_ERR_K, "k_frames and k_blocks must be >= 0");
  if (max_sel < max_sel_of(kg, k_frames, k_blocks)) return fail(LF_ERR_K, "max_sel smaller than lf_max_sel()");
  if (q == nullptr || n_sel == nullptr || (max_sel > 0 && sel_blocks == nullptr))
    return fail(LF_ERR_NULL, "q / sel_blocks / n_sel is NULL");
  if (kg.Fh > 0 && (kp_blk == nullptr || kp_frm == nullptr)) return fail(LF_ERR_NULL, "kp_blk / kp_frm is NULL");
  if (!aligned16(q) || !aligned16(q_blk) || (kg.Fh > 0 && (!aligned16(kp_blk) || !aligned16(kp_frm))))
    return fail(LF_ERR_ALIGN, "pointers must be 16-byte aligned");
  const int kf = k_frames < kg.Fh - kg.ns ? k_frames : kg.Fh - kg.ns;
  const int kb = k_blocks < kg.nb ? k_blocks : kg.nb;
  return hip_status(lf::launch_select_fused(kg, g->dtype, q, kp_blk, kp_frm, kf, kb, k_frames, sel_frames, sel_blocks,
                                            n_sel, max_sel, q_blk, static_cast<hipStream_t>(stream)),
                    "lf_select_fused launch");
}

int32_t lf_max_sel_1d(const lf_geom* g, int32_t k_total) {
  lf::KGeom kg;
  if (make_geom(g, nullptr, &kg) != LF_OK || k_total < 0) return -1;
  const int64_t ncand = (int64_t)(kg.Fh - kg.ns) * kg.nb;
  return (int32_t)((int64_t)kg.ns * kg.nb + (k_total < ncand ? k_total : ncand));
}

lf_status lf_select_blocks(const lf_geom* g, const float* q_blk, const float* k_blk, int32_t k_total,
                           int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, lf_stream stream) {
  lf::KGeom kg;
  lf_status st = make_geom(g, nullptr, &kg);
  if (st != LF_OK) return st;
  if (k_total < 0) return fail(LF_ERR_K, "k_total must be >= 0");
  const int64_t ncand = (int64_t)(kg.Fh - kg.ns) * kg.nb;
  if (ncand > LF_MAX_CANDIDATES_1D) return fail(LF_ERR_GEOM, "more than LF_MAX_CANDIDATES_1D candidate blocks");
  const int k = (int)(k_total < ncand ? k_total : ncand);
  if (max_sel < (int64_t)kg.ns * kg.nb + k) return fail(LF_ERR_K, "max_sel smaller than lf_max_sel_1d()");
  if (q_blk == nullptr || n_sel == nullptr || (max_sel > 0 && sel_blocks == nullptr))
    return fail(LF_ERR_NULL, "q_blk / sel_blocks / n_sel is NULL");
  if (kg.Fh > 0 && k_blk == nullptr) return fail(LF_ERR_NULL, "k_blk is NULL");
  if (!aligned16(q_blk) || (kg.Fh > 0 && !aligned16(k_blk)))
    return fail(LF_ERR_ALIGN, "pooled tensors must be 16-byte aligned");
  return hip_status(lf::launch_select_blocks(kg, q_blk, k_blk, k, sel_blocks, n_sel, max_sel,
                                             static_cast<hipStream_t>(stream)),
                    "lf_select_blocks launch");
}

lf_status lf_select(const lf_geom* g, const float* q_blk, const float* k_blk, const float* k_frm, int32_t k_frames,
                    int32_t k_blocks, int32_t* sel_frames, int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel,
                    lf_stream stream) {
  lf::KGeom kg;
  lf_status st = make_geom(g, nullptr, &kg);
  if (st != LF_OK) return st;
  if (k_frames < 0 || k_blocks < 0) return fail(LF_ERR_K, "k_frames and k_blocks must be >= 0");
  const int64_t need = max_sel_of(kg, k_frames, k_blocks);
  if (max_sel < need) return fail(LF_ERR_K, "max_sel smaller than lf_max_sel()");
  if (q_blk == nullptr || n_sel == nullptr || (max_sel > 0 && sel_blocks == nullptr))
    return fail(LF_ERR_NULL, "q_blk / sel_blocks / n_sel is NULL");
  if (kg.Fh > 0 && (k_blk == nullptr || k_frm == nullptr)) return fail(LF_ERR_NULL, "k_blk / k_frm is NULL");
  if (!aligned16(q_blk) || (kg.Fh > 0 && (!aligned16(k_blk) || !aligned16(k_frm))))
    return fail(LF_ERR_ALIGN, "pooled tensors must be 16-byte aligned");
  const int kf = k_frames < kg.Fh - kg.ns ? k_frames : kg.Fh - kg.ns;
  const int kb = k_blocks < kg.nb ? k_blocks : kg.nb;
  return hip_status(lf::launch_select(kg, q_blk, k_blk, k_frm, kf, kb, k_frames, sel_frames, sel_blocks, n_sel,
                                      max_sel, static_cast<hipStream_t>(stream)),
                    "lf_select launch");
}

lf_status lf_check_selection(const lf_geom* g, const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel,
                             int32_t* result, lf_stream stream) {
  lf::KGeom kg;
  lf_status st = make_geom(g, nullptr, &kg);
  if (st != LF_OK) return st;
  if (max_sel < 0 || max_sel > LF_MAX_SEL) return fail(LF_ERR_K, "max_sel must be in [0, LF_MAX_SEL]");
  if (n_sel == nullptr || result == nullptr || (max_sel > 0 && sel_blocks == nullptr))
    return fail(LF_ERR_NULL, "sel_blocks / n_sel / result is NULL");
  return hip_status(lf::launch_check_selection(kg, sel_blocks, n_sel, max_sel, result, static_cast<hipStream_t>(stream)),
                    "lf_check_selection launch");
}

lf_status lf_block_sparse_attn(const lf_geom* g, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* frame_slot, const int32_t* sel_blocks, const int32_t* n_sel,
                               int32_t max_sel, float softmax_scale, void* out, float* lse, lf_stream stream) {
  if (frame_slot == nullptr) return fail(LF_ERR_NULL, "frame_slot is NULL");
  lf::KGeom kg;
  lf_status st = make_geom(g, frame_slot, &kg);
  if (st != LF_OK) return st;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr)
    return fail(LF_ERR_NULL, "q / k_cache / v_cache / out is NULL");
  if (max_sel < 0 || max_sel > LF_MAX_SEL) return fail(LF_ERR_K, "max_sel must be in [0, LF_MAX_SEL]");
  if (max_sel > 0 && (sel_blocks == nullptr || n_sel == nullptr))
    return fail(LF_ERR_NULL, "sel_blocks / n_sel is NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(LF_ERR_ALIGN, "q / caches / out must be 16-byte aligned");
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return fail(LF_ERR_ARG, "softmax_scale must be > 0");
  return hip_status(lf::launch_attention(kg, g->dtype, q, k_cache, v_cache, sel_blocks, n_sel, max_sel,
                                         softmax_scale, out, lse, static_cast<hipStream_t>(stream)),
                    "lf_block_sparse_attn launch");
}

lf_status lf_block_sparse_attn_fp8(const lf_geom* g, const uint8_t* q8, const uint8_t* q_scale, const uint8_t* k8_cache,
                                   const uint8_t* k_scale, const void* v_cache, const int32_t* frame_slot,
                                   const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel,
                                   float softmax_scale, void* out, float* lse, lf_stream stream) {
  if (frame_slot == nullptr) return fail(LF_ERR_NULL, "frame_slot is NULL");
  lf::KGeom kg;
  lf_status st = make_geom(g, frame_slot, &kg);
  if (st != LF_OK) return st;
  if (g->dtype != LF_BF16) return fail(LF_ERR_DTYPE, "the FP8 variant takes bf16 values and writes bf16");
  if (g->head_dim != 128) return fail(LF_ERR_GEOM, "the FP8 variant needs head_dim 128");
  if (q8 == nullptr || q_scale == nullptr || k8_cache == nullptr || k_scale == nullptr || v_cache == nullptr ||
      out == nullptr)
    return fail(LF_ERR_NULL, "q8 / q_scale / k8_cache / k_scale / v_cache / out is NULL");
  if (max_sel < 0 || max_sel > LF_MAX_SEL) return fail(LF_ERR_K, "max_sel must be in [0, LF_MAX_SEL]");
  if (max_sel > 0 && (sel_blocks == nullptr || n_sel == nullptr))
    return fail(LF_ERR_NULL, "sel_blocks / n_sel is NULL");
  if (!aligned16(q8) || !aligned16(k8_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(q_scale) & 3u) != 0 || (reinterpret_cast<uintptr_t>(k_scale) & 3u) != 0)
    return fail(LF_ERR_ALIGN, "codes / v_cache / out must be 16-byte aligned, scales 4-byte aligned");
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return fail(LF_ERR_ARG, "softmax_scale must be > 0");
  return hip_status(lf::launch_attention_fp8(kg, q8, q_scale, k8_cache, k_scale, v_cache, sel_blocks, n_sel, max_sel,
                                             softmax_scale, out, lse, static_cast<hipStream_t>(stream)),
                    "lf_block_sparse_attn_fp8 launch");
}

lf_status lf_block_sparse_attn_bwd(const lf_geom* g, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* frame_slot, const int32_t* sel_blocks, const int32_t* n_sel,
                                   int32_t max_sel, float softmax_scale, const void* out, const float* lse,
                                   const void* dout, float* delta, float* dq, float* dk_cache, float* dv_cache,
                                   lf_stream stream) {
  if (frame_slot == nullptr) return fail(LF_ERR_NULL, "frame_slot is NULL");
  lf::KGeom kg;
  lf_status st = make_geom(g, frame_slot, &kg);
  if (st != LF_OK) return st;
  if (g->dtype != LF_BF16) return fail(LF_ERR_DTYPE, "the backward takes bf16 inputs");
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr || lse == nullptr ||
      dout == nullptr || delta == nullptr || dq == nullptr || dk_cache == nullptr || dv_cache == nullptr)
    return fail(LF_ERR_NULL, "an input or output of the backward is NULL");
  if (max_sel < 0 || max_sel > LF_MAX_SEL) return fail(LF_ERR_K, "max_sel must be in [0, LF_MAX_SEL]");
  if (max_sel > 0 && (sel_blocks == nullptr || n_sel == nullptr))
    return fail(LF_ERR_NULL, "sel_blocks / n_sel is NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk_cache) || !aligned16(dv_cache))
    return fail(LF_ERR_ALIGN, "q / caches / out / dout / gradients must be 16-byte aligned");
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return fail(LF_ERR_ARG, "softmax_scale must be > 0");
  return hip_status(lf::launch_attention_bwd(kg, q, k_cache, v_cache, sel_blocks, n_sel, max_sel, softmax_scale, out,
                                             lse, dout, delta, dq, dk_cache, dv_cache,
                                             static_cast<hipStream_t>(stream)),
                    "lf_block_sparse_attn_bwd launch");
}

lf_status lf_block_sparse_attn_bwd_noalloc(const lf_geom* g, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* frame_slot, const int32_t* sel_blocks,
                                           const int32_t* n_sel, int32_t max_sel, float softmax_scale,
                                           const void* out, const float* lse, const void* dout, float* dq,
                                           float* dk_cache, float* dv_cache, lf_stream stream) {
  if (g == nullptr) return fail(LF_ERR_NULL, "geometry is NULL");
  const int64_t rows = (int64_t)g->batch * g->heads * g->chunk_frames * g->tokens_per_frame;
  if (g->batch >= 1 && g->heads >= 1 && g->chunk_frames >= 1 && g->tokens_per_frame >= 1 &&
      rows > LF_NOALLOC_MAX_ROWS)
    return fail(LF_ERR_GEOM, "B*H*Fc*T exceeds LF_NOALLOC_MAX_ROWS (the fixed row scratch)");
  float* delta = nullptr;
  const hipError_t e = lf::noalloc_scratch(&delta);
  if (e != hipSuccess) return hip_status(e, "lf_block_sparse_attn_bwd_noalloc: device address of the row scratch");
  return lf_block_sparse_attn_bwd(g, q, k_cache, v_cache, frame_slot, sel_blocks, n_sel, max_sel, softmax_scale, out,
                                  lse, dout, delta, dq, dk_cache, dv_cache, stream);
}

lf_status lf_chunk_budget(int32_t n_chunks, const double* sigma, const double* weight, const uint8_t* dense,
                          double s_base, double s_target, const int32_t* hist_frames, const int32_t* n_sink,
                          int32_t blocks_per_frame, int32_t k_frames_min, double* sparsity_out, double* beta_out,
                          int32_t* k_frames_out, int32_t* k_blocks_out) {
  if (n_chunks < 0) return fail(LF_ERR_ARG, "n_chunks must be >= 0");
  if (n_chunks > 0 && (sigma == nullptr || dense == nullptr || hist_frames == nullptr || sparsity_out == nullptr ||
                       k_frames_out == nullptr || k_blocks_out == nullptr))
    return fail(LF_ERR_NULL, "a required array is NULL");
  if (beta_out == nullptr) return fail(LF_ERR_NULL, "beta_out is NULL");
  if (blocks_per_frame < 1 || k_frames_min < 0) return fail(LF_ERR_ARG, "blocks_per_frame >= 1, k_frames_min >= 0");
  double num = 0.0, den = 0.0;
  for (int i = 0; i < n_chunks; ++i) {
    const int ns = n_sink ? n_sink[i] : 0;
    if (hist_frames[i] < 0 || ns < 0 || ns > hist_frames[i]) return fail(LF_ERR_ARG, "bad hist_frames / n_sink");
    if (dense[i]) continue;
    if (!(sigma[i] > 0.0)) return fail(LF_ERR_ARG, "sigma must be > 0");
    const double w = weight ? weight[i] : 1.0;
    num += w;
    den += w / sqrt(sigma[i]);
  }
  // beta = (s_base - s_target) * sum w / sum (w / sqrt(sigma)) over the non-dense chunks.
  const double beta = den != 0.0 ? (s_base - s_target) * num / den : 0.0;
  *beta_out = beta;
  for (int i = 0; i < n_chunks; ++i) {
    const int F = hist_frames[i];
    const int ns = n_sink ? n_sink[i] : 0;
    const int cand = F - ns > 0 ? F - ns : 0;
    if (dense[i]) {
      sparsity_out[i] = 0.0;
      k_frames_out[i] = cand;
      k_blocks_out[i] = cand > 0 ? blocks_per_frame : 0;
      continue;
    }
    const double s = s_base - beta / sqrt(sigma[i]);
    sparsity_out[i] = s;
    const double budget = (1.0 - s) * F * blocks_per_frame - (double)ns * blocks_per_frame;
    if (cand == 0 || budget <= 0.0) {
      k_frames_out[i] = 0;
      k_blocks_out[i] = 0;
      continue;
    }
    int kf = (int)ceil(budget / blocks_per_frame - 1e-9);
    if (kf < k_frames_min) kf = k_frames_min;
    if (kf > cand) kf = cand;
    int kb = (int)floor(budget / kf + 0.5);
    if (kb < 1) kb = 1;
    if (kb > blocks_per_frame) kb = blocks_per_frame;
    k_frames_out[i] = kf;
    k_blocks_out[i] = kb;
  }
  return LF_OK;
}

lf_status lf_cache_frame_slots(int32_t policy, int32_t cache_slots, int32_t n_sink, int32_t chunk_frames,
                               int32_t chunk_index, int32_t* hist_frames_out, int32_t* frame_slot_out,
                               int32_t* frame_ids_out) {
  if (hist_frames_out == nullptr || frame_slot_out == nullptr) return fail(LF_ERR_NULL, "output is NULL");
  if (policy != LF_CACHE_ROLLING && policy != LF_CACHE_ANCHORED) return fail(LF_ERR_ARG, "unknown cache policy");
  const int anchors = policy == LF_CACHE_ANCHORED ? n_sink : 0;
  if (chunk_frames < 1 || chunk_index < 0 || anchors < 0 || cache_slots < chunk_frames + anchors)
    return fail(LF_ERR_ARG, "cache too small for the chunk and its anchors");
  if (cache_slots > LF_MAX_FRAMES) return fail(LF_ERR_ARG, "cache_slots > LF_MAX_FRAMES");
  const int64_t first = (int64_t)chunk_index * chunk_frames;  // first absolute frame of the chunk
  const int64_t hist = first < cache_slots - chunk_frames ? first : cache_slots - chunk_frames;
  const int kept_anchors = (int)(anchors < hist ? anchors : hist);
  const int64_t recent = hist - kept_anchors;
  int n = 0;
  auto slot_of = [&](int64_t a) -> int32_t {
    if (policy == LF_CACHE_ANCHORED)
      return (int32_t)(a < anchors ? a : anchors + (a - anchors) % (cache_slots - anchors));
    return (int32_t)(a % cache_slots);
  };
  auto emit = [&](int64_t a) {
    frame_slot_out[n] = slot_of(a);
    if (frame_ids_out) frame_ids_out[n] = (int32_t)a;
    ++n;
  };
  for (int a = 0; a < kept_anchors; ++a) emit(a);
  for (int64_t a = first - recent; a < first; ++a) emit(a);
  for (int64_t a = first; a < first + chunk_frames; ++a) emit(a);
  *hist_frames_out = (int32_t)hist;
  return LF_OK;
}

}  // extern "C"
