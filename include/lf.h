/*
 * lf.h -- C ABI of liblf.so, an MI355X (gfx950) implementation of Light
 * Forcing's hierarchical sparse attention for chunk-wise autoregressive video
 * diffusion, and of its chunk-aware sparsity budget.
 *
 * Source pages (cited by title and section):
 *   [LF-tech]  "Light Forcing: Accelerating Autoregressive Video Diffusion via
 *              Sparse Attention" (arXiv 2602.04789), technical summary:
 *              2.1 chunk-aware growth (CAG), 2.2 hierarchical sparse attention
 *              (HSA: token compression, two-stage mask selection, execution).
 *   [LF-press] press summary of the same paper, section 3 (hierarchical
 *              sparse attention), section 2 (chunk-aware growth),
 *              section 4 (experiments, ablation paragraph) and section 5
 *              (deployment: FP8 with per-token activation scales).
 *   [SF]       Self Forcing news page, rolling KV cache paragraph.
 *   [RF]       Rolling Forcing page, section 3, dual cache / attention anchor.
 *
 * Conventions shared by every entry point
 *   - Geometry: a frame is `tokens_per_frame` (T) tokens. Every frame is cut
 *     into nb = ceil(T / block) blocks; the last block of a frame holds the
 *     remaining T - (nb-1)*block tokens. Blocks never straddle frames.
 *     The current chunk has `chunk_frames` (Fc) frames, Lq = Fc*T queries and
 *     nqb = Fc*nb query blocks (query block qb = frame qb/nb, block qb%nb).
 *     The cache holds `hist_frames` (Fh) history frames; the first `n_sink`
 *     of them are attention sinks (always attended in full, never ranked).
 *   - Logical frames: 0..Fh-1 are the history (oldest first), Fh..Fh+Fc-1 the
 *     current chunk. `frame_slot` is a HOST array of Fh+Fc int32 giving the
 *     cache slot of each logical frame (distinct values in [0, cache_slots));
 *     it is read during the call and copied into the launch, so the caller
 *     may reuse it as soon as the call returns. This is how a rolling or an
 *     anchored cache rotates without moving data.
 *   - Logical block id of block j of history frame f: f*nb + j.
 *   - Layouts (all row-major, contiguous, device memory):
 *       q        [B, H, Lq, D]               dtype
 *       k_cache  [B, H, cache_slots, T, D]   dtype (v_cache the same)
 *       q_blk    [B, H, nqb, D]              float32
 *       k_blk    [B, H, Fh*nb, D]            float32
 *       k_frm    [B, H, Fh, D]               float32
 *       out      [B, H, Lq, D]               dtype;  lse [B, H, Lq] float32
 *     D (head_dim) is 64 or 128. dtype LF_BF16 or LF_F32. q, caches and out
 *     must be 16-byte aligned.
 *   - Ownership: every pointer is owned by the caller. The library never
 *     allocates, frees or synchronises; device work is enqueued on `stream`
 *     (a hipStream_t; NULL is the null stream) and the call returns at once.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued. A failing call returns a negative lf_status and enqueues
 *     nothing. LF_ERR_HIP reports a launch failure; lf_last_error() gives the
 *     detail string (per thread).
 *   - Global state: besides that per-thread string, a per-device cache of the
 *     compute-unit count (filled once, read-only after) and the per-device
 *     row scratch of lf_block_sparse_attn_bwd_noalloc (its address looked up
 *     once per device). Every entry point is safe to call from several host
 *     threads; only lf_block_sparse_attn_bwd_noalloc calls that overlap on
 *     one GPU share memory (its scratch).
 *
 * One attention call of one layer at one denoise step of a chunk:
 *   lf_cache_frame_slots(policy, S, n_sink, Fc, chunk, &Fh, frame_slot, ids);
 *   lf_chunk_budget(...)  -> k_frames, k_blocks of this chunk
 *   lf_compress(g, q, k_cache, frame_slot, q_blk, k_blk, k_frm, stream);
 *   lf_select(g, q_blk, k_blk, k_frm, k_frames, k_blocks, NULL, sel_blocks,
 *             n_sel, lf_max_sel(g, k_frames, k_blocks), stream);
 *   lf_block_sparse_attn(g, q, k_cache, v_cache, frame_slot, sel_blocks,
 *                        n_sel, max_sel, 1/sqrt(D), out, lse, stream);
 * With pooling on commit, lf_pool_keys runs once per committed frame and
 * lf_select_fused replaces lf_compress + lf_select. Buffers (q_blk ...
 * sel_blocks) can be reused across calls of the same geometry.
 */
#ifndef LF_H_
#define LF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LF_OK = 0,
  LF_ERR_NULL = -1,      /* a required pointer is NULL */
  LF_ERR_GEOM = -2,      /* geometry out of the supported range */
  LF_ERR_DTYPE = -3,     /* unknown dtype */
  LF_ERR_K = -4,         /* top-k sizes / selection capacity invalid */
  LF_ERR_ALIGN = -5,     /* a device pointer is not 16-byte aligned */
  LF_ERR_HIP = -6,       /* the HIP runtime rejected a launch */
  LF_ERR_SLOT = -7,      /* frame_slot entry out of range or repeated */
  LF_ERR_ARG = -8        /* another argument out of range */
} lf_status;

typedef enum { LF_F32 = 0, LF_BF16 = 1 } lf_dtype;

typedef enum { LF_CACHE_ROLLING = 0, LF_CACHE_ANCHORED = 1 } lf_cache_policy;

/* Most logical frames (Fh + Fc) one call may name. */
#define LF_MAX_FRAMES 256
/* Most blocks per frame (nb) the selection supports. */
#define LF_MAX_BLOCKS_PER_FRAME 512
/* Most cache slots (S) of a cache (a slot index is a 14-bit field of the
 * attention kernel's tile table). */
#define LF_MAX_CACHE_SLOTS 16384
/* Largest block (tokens) the attention kernel supports. */
#define LF_MAX_BLOCK 128
/* Most selected blocks per query block the attention kernel reads (max_sel). */
#define LF_MAX_SEL 512
/* Most candidate blocks ((Fh - n_sink) * nb) the single-level selection ranks. */
#define LF_MAX_CANDIDATES_1D 4096
/* Most query rows (B * H * Fc * T) lf_block_sparse_attn_bwd_noalloc takes:
 * its row scratch is a fixed device array of this many floats (4 MiB). */
#define LF_NOALLOC_MAX_ROWS (1 << 20)

typedef struct {
  int32_t batch;            /* B >= 1 */
  int32_t heads;            /* H >= 1 */
  int32_t head_dim;         /* D: 64 or 128 */
  int32_t tokens_per_frame; /* T >= 1 */
  int32_t block;            /* b: 1..LF_MAX_BLOCK */
  int32_t chunk_frames;     /* Fc >= 1 */
  int32_t hist_frames;      /* Fh >= 0; Fh + Fc <= LF_MAX_FRAMES */
  int32_t n_sink;           /* 0 <= n_sink <= Fh */
  int32_t cache_slots;      /* >= Fh + Fc, <= LF_MAX_CACHE_SLOTS; B*H*cache_slots*T < 2^32 */
  int32_t dtype;            /* lf_dtype */
} lf_geom;

typedef void* lf_stream; /* hipStream_t */

/* ---------------------------------------------------------------------------
 * Token compression  ([LF-tech] 2.2 "token compression"; [LF-press] 3).
 * Mean pooling: q_blk[qb] = mean of the query block's tokens; k_blk[f*nb+j] =
 * mean of block j of history frame f; k_frm[f] = mean of all T tokens of
 * history frame f. Means are accumulated in float64 and rounded once to
 * float32 (mean = (float)(sum / count)). One launch; no workspace.
 * ------------------------------------------------------------------------- */
lf_status lf_compress(const lf_geom* g, const void* q, const void* k_cache, const int32_t* frame_slot,
                      float* q_blk, float* k_blk, float* k_frm, lf_stream stream);

/* ---------------------------------------------------------------------------
 * Two-stage mask selection ([LF-tech] 2.2 "two-stage mask selection";
 * [LF-press] 3). Per (batch, head, query block):
 *   1. frame score s_f = <q_blk, k_frm[f]> in float64 for the non-sink
 *      history frames; keep the kf = min(k_frames, Fh - n_sink) largest;
 *   2. inside each kept frame, block score <q_blk, k_blk[f*nb+j]>; keep the
 *      kb = min(k_blocks, nb) largest;
 *   3. selected ids = all blocks of the sink frames + the kept (f, j),
 *      ascending. Ties in either top-k go to the lower index.
 * Outputs: sel_blocks [B,H,nqb,max_sel] int32 (ids ascending, then -1),
 * n_sel [B,H,nqb] int32, and optionally (nullable) sel_frames
 * [B,H,nqb,k_frames] int32 (kept frames ascending, then -1).
 * max_sel must be >= lf_max_sel(g, k_frames, k_blocks). k_frames, k_blocks
 * must be >= 0. The selected count never depends on Fh beyond the clamps.
 * ------------------------------------------------------------------------- */
int32_t lf_max_sel(const lf_geom* g, int32_t k_frames, int32_t k_blocks);
lf_status lf_select(const lf_geom* g, const float* q_blk, const float* k_blk, const float* k_frm,
                    int32_t k_frames, int32_t k_blocks, int32_t* sel_frames, int32_t* sel_blocks,
                    int32_t* n_sel, int32_t max_sel, lf_stream stream);

/* ---------------------------------------------------------------------------
 * Pool-on-commit and the fused per-step selection ([LF-tech] 2.2; [SF]
 * rolling cache: frames in the cache do not change until evicted, so their
 * pooled keys are computed once, when the frame is committed).
 *
 * lf_pool_keys pools the frames held in cache slots slots[0 .. n_slots-1]
 * (a HOST array of distinct slots in [0, cache_slots), n_slots <=
 * LF_MAX_FRAMES) into caches indexed by slot, with lf_compress's numerics:
 *   kp_blk [B, H, cache_slots, nb, D] float32   block means
 *   kp_frm [B, H, cache_slots, D]     float32   frame means
 * Other slots are left untouched. n_slots == 0 is a no-op.
 *
 * lf_select_fused does, per query block, lf_compress's query pooling and
 * lf_select's two-stage selection in one launch, reading the pooled keys of
 * logical frame f from slot frame_slot[f] of kp_blk / kp_frm. Its outputs
 * equal lf_compress + lf_select on the same inputs bit for bit. q_blk
 * (nullable) receives the pooled queries. Other arguments as lf_select.
 * ------------------------------------------------------------------------- */
lf_status lf_pool_keys(const lf_geom* g, const void* k_cache, const int32_t* slots, int32_t n_slots, float* kp_blk,
                       float* kp_frm, lf_stream stream);
lf_status lf_select_fused(const lf_geom* g, const void* q, const float* kp_blk, const float* kp_frm,
                          const int32_t* frame_slot, int32_t k_frames, int32_t k_blocks, int32_t* sel_frames,
                          int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, float* q_blk, lf_stream stream);

/* ---------------------------------------------------------------------------
 * Single-level ("1D") selection, the ablation baseline ([LF-press] 4,
 * ablation paragraph: block sparse attention without the frame stage). Per
 * (batch, head, query block): block score <q_blk, k_blk[id]> in float64 for
 * every block of the non-sink history frames; keep the k = min(k_total,
 * candidates) largest (ties to the lower id); selected ids = all blocks of
 * the sink frames + the kept ids, ascending. With k_total = k_frames *
 * k_blocks it spends the same block budget as lf_select. Outputs as
 * lf_select's sel_blocks / n_sel. max_sel must be >= lf_max_sel_1d(g,
 * k_total); (Fh - n_sink) * nb must be <= LF_MAX_CANDIDATES_1D. The uniform
 * allocation baseline needs no entry point: lf_chunk_budget with s_target ==
 * s_base gives beta = 0, the same sparsity for every chunk.
 * ------------------------------------------------------------------------- */
int32_t lf_max_sel_1d(const lf_geom* g, int32_t k_total);
lf_status lf_select_blocks(const lf_geom* g, const float* q_blk, const float* k_blk, int32_t k_total,
                           int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, lf_stream stream);

/* ---------------------------------------------------------------------------
 * Debug check of selection lists against the invariants lf_select's output
 * has ([LF-tech] 2.2, two-stage selection: a top-k of distinct blocks) and
 * that lf_block_sparse_attn and lf_block_sparse_attn_bwd rely on (a block
 * named twice in one list would be attended twice). For every (batch, head,
 * query block) row r = (b*H + h)*nqb + qb: 0 <= n_sel[r] <= max_sel, and the
 * first n_sel[r] ids of sel_blocks row r (row stride max_sel) are in
 * [0, Fh*nb) and strictly ascending, hence distinct. Writes, on the stream,
 * result[0] = the number of rows that break this and result[1] = the
 * smallest such row, or -1 (result: 2 int32, device memory, caller-owned).
 * One workgroup; the host is not synchronised (read result after the
 * stream). max_sel must be in [0, LF_MAX_SEL]; NULL pointers give
 * LF_ERR_NULL (sel_blocks may be NULL when max_sel is 0).
 * ------------------------------------------------------------------------- */
lf_status lf_check_selection(const lf_geom* g, const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel,
                             int32_t* result, lf_stream stream);

/* ---------------------------------------------------------------------------
 * Block-sparse attention ([LF-tech] 2.2 "execution"; [LF-press] 3).
 * Each query row of query block qb attends, with softmax(scale * q k^T) v, to
 * the tokens of the history blocks sel_blocks[qb][0 .. n_sel[qb]-1] and to
 * every token of the current chunk (logical frames Fh..Fh+Fc-1; the chunk is
 * denoised jointly, so its own tokens are all visible). Ids outside
 * [0, Fh*nb) and entries at or beyond min(n_sel, max_sel) are ignored; the
 * ids of one query block must be distinct (lf_select's are, and ascending).
 * max_sel (the row stride of sel_blocks) must be <= LF_MAX_SEL.
 * Accumulation and the online softmax run in float32 on bf16 (or f32) MFMA
 * products. out gets the normalised output in dtype; lse (nullable) the
 * natural-log normaliser per query row.
 * ------------------------------------------------------------------------- */
lf_status lf_block_sparse_attn(const lf_geom* g, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* frame_slot, const int32_t* sel_blocks, const int32_t* n_sel,
                               int32_t max_sel, float softmax_scale, void* out, float* lse, lf_stream stream);

/* ---------------------------------------------------------------------------
 * lf_block_sparse_attn with FP8 queries and keys ([LF-press] 5: the
 * deployment runs in FP8 with per-token scales for activations; here that
 * form is applied to the attention's score product). Same masks, outputs and
 * validation as lf_block_sparse_attn; q and k_cache are replaced by
 *   q8        [B, H, Lq, D]              uint8  OCP E4M3 codes (no infinities,
 *                                               0x7F/0xFF are NaN)
 *   q_scale   [B, H, Lq, D/32]           uint8  OCP MX E8M0 scales (2^(e-127),
 *                                               0xFF NaN), one per 32 channels
 *   k8_cache  [B, H, cache_slots, T, D]  uint8  E4M3 codes
 *   k_scale   [B, H, cache_slots, T, D/32] uint8 E8M0 scales
 * so channel c of a token stands for decode(code[c]) * 2^(scale[c/32]-127).
 * v_cache and out are bf16 (g->dtype must be LF_BF16, else LF_ERR_DTYPE);
 * head_dim must be 128 (else LF_ERR_GEOM). The score
 * products run on the scaled FP8 MFMA with float32 accumulation; P and V
 * enter the PV product in bf16 as in lf_block_sparse_attn. Codes and v_cache
 * and out must be 16-byte aligned, scales 4-byte aligned (LF_ERR_ALIGN).
 * ------------------------------------------------------------------------- */
lf_status lf_block_sparse_attn_fp8(const lf_geom* g, const uint8_t* q8, const uint8_t* q_scale,
                                   const uint8_t* k8_cache, const uint8_t* k_scale, const void* v_cache,
                                   const int32_t* frame_slot, const int32_t* sel_blocks, const int32_t* n_sel,
                                   int32_t max_sel, float softmax_scale, void* out, float* lse, lf_stream stream);

/* ---------------------------------------------------------------------------
 * Backward of lf_block_sparse_attn, for sparse fine-tuning ([LF-press] 4,
 * ablation paragraph: the sparse attention is fine-tuned in place; the
 * gradients below are those of the loss sum(out * dout) through the same
 * block masks, the selection itself not being differentiated).
 * Inputs: the forward's q, caches, frame_slot, sel_blocks / n_sel / max_sel
 * and softmax_scale, its outputs out [B,H,Lq,D] and lse [B,H,Lq] (float32,
 * as lf_block_sparse_attn writes them), and dout [B,H,Lq,D]. q, caches, out
 * and dout are bf16 (g->dtype must be LF_BF16, else LF_ERR_DTYPE).
 * Outputs, float32: dq [B,H,Lq,D]; dk_cache and dv_cache [B,H,S,T,D], where
 * every row of a slot that frame_slot names gets its full gradient (summed
 * over all query blocks that see it; zero if none does) and rows of other
 * slots are left untouched; delta [B,H,Lq] is scratch the call writes
 * (rowsum(dout * out)). While the call runs, the dk_cache rows of the first
 * chunk frame of (batch 0, head 0) also hold the launch order of the
 * history pass, before their gradients are written. P and dS enter the
 * MFMAs rounded to bf16, with float32 accumulation. Same validation and
 * error codes as the forward.
 * ------------------------------------------------------------------------- */
lf_status lf_block_sparse_attn_bwd(const lf_geom* g, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* frame_slot, const int32_t* sel_blocks, const int32_t* n_sel,
                                   int32_t max_sel, float softmax_scale, const void* out, const float* lse,
                                   const void* dout, float* delta, float* dq, float* dk_cache, float* dv_cache,
                                   lf_stream stream);

/* ---------------------------------------------------------------------------
 * lf_block_sparse_attn_bwd without the delta argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). The row scratch (delta) lives in
 * a fixed array of LF_NOALLOC_MAX_ROWS floats in the library's device memory,
 * one per GPU, held until the process ends; its address is looked up once per
 * device at the first call on it. The call allocates nothing.
 * Arguments, outputs and errors as lf_block_sparse_attn_bwd; in addition
 * B * H * Fc * T > LF_NOALLOC_MAX_ROWS returns LF_ERR_GEOM, and a failed
 * lookup of the scratch returns LF_ERR_HIP. Calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be ordered by the caller. Every row of the scratch a
 * call reads it has written before, so nothing needs clearing.
 * ------------------------------------------------------------------------- */
lf_status lf_block_sparse_attn_bwd_noalloc(const lf_geom* g, const void* q, const void* k_cache,
                                           const void* v_cache, const int32_t* frame_slot, const int32_t* sel_blocks,
                                           const int32_t* n_sel, int32_t max_sel, float softmax_scale,
                                           const void* out, const float* lse, const void* dout, float* dq,
                                           float* dk_cache, float* dv_cache, lf_stream stream);

/* ---------------------------------------------------------------------------
 * Chunk-aware growth budget ([LF-tech] 2.1; [LF-press] 2). Host only.
 * s_i = s_base - beta / sqrt(sigma_i) for the non-dense chunks, s_i = 0 for
 * dense ones; beta makes the weight-weighted mean of s_i over the non-dense
 * chunks equal s_target:
 *   beta = (s_base - s_target) * sum w_i / sum (w_i / sqrt(sigma_i)).
 * Top-k sizes of chunk i (Fi = hist_frames[i], ns = n_sink[i], nb blocks per
 * frame): budget = (1 - s_i) * Fi * nb - ns * nb blocks beyond the sinks;
 *   k_frames = min(Fi - ns, max(k_frames_min, ceil(budget / nb)))
 *   k_blocks = min(nb, max(1, floor(budget / k_frames + 0.5)))
 * (ceil with a 1e-9 allowance); 0 and 0 when there is nothing to select.
 * A dense chunk gets k_frames = Fi - ns and k_blocks = nb (everything).
 * weight and n_sink may be NULL (all 1 / all 0). sigma_i must be > 0.
 * ------------------------------------------------------------------------- */
lf_status lf_chunk_budget(int32_t n_chunks, const double* sigma, const double* weight, const uint8_t* dense,
                          double s_base, double s_target, const int32_t* hist_frames, const int32_t* n_sink,
                          int32_t blocks_per_frame, int32_t k_frames_min, double* sparsity_out,
                          double* beta_out, int32_t* k_frames_out, int32_t* k_blocks_out);

/* ---------------------------------------------------------------------------
 * KV-cache slot table ([SF] rolling cache: keep the last frames, evict the
 * oldest; [RF] dual cache: the first n_sink frames stay as an anchor). Host
 * only. For the chunk with index `chunk_index` (its frames are absolute
 * frames c*Fc .. c*Fc+Fc-1), returns the history kept next to it and the
 * slot of every logical frame: absolute frame a lives in slot
 *   rolling : a mod cache_slots
 *   anchored: a if a < n_sink, else n_sink + (a - n_sink) mod (cache_slots - n_sink)
 * The history is the newest frames that fit beside the current chunk (plus
 * the anchors), oldest first. frame_slot_out needs cache_slots entries;
 * frame_ids_out (nullable) gets the absolute frame of each logical frame.
 * ------------------------------------------------------------------------- */
lf_status lf_cache_frame_slots(int32_t policy, int32_t cache_slots, int32_t n_sink, int32_t chunk_frames,
                               int32_t chunk_index, int32_t* hist_frames_out, int32_t* frame_slot_out,
                               int32_t* frame_ids_out);

/* Human-readable status name; the detail of the last failure on this thread. */
const char* lf_status_str(lf_status s);
/* Hash of the sources (csrc/ and this header) the library was built from;
 * the Python binding refuses a library whose id differs from its tree's. */
const char* lf_build_id(void);
const char* lf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LF_H_ */
