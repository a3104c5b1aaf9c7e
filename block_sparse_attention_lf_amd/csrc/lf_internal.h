// Internal declarations shared by the HIP kernels and the C-ABI host code of
// liblf.so. Not part of the public interface (include/lf.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf.h"

namespace lf {

// Geometry as the kernels see it: everything derived once on the host, plus
// the slot table copied by value into the launch (no device copy needed).
struct KGeom {
  int32_t B, H, D, T, b, Fc, Fh, ns, S;
  int32_t nb;   // blocks per frame = ceil(T / b)
  int32_t nqb;  // query blocks = Fc * nb
  int32_t Lq;   // queries = Fc * T
  int32_t slot[LF_MAX_FRAMES];
};

// Launchers (one per kernel family). They assume validated arguments and
// return the HIP error of the launch.
hipError_t launch_compress(const KGeom& g, int32_t dtype, const void* q, const void* k_cache, float* q_blk, float* k_blk,
                           float* k_frm, hipStream_t stream);
// Pools the frames in cache slots g.slot[0..g.Fh) into slot-indexed pooled caches.
hipError_t launch_pool_slots(const KGeom& g, int32_t dtype, const void* k_cache, float* kp_blk, float* kp_frm,
                             hipStream_t stream);
hipError_t launch_select(const KGeom& g, const float* q_blk, const float* k_blk, const float* k_frm,
                         int32_t kf, int32_t kb, int32_t k_frames_stride, int32_t* sel_frames,
                         int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, hipStream_t stream);
hipError_t launch_select_fused(const KGeom& g, int32_t dtype, const void* q, const float* kp_blk, const float* kp_frm,
                               int32_t kf, int32_t kb, int32_t k_frames_stride, int32_t* sel_frames,
                               int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, float* q_blk,
                               hipStream_t stream);
hipError_t launch_select_blocks(const KGeom& g, const float* q_blk, const float* k_blk, int32_t k,
                                int32_t* sel_blocks, int32_t* n_sel, int32_t max_sel, hipStream_t stream);
// Counts the selection rows that break the lists' invariants (result[0]) and
// gives the first such row (result[1], -1 if none); one workgroup.
hipError_t launch_check_selection(const KGeom& g, const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel,
                                  int32_t* result, hipStream_t stream);
hipError_t launch_attention(const KGeom& g, int32_t dtype, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel, float scale,
                            void* out, float* lse, hipStream_t stream);
// launch_attention with MX-FP8 queries and keys (E4M3 codes, one E8M0 scale
// per 32 channels) and bf16 values/output; D = 128, 32 < block <= 64.
hipError_t launch_attention_fp8(const KGeom& g, const uint8_t* q8, const uint8_t* q_scale, const uint8_t* k8_cache,
                                const uint8_t* k_scale, const void* v_cache, const int32_t* sel_blocks,
                                const int32_t* n_sel, int32_t max_sel, float scale, void* out, float* lse,
                                hipStream_t stream);
// Backward of launch_attention (bf16): dq [B,H,Lq,D], dk/dv rows of the
// frames in g.slot, delta [B,H,Lq] scratch; all float32.
hipError_t launch_attention_bwd(const KGeom& g, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* sel_blocks, const int32_t* n_sel, int32_t max_sel, float scale,
                                const void* out, const float* lse, const void* dout, float* delta, float* dq,
                                float* dk_cache, float* dv_cache, hipStream_t stream);

// Device address of the fixed row scratch of the allocation-free backward on
// the current device (looked up once per device); hipSuccess or the lookup's error.
hipError_t noalloc_scratch(float** ptr);

}  // namespace lf
