// Stand-ins for the kernel launchers and the two HIP runtime calls host.cpp
// makes, so that the host library builds with g++ alone (AddressSanitizer
// and UBSan builds of the host code; no GPU). Every launcher records that it
// was reached and returns success.
#include "lf_internal.h"

int g_launches = 0;

namespace lf {
hipError_t launch_compress(const KGeom&, int32_t, const void*, const void*, float*, float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_pool_slots(const KGeom&, int32_t, const void*, float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select(const KGeom&, const float*, const float*, const float*, int32_t, int32_t, int32_t, int32_t*,
                         int32_t*, int32_t*, int32_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select_fused(const KGeom&, int32_t, const void*, const float*, const float*, int32_t, int32_t,
                               int32_t, int32_t*, int32_t*, int32_t*, int32_t, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select_blocks(const KGeom&, const float*, const float*, int32_t, int32_t*, int32_t*, int32_t,
                                hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_check_selection(const KGeom&, const int32_t*, const int32_t*, int32_t, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attention(const KGeom&, int32_t, const void*, const void*, const void*, const int32_t*,
                            const int32_t*, int32_t, float, void*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attention_fp8(const KGeom&, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                                const void*, const int32_t*, const int32_t*, int32_t, float, void*, float*,
                                hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attention_bwd(const KGeom&, const void*, const void*, const void*, const int32_t*, const int32_t*,
                                int32_t, float, const void*, const float*, const void*, float*, float*, float*,
                                float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
static float g_scratch[16];
hipError_t noalloc_scratch(float** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
}  // namespace lf

const char* hipGetErrorString(hipError_t) { return "stub"; }
