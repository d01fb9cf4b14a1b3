// Stand-ins for the GPU launchers, so that the host ABI (abi.cpp) links into
// a sanitizer build without device code. Every launch reports that no
// device is present; the kernel choices follow the library's rules only as
// far as the checks in abi_checks.cpp need.
#include "mis_internal.h"

namespace mis {

hipError_t launch_segments(const mis_segments &, const int32_t *, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_segments_inline(const mis_segments &, const InlineLayout &, const InlineMeta &, int32_t *,
                                  hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attention_f32(const mis_segments &, const float *, const float *, const float *, float *, int, int,
                                int, float, int, hipStream_t) {
  return hipErrorNoDevice;
}
AttnKernel pick_attention_bf16(const mis_segments &, int, int, AttnForce) { return AttnKernel::Pipe32; }
const char *attention_bf16_name(AttnKernel) { return "stub"; }
hipError_t launch_attention_bf16(const mis_segments &, const void *, const void *, const void *, void *, int, int, int,
                                 float, int, AttnKernel, const float *, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_rope(const mis_segments &, void *, void *, mis_dtype, int, int, int, const RopeFreq &,
                       hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_rope_table(float *, int, int, const RopeFreq &, hipStream_t) { return hipErrorNoDevice; }
ScoreKernel pick_score(int, int, mis_dtype, ScoreForce, int) { return {ScoreKind::Narrow, 1}; }
void score_kernel_name(const ScoreKernel &, char *buf, size_t n) {
  if (n) buf[0] = 0;
}
hipError_t score_scratch(void **) { return hipErrorNoDevice; }
hipError_t launch_score(const int32_t *, int, const void *, int, const void *, int, mis_dtype, const LabelArgs &, int,
                        float *, float *, const ScoreKernel &, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace mis
