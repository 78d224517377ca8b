// Host-only stand-ins for the kernel launchers of fa_kernels.h, for running
// the C-ABI code (fa_api.cpp) under AddressSanitizer and UBSan on a machine
// without a GPU. Each stub only counts the launch; no device work, no memory
// access through the pointers it receives.
#include "fa_kernels.h"

namespace fa {
int g_launches = 0;
static hipError_t count() {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_forward_bf16(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_forward_f32(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_forward_splitkv_bf16(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_forward_fp8(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_quantize_fp8(const void*, uint8_t*, float*, int, int, int, int, int, hipStream_t) {
  return count();
}
hipError_t launch_bwd_preprocess(const AttnArgs&, hipStream_t, bool) { return count(); }
hipError_t launch_bwd_dkdv_bf16(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_bwd_dq_bf16(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_bwd_dkdv_f32(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_bwd_dq_f32(const AttnArgs&, hipStream_t) { return count(); }
hipError_t launch_dropout_mask(uint64_t, int, int, int, uint32_t, int, int, int, int, uint8_t*,
                               hipStream_t) {
  return count();
}
}  // namespace fa
