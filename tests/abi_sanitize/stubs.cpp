// Launcher stubs for the host-sanitizer build of the C ABI (api.cpp): the
// refusal paths under test return before any launcher is reached, and
// nothing here touches a device.  Test infrastructure only.
#include "../../block_scaled_fp4_mxfp4_amd/csrc/internal.h"

namespace fp4q {
int device_cus() { return 256; }
hipError_t launch_quant_nvfp4(const void*, int, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, float*, int, int,
                              hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_amax_to_cell(const void*, int, int64_t, int64_t, int64_t, float*, uint8_t*, int64_t,
                               hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quant_mxfp4(const void*, int, int64_t, int64_t, int64_t, const float*, int, uint8_t*, uint8_t*,
                              hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_hadamard32_scale(const void*, int, int64_t, int64_t, int64_t, const float*, float*, int64_t,
                                   hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_balance_scale(const void*, int, int64_t, int64_t, int64_t, const void*, int, int64_t, int64_t,
                                double, float*, float*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_sigma_delta(const fp4q_sd_segment*, int, int, int64_t, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_stochastic_round(const fp4q_sd_segment*, int, int, int64_t, uint64_t, uint32_t, int,
                                   hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_harmonize_nvfp4(const fp4q_nv_member*, int, float*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_hessian(const float*, int64_t, int64_t, int64_t, double*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_macaq_refine(const float*, int64_t, int64_t, int64_t, const double*, double, int, uint8_t*,
                               uint8_t*, int32_t*, double*, hipStream_t) { return hipErrorInvalidValue; }
int64_t macaq_scratch_rows(int64_t n) { return n < 1 ? 0 : (kMacaqScratchDoubles - 32 - ((n + 31) / 32) * 32) / n; }
hipError_t launch_macaq_refine_static(const float*, int64_t, int64_t, int64_t, const double*, double, int,
                                      uint8_t*, uint8_t*, int32_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_mxfp4(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t,
                             int64_t, float*, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_mxfp4_staged(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t,
                                    int64_t, int64_t, float*, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_nvfp4_staged(const uint8_t*, const uint8_t*, const float*, const uint8_t*, const uint8_t*,
                                    const float*, int64_t, int64_t, int64_t, float*, int64_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_gemm_nvfp4(const uint8_t*, const uint8_t*, const float*, const uint8_t*, const uint8_t*,
                             const float*, int64_t, int64_t, int64_t, float*, int64_t, hipStream_t) {
  return hipErrorInvalidValue;
}
bool w4a16_direct_supported(int64_t, int64_t, int64_t, int64_t) { return false; }
hipError_t launch_gemm_w4a16_direct(const void*, int64_t, const uint8_t*, const uint8_t*, const float*, int64_t,
                                    int64_t, int64_t, float*, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_w4a16(const void*, int64_t, const uint8_t*, const uint8_t*, const float*, int64_t, int64_t,
                             int64_t, float*, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_w4a16_grouped(const fp4q_w4a16_problem*, int, hipStream_t) { return hipErrorInvalidValue; }
bool skinny_supported(int64_t K) { return K <= 7168; }
hipError_t launch_gemm_nvfp4_skinny(const void*, int64_t, const uint8_t*, const uint8_t*, const float*, int,
                                    const uint8_t*, const uint8_t*, const float*, int64_t, int64_t, int64_t, float*,
                                    int64_t, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace fp4q
