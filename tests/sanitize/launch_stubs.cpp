// Host-only stand-ins for the kernel launchers of libfp8q, for the
// sanitizer build of the C ABI layer (api.cpp compiled by g++ with
// AddressSanitizer and UndefinedBehaviorSanitizer). Every launcher fails as
// it would on a machine without a GPU, so a call that passes validation
// returns FP8Q_ERR_HIP, exactly as the real library does there; nothing is
// launched or dereferenced. Signatures follow launch.h (a mismatch leaves
// an undefined symbol, and the sanitizer library then fails to load).
#include "launch.h"

namespace fp8q {
namespace {
constexpr hipError_t kNoGpu = hipErrorNoDevice;
}

hipError_t launch_quant_act_1x128(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                                  hipStream_t) { return kNoGpu; }
hipError_t launch_quant_act_scatter(const uint16_t*, int64_t, int64_t, int64_t, int, const int32_t*, int64_t,
                                    uint8_t*, int64_t, float*, int64_t, hipStream_t) { return kNoGpu; }
hipError_t launch_quant_mx(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint32_t*, int64_t,
                           hipStream_t) { return kNoGpu; }
hipError_t launch_quant_mx_pair(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint32_t*, int64_t,
                                const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint32_t*, int64_t,
                                hipStream_t) { return kNoGpu; }
hipError_t launch_quant_act_128x1(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                                  hipStream_t) { return kNoGpu; }
hipError_t launch_quant_act_128x1_pair(int64_t, const uint16_t*, int64_t, int64_t, uint8_t*, int64_t, float*,
                                       int64_t, const uint16_t*, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                                       hipStream_t) { return kNoGpu; }
hipError_t launch_quant_retile_128x1(int64_t, const uint16_t*, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                                     const uint8_t*, int64_t, int64_t, const float*, int64_t, uint8_t*, int64_t,
                                     float*, int64_t, hipStream_t) { return kNoGpu; }
hipError_t launch_retile_128x1(const uint8_t*, int64_t, int64_t, int64_t, const float*, int64_t, uint8_t*, int64_t,
                               float*, int64_t, hipStream_t) { return kNoGpu; }
hipError_t launch_quant_act_weight(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                                   const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t,
                                   uint8_t*, int64_t, float*, int64_t, hipStream_t) { return kNoGpu; }
hipError_t launch_quant_weight(int64_t, const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint8_t*, int64_t,
                               int64_t, float*, int64_t, int64_t, uint8_t*, int64_t, int64_t, float*, int64_t,
                               int64_t, hipStream_t) { return kNoGpu; }
hipError_t launch_gemm(const GemmProblem&, hipStream_t) { return kNoGpu; }
hipError_t launch_grouped_gemm(const GemmProblem&, hipStream_t) { return kNoGpu; }
hipError_t grouped_scratch(void**) { return kNoGpu; }
hipError_t launch_grouped_k_gemm(const GemmProblem&, hipStream_t) { return kNoGpu; }
hipError_t launch_gemm_mx(const GemmProblem&, hipStream_t) { return kNoGpu; }
hipError_t launch_gemm_tensor(const GemmProblem&, hipStream_t) { return kNoGpu; }

}  // namespace fp8q
