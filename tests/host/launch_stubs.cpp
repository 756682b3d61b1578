// Kernel launchers replaced by stubs, for a CPU-only build of the C ABI's host
// code (api.cpp, nf4_table.cpp, plan.cpp) under the address and
// undefined-behaviour sanitizers.  Argument validation runs entirely before any
// launch, so the host tests never reach these; if one is reached it reports
// hipErrorNoDevice, as a launch on a machine without a GPU does.
#include "launch.hpp"

namespace nf4k {

#define NF4_STUB return hipErrorNoDevice

hipError_t launch_quantize(const float*, int64_t, bool, uint8_t*, void*, float*, uint8_t*, void*, float*,
                           const NF4Enc&, const NF4Consts&, hipStream_t) { NF4_STUB; }
hipError_t launch_dequantize(const uint8_t*, const void*, const float*, const uint8_t*, const void*, const float*,
                             int64_t, bool, bool, void*, const NF4Consts&, hipStream_t) { NF4_STUB; }
hipError_t launch_quantize_error(const float*, int64_t, bool, uint8_t*, void*, float*, bool, double*, double*,
                                 const NF4Enc&, const NF4Consts&, hipStream_t) { NF4_STUB; }
hipError_t launch_error(const float*, int64_t, bool, double*, double*, const NF4Enc&, hipStream_t) { NF4_STUB; }
hipError_t launch_error_batch(const float* const*, const int64_t*, const int64_t*, int32_t, bool, double*, double*,
                              const NF4Enc&, hipStream_t) { NF4_STUB; }
hipError_t launch_topk(const double*, int, int, int*, hipStream_t) { NF4_STUB; }
hipError_t launch_check_finite(const float*, int64_t, int*, hipStream_t) { NF4_STUB; }
hipError_t launch_mfma_peak(int, int, float*, hipStream_t) { NF4_STUB; }
hipError_t noalloc_scratch(void**) { NF4_STUB; }
hipError_t launch_nf4_gemm(int, int, const uint16_t*, const uint16_t*, const uint8_t*, const void*, const float*,
                           const uint8_t*, const void*, const float*, const uint16_t*, const uint16_t*, int, int,
                           uint16_t*, int64_t, int, int, const NF4Consts&, hipStream_t) { NF4_STUB; }
hipError_t launch_merge(int, const float*, const uint8_t*, const void*, const float*, const uint8_t*, const void*,
                        const float*, const uint16_t*, const uint16_t*, int, float, int64_t, int64_t, bool, void*,
                        const NF4Consts&, hipStream_t) { NF4_STUB; }
hipError_t launch_prep(const PrepArgs&, hipStream_t) { NF4_STUB; }
hipError_t launch_skinny_nt(const NtArgs&, int, hipStream_t) { NF4_STUB; }
hipError_t launch_skinny_tn(const TnArgs&, int, hipStream_t) { NF4_STUB; }
hipError_t launch_skinny_tn2(const TnArgs&, const TnArgs*, int, hipStream_t) { NF4_STUB; }

}  // namespace nf4k
