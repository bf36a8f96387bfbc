// Prefill expert FFN (T > 8 tokens): grouped GEMM on MFMA (gfx950).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace moe {

bool gemm_shape_supported(const moe_config&) { return false; }

hipError_t launch_ffn_gemm(const moe_config&, const BlobLayout&, const void*, int32_t, const int32_t*,
                           const int32_t*, const void*, const void*, const ExpertList&, float*, void*,
                           hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace moe
