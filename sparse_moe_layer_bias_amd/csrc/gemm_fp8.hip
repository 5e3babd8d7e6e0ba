// gemm_fp8.hip -- FP8 E4M3 grouped SwiGLU expert FFN (not yet enabled).
#include "moe_internal.h"

namespace moe {

hipError_t launch_expert_ffn_fp8(const moe_cfg&, const FfnArgs&, const int2*, const int32_t*,
                                 void*, void*, float*, float*, int64_t, int64_t, hipStream_t) {
    return hipErrorNotSupported;
}

size_t packed_weight_bytes_fp8(const moe_cfg&, int) { return 0; }

hipError_t launch_pack_weights_fp8(const moe_cfg&, int, const void*, void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace moe
