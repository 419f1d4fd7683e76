// FP8 (E4M3, block-scaled) expert GEMMs: not built yet.
#include "common.h"
#include "kernels.h"

namespace moe {

moe_status launch_ffn_fp8(const moe_cfg*, const fp8_t*, const float*, const int32_t*,
                          const moe_expert_weights*, const bf16_t*, bf16_t*, bf16_t*, void*, int,
                          hipStream_t) {
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
