// Launchers shared between the translation units of libmoe.
#pragma once

#include "common.h"

namespace moe {

moe_status launch_route_topk(const moe_cfg* c, const float* scores, const float* bias, int32_t* idx,
                             float* w, hipStream_t st);

moe_status launch_router_bf16(const moe_cfg* c, const bf16_t* x, const bf16_t* w_router,
                              const float* offset, float* scores, hipStream_t st);

// x_perm: the expert-sorted rows written by dispatch; or perm != nullptr: the
// routed gate/up rows are gathered from x (row p = token perm[p] / k) and
// x_perm is not read.
moe_status launch_ffn_bf16(const moe_cfg* c, const bf16_t* x_perm, const int32_t* perm,
                           const int32_t* offsets, const moe_expert_weights* w, const bf16_t* x,
                           bf16_t* y_perm, bf16_t* y_shared, void* ws, int phase, hipStream_t st);

moe_status launch_ffn_f32(const moe_cfg* c, const float* x_perm, const int32_t* perm,
                          const int32_t* offsets, const moe_expert_weights* w, const float* x,
                          float* y_perm, float* y_shared, void* ws, int phase, hipStream_t st);

moe_status launch_ffn_fp8(const moe_cfg* c, const fp8_t* x_perm, const float* x_perm_scale,
                          const int32_t* perm, const int32_t* offsets, const moe_expert_weights* w,
                          const bf16_t* x, bf16_t* y_perm, bf16_t* y_shared, void* ws, int phase,
                          hipStream_t st);

// Builds the tile tables of the grouped GEMMs from the per-expert offsets.
moe_status launch_build_tiles(const moe_cfg* c, const int32_t* offsets, void* ws, hipStream_t st);

// Quantises rows of bf16 values to E4M3 per 1 x 128 tile (sc = amax/448).
moe_status launch_quantize_rows(const bf16_t* src, int64_t rows, int cols, fp8_t* dst, float* scales,
                                hipStream_t st);

}  // namespace moe
