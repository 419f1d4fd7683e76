// Launchers shared between the translation units of libmoe.
#pragma once

#include "common.h"

namespace moe {

moe_status launch_route_topk(const moe_cfg* c, const float* scores, const float* bias, int32_t* idx,
                             float* w, hipStream_t st);

moe_status launch_router_bf16(const moe_cfg* c, const bf16_t* x, const bf16_t* w_router,
                              const float* offset, float* scores, hipStream_t st);

// Router GEMM + sigmoid + biased group-limited top-k + gates in one kernel
// (scores may be null); router_topk_fusable tells whether it covers c.
bool router_topk_fusable(const moe_cfg* c);
moe_status launch_router_topk_bf16(const moe_cfg* c, const bf16_t* x, const bf16_t* w_router, const float* offset,
                                   const float* bias, float* scores, int32_t* idx, float* w, hipStream_t st);

// x_perm: the expert-sorted rows written by dispatch; or perm != nullptr: the
// routed gate/up rows are gathered from x (row p = token perm[p] / k) and
// x_perm is not read.  saved != nullptr: the gate/up GEMM also stores its gate
// and up outputs there.
moe_status launch_ffn_bf16(const moe_cfg* c, const bf16_t* x_perm, const int32_t* perm,
                           const int32_t* offsets, const moe_expert_weights* w, const bf16_t* x,
                           bf16_t* y_perm, bf16_t* y_shared, const moe_ffn_saved* saved, void* ws, int phase,
                           hipStream_t st);

moe_status launch_ffn_f32(const moe_cfg* c, const float* x_perm, const int32_t* perm,
                          const int32_t* offsets, const moe_expert_weights* w, const float* x,
                          float* y_perm, float* y_shared, void* ws, int phase, hipStream_t st);

moe_status launch_ffn_fp8(const moe_cfg* c, const fp8_t* x_perm, const float* x_perm_scale,
                          const int32_t* perm, const int32_t* offsets, const moe_expert_weights* w,
                          const bf16_t* x, bf16_t* y_perm, bf16_t* y_shared, void* ws, int phase,
                          hipStream_t st);

// Builds the tile tables of the grouped GEMMs from the per-expert offsets.
moe_status launch_build_tiles(const moe_cfg* c, const int32_t* offsets, void* ws, hipStream_t st);

struct TileDesc;
// Two tables (t1: row height bm1, or bm1_alt for a segment that needs no more
// tiles of that height (bm1_alt = 0: never), nt1 column tiles per routed
// segment, nt1s for the shared one; t2: bm2 or bm2_alt alike and nt2 for every
// segment) and their
// sizes in hdr[0], hdr[1], and the tiles of their routed segments (which come
// before the shared ones) in hdr[4], hdr[5]; t2 == nullptr builds t1 only
// (hdr[1] = hdr[5] = 0).  hdr holds at least 8 ints.
moe_status launch_build_tile_tables(const moe_cfg* c, const int32_t* offsets, int bm1, int bm1_alt, int nt1,
                                    int nt1s, TileDesc* t1, int64_t max1, int bm2, int bm2_alt, int nt2, TileDesc* t2,
                                    int64_t max2, int32_t* hdr, hipStream_t st);

// Quantises rows of bf16 values to E4M3 per 1 x 128 tile (sc = amax/448).
moe_status launch_quantize_rows(const bf16_t* src, int64_t rows, int cols, fp8_t* dst, float* scales,
                                hipStream_t st);

// The gate/up GEMM storing its gate and up outputs (bf16, [rows, I] routed,
// [T, S*I] shared) over a table built with the gate/up tile (kBM1 rows, kBNH
// columns): the recomputation the backward pass starts from.
moe_status launch_gateup_recompute_bf16(const moe_cfg* c, const bf16_t* x_perm, const bf16_t* x,
                                        const moe_expert_weights* w, const TileDesc* tiles,
                                        const int32_t* ntiles, int64_t max_tiles, bf16_t* g, bf16_t* u,
                                        bf16_t* gs, bf16_t* us, hipStream_t st);

// Backward GEMMs (gemm_bwd.hip): the expert part (g, u from saved, or
// recomputed when saved == nullptr; dh -> dgu, h; dx; dW_gu; dW_d) and the
// router part (dW_r by split-K partials, dx_router).
moe_status launch_ffn_bwd_bf16(const moe_cfg* c, const bf16_t* x_perm, const bf16_t* x, const int32_t* offsets,
                               const moe_expert_weights* w, const moe_ffn_saved* saved, const bf16_t* dy_perm,
                               const bf16_t* dy, bf16_t* dx_perm, bf16_t* dx_shared, const moe_expert_grads* gr,
                               void* ws, hipStream_t st);
moe_status launch_router_bwd_gemms(const moe_cfg* c, const bf16_t* x, const bf16_t* w_router,
                                   const bf16_t* dlogit, float* part, int nsplit, float* dw_router,
                                   float* dx_router, hipStream_t st);

}  // namespace moe
