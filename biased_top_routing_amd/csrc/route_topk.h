// Biased, group-limited top-k of one token by 16 lanes, shared by the
// standalone top-k kernel (affinities read from memory) and the fused router
// kernel (affinities read from LDS right after the router GEMM), so that both
// select and gate with the same instructions.
//
// The bias enters only the ranking used to select the top-k experts; the gate
// that later multiplies an expert's output uses the original affinity
// (DeepSeek-V3 Technical Report reading notes, Method §1 "Auxiliary-loss-free
// 负载均衡"; DeepSeek V3 product page, "公式解密" box).  A token may use at
// most M of the G expert groups (the one-GPU form of the limit of M nodes per
// token in the same notes).
#pragma once

#include "common.h"

namespace moe {

// Cross-lane moves inside a row of 16 lanes with DPP (VALU rate, no LDS):
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes at xor 1 and xor 2; the
// half-row mirror pairs lane i with 7-i and the row mirror lane i with 15-i.
// Applied in this order, each step pairs lanes whose partial results cover
// disjoint lane sets, so after 1/2/3/4 steps every lane holds the result over
// its 2/4/8/16-lane block.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

// Merge the partner's top-R list into this lane's (both descending).
template <int CTRL, int R>
__device__ __forceinline__ void merge_step(float (&top)[R]) {
  float other[R];
#pragma unroll
  for (int i = 0; i < R; ++i) other[i] = dpp_f32<CTRL>(top[i]);
#pragma unroll
  for (int i2 = 0; i2 < R; ++i2) {
    float v = other[i2];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float hi = fmaxf(top[i], v), lo = fminf(top[i], v);
      top[i] = hi;
      v = lo;
    }
  }
}

// One token per 16 lanes (the caller's wavefront holds four such slices, all
// lanes active).  E = 16 * EPL; lane sl of the slice holds experts
// [sl*EPL, (sl+1)*EPL) and every group spans LG = (E/G)/EPL consecutive lanes
// (a power of two).  `row` points at the token's E affinities (global memory
// or LDS); `b` holds this lane's EPL biases.  Steps:
//   q = s + b (fp32);  each lane keeps the top-TOPR q of its experts, the LG
//   lanes of a group merge their lists, so each holds the group's top-TOPR,
//   added largest first (fp32);  a group's rank = number of groups with a
//   larger score or an equal score and a lower index;  chosen = rank < M;
//   k rounds over 32-bit order keys of q: the largest key (per-lane max, then
//   a 16-lane DPP max), then among the lanes holding it the lowest expert
//   index (DPP min), so ties go to the lower index; the winner clears its
//   entry;  gates = scale * s / sum(s) over the winners, s read back from row.
// Lane sl < k writes slot sl of idx_out / w_out (the token's output rows)
// when `valid`; an invalid token's lanes only take part in the cross-lane moves.
template <int EPL, int TOPR>
__device__ __forceinline__ void topk16_token(const float* row, const float (&b)[EPL], bool valid, int G,
                                             int M, int k, float scale, int32_t* idx_out, float* w_out) {
  constexpr int LPT = 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int sl = lane & (LPT - 1);
  const int slice0 = lane & ~(LPT - 1);     // first lane of this token's slice
  const int E = LPT * EPL;
  const int LG = (E / G) / EPL;              // lanes per group
  const int grp = sl / LG;
  const float* mine = row + sl * EPL;
  float s[EPL], q[EPL];
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int j = 0; j < EPL; j += 4) {
      const float4 v = valid ? *reinterpret_cast<const float4*>(mine + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      s[j] = v.x; s[j + 1] = v.y; s[j + 2] = v.z; s[j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) s[j] = valid ? mine[j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) q[j] = s[j] + b[j];
  // ---- group score: top-TOPR of the group, summed largest first
  float top[TOPR];
#pragma unroll
  for (int i = 0; i < TOPR; ++i) top[i] = -__builtin_huge_valf();
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    float v = q[j];
#pragma unroll
    for (int i = 0; i < TOPR; ++i) {
      const float hi = fmaxf(top[i], v), lo = fminf(top[i], v);
      top[i] = hi;
      v = lo;
    }
  }
  // the LG lanes of a group (an aligned block of 1, 2, 4, 8 or 16 lanes)
  if (LG >= 2) merge_step<kDppXor1>(top);
  if (LG >= 4) merge_step<kDppXor2>(top);
  if (LG >= 8) merge_step<kDppHalfMirror>(top);
  if (LG >= 16) merge_step<kDppMirror>(top);
  float gs = top[0];
#pragma unroll
  for (int i = 1; i < TOPR; ++i) gs = gs + top[i];
  // ---- group rank among the G groups of this token
  int rank = 0;
  for (int h = 0; h < G; ++h) {
    const float o = __shfl(gs, slice0 + h * LG);
    rank += (o > gs) || (o == gs && h < grp);
  }
  const bool chosen = rank < M;
  // ---- k rounds of the 16-lane max over order keys (0 = not selectable: a
  // non-chosen group, a cleared winner, an invalid token)
  uint32_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) key[j] = (valid && chosen) ? float_order_key(q[j]) : 0u;
  int my_e = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t m = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) m = max(m, key[j]);
    m = max(m, dpp_u32<kDppXor1>(m));
    m = max(m, dpp_u32<kDppXor2>(m));
    m = max(m, dpp_u32<kDppHalfMirror>(m));
    m = max(m, dpp_u32<kDppMirror>(m));
    int jl = EPL;                                   // lowest local position holding the max
#pragma unroll
    for (int j = EPL - 1; j >= 0; --j) jl = key[j] == m ? j : jl;
    uint32_t we = jl < EPL ? (uint32_t)(sl * EPL + jl) : 0xFFFFFFFFu;
    we = min(we, dpp_u32<kDppXor1>(we));
    we = min(we, dpp_u32<kDppXor2>(we));
    we = min(we, dpp_u32<kDppHalfMirror>(we));
    we = min(we, dpp_u32<kDppMirror>(we));
    const int jw = (int)we - sl * EPL;              // in [0, EPL) on the winning lane only
#pragma unroll
    for (int j = 0; j < EPL; ++j) key[j] = j == jw ? 0u : key[j];
    if (sl == r) my_e = (int)we;
  }
  const float my_s = (valid && sl < k) ? row[my_e] : 0.f;
  float tot = my_s;
  tot += dpp_f32<kDppXor1>(tot);
  tot += dpp_f32<kDppXor2>(tot);
  tot += dpp_f32<kDppHalfMirror>(tot);
  tot += dpp_f32<kDppMirror>(tot);
  if (valid && sl < k) {
    idx_out[sl] = my_e;
    w_out[sl] = scale * my_s / tot;
  }
}

// E = 16 * EPL, groups of whole lanes (LG a power of two), k <= 16, top-r <= 4.
inline bool topk16_fits(const moe_cfg* c) {
  if (c->E % 16 || c->E / 16 > 16 || c->k > 16 || c->group_topr > 4) return false;
  const int epl = c->E / 16, gsz = c->E / c->G;
  if (gsz % epl) return false;
  const int lg = gsz / epl;
  return (lg & (lg - 1)) == 0;
}

}  // namespace moe
