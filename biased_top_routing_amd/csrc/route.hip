// moe_route: router GEMM + sigmoid affinity, then biased group-limited top-k
// with gates from the raw affinity.
//
// The bias enters only the ranking used to select the top-k experts; the gate
// that later multiplies an expert's output uses the original affinity
// (DeepSeek-V3 Technical Report reading notes, Method §1 "Auxiliary-loss-free
// 负载均衡"; DeepSeek-V3 Technical Report：中英对照解读, §3; DeepSeek V3
// product page, "公式解密" box).  A token may use at most M of the G expert
// groups, the one-GPU form of the pages' limit of M nodes per token.
#include "common.h"
#include "kernels.h"
#include "route_topk.h"

namespace moe {

// ------------------------------------------------------------------ fp32 router
// One thread per (token, expert) logit; used for the small fp32 configuration.
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ off,
                                                         float* __restrict__ scores, int T, int H,
                                                         int E) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)T * E) return;
  const int t = (int)(id / E), e = (int)(id % E);
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)t * H);
  const float4* wr = reinterpret_cast<const float4*>(w + (int64_t)e * H);
  float acc = 0.f;
  for (int i = 0; i < H / 4; ++i) {
    const float4 a = xr[i], b = wr[i];
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
  }
  if (off) acc += off[e];
  scores[id] = 1.0f / (1.0f + expf(-acc));
}

// ------------------------------------------------------------------ top-k
// One token per slice of LPT lanes (64 / LPT tokens per wavefront); lane l of
// a slice holds experts [l*EPL, (l+1)*EPL).  Steps per token:
//   q = s + b (fp32);  group score = fp32 sum of the group's top-r q, largest
//   first (one lane per group);  chosen groups = rank < M under (score desc,
//   index asc);  then k rounds of a slice-wide max over 64-bit keys
//   (order key of q, ~expert) restricted to the chosen groups;
//   gates = scale * s / sum(s) over the selected experts.
template <int EPL, int LPT>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int T, int E, int G, int M,
    int k, int topr, float scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  constexpr int TPW = kWave / LPT;   // tokens per wavefront
  constexpr int TPB = 4 * TPW;       // tokens per block
  extern __shared__ float lds[];
  // per token slot: q[E], s[E], group score[G] (as float), chosen[G] (as int)
  const int stride = 2 * E + 2 * G;
  const int lane = threadIdx.x & (kWave - 1);
  const int sl = lane & (LPT - 1);                      // lane in slice
  const int ts = (threadIdx.x >> 6) * TPW + lane / LPT;  // token slot in block
  float* q_l = lds + ts * stride;
  float* s_l = q_l + E;
  float* gs_l = s_l + E;
  int* ch_l = reinterpret_cast<int*>(gs_l + G);
  const int gsz = E / G;

  float b[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sl * EPL + j;
    b[j] = e < E ? bias[e] : 0.f;
  }

  for (int t0 = blockIdx.x * TPB; t0 < T; t0 += gridDim.x * TPB) {
    const int t = t0 + ts;
    const bool valid = t < T;
    float s[EPL], q[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = sl * EPL + j;
      s[j] = (valid && e < E) ? scores[(int64_t)t * E + e] : 0.f;
      q[j] = s[j] + b[j];
      if (e < E) {
        q_l[e] = q[j];
        s_l[e] = s[j];
      }
    }
    __syncthreads();
    // group scores: lane g of the slice scans group g
    if (sl < G) {
      float top[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) top[i] = -__builtin_huge_valf();
      for (int e = sl * gsz; e < (sl + 1) * gsz; ++e) {
        float v = q_l[e];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i < topr && v > top[i]) {
            const float tmp = top[i];
            top[i] = v;
            v = tmp;
          }
        }
      }
      float gsum = top[0];
#pragma unroll
      for (int i = 1; i < 8; ++i)
        if (i < topr) gsum = gsum + top[i];
      gs_l[sl] = gsum;
    }
    __syncthreads();
    if (sl < G) {
      const float mine = gs_l[sl];
      int rank = 0;
      for (int h = 0; h < G; ++h) {
        const float o = gs_l[h];
        rank += (o > mine) || (o == mine && h < sl);
      }
      ch_l[sl] = rank < M;
    }
    __syncthreads();
    uint64_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = sl * EPL + j;
      const bool ok = valid && e < E && ch_l[e / gsz];
      key[j] = ok ? (((uint64_t)float_order_key(q[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e))
                  : 0ull;
    }
    int my_e = 0;
    for (int r = 0; r < k; ++r) {
      uint64_t best = key[0];
#pragma unroll
      for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
      for (int off = LPT / 2; off > 0; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)best, off);
        const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        best = o > best ? o : best;
      }
      if (sl == r) my_e = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
      for (int j = 0; j < EPL; ++j) key[j] = key[j] == best ? 0ull : key[j];
    }
    const float my_s = (sl < k) ? s_l[my_e] : 0.f;
    float tot = my_s;
#pragma unroll
    for (int off = LPT / 2; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
    if (valid && sl < k) {
      idx_out[(int64_t)t * k + sl] = my_e;
      w_out[(int64_t)t * k + sl] = scale * my_s / tot;
    }
    __syncthreads();   // LDS slots are reused by the next token
  }
}

// Fast form for E = 16 * EPL with groups of whole lanes: one token per 16
// lanes (four per wavefront), no LDS and no barrier; the per-token work is
// topk16_token (route_topk.h), which the fused router kernel runs as well.
template <int EPL, int TOPR>
__global__ __launch_bounds__(256) void route_topk16_kernel(
    const float* __restrict__ scores, const float* __restrict__ bias, int T, int E, int G, int M,
    int k, float scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  constexpr int LPT = 16;
  const int sl = threadIdx.x & (LPT - 1);
  float b[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) b[j] = bias[sl * EPL + j];
  const int64_t tokens_per_grid = (int64_t)gridDim.x * (blockDim.x / LPT);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / LPT) + (threadIdx.x / LPT); t - (threadIdx.x % kWave) / LPT <
       (int64_t)T; t += tokens_per_grid) {
    // (the loop condition keeps whole wavefronts iterating together; lanes of a
    //  token past T load nothing and store nothing)
    const bool valid = t < T;
    const int64_t tr = valid ? t : 0;
    topk16_token<EPL, TOPR>(scores + tr * E, b, valid, G, M, k, scale, idx_out + tr * k, w_out + tr * k);
  }
}

template <int EPL, int TOPR>
static void launch_topk16(const moe_cfg* c, const float* scores, const float* bias, int32_t* idx,
                          float* w, hipStream_t st) {
  const int blocks = (int)std::min<int64_t>(((int64_t)c->T + 15) / 16, 16384);
  hipLaunchKernelGGL((route_topk16_kernel<EPL, TOPR>), dim3(blocks), dim3(256), 0, st, scores, bias, c->T,
                     c->E, c->G, c->M, c->k, c->route_scale, idx, w);
}

template <int EPL>
static void launch_topk16_r(const moe_cfg* c, const float* scores, const float* bias, int32_t* idx,
                            float* w, hipStream_t st) {
  switch (c->group_topr) {
    case 1: launch_topk16<EPL, 1>(c, scores, bias, idx, w, st); break;
    case 2: launch_topk16<EPL, 2>(c, scores, bias, idx, w, st); break;
    case 3: launch_topk16<EPL, 3>(c, scores, bias, idx, w, st); break;
    default: launch_topk16<EPL, 4>(c, scores, bias, idx, w, st); break;
  }
}

template <int EPL, int LPT>
static void launch_topk(const moe_cfg* c, const float* scores, const float* bias, int32_t* idx,
                        float* w, hipStream_t st) {
  constexpr int TPB = 4 * (kWave / LPT);
  const int blocks = (int)std::min<int64_t>(((int64_t)c->T + TPB - 1) / TPB, 8192);
  const size_t lds = (size_t)TPB * (2 * c->E + 2 * c->G) * sizeof(float);
  hipLaunchKernelGGL((route_topk_kernel<EPL, LPT>), dim3(blocks), dim3(256), lds, st, scores, bias,
                     c->T, c->E, c->G, c->M, c->k, c->group_topr, c->route_scale, idx, w);
}

moe_status launch_route_topk(const moe_cfg* c, const float* scores, const float* bias, int32_t* idx,
                             float* w, hipStream_t st) {
  if (topk16_fits(c)) {
    switch (c->E / 16) {
      case 1: launch_topk16_r<1>(c, scores, bias, idx, w, st); break;
      case 2: launch_topk16_r<2>(c, scores, bias, idx, w, st); break;
      case 4: launch_topk16_r<4>(c, scores, bias, idx, w, st); break;
      case 8: launch_topk16_r<8>(c, scores, bias, idx, w, st); break;
      case 16: launch_topk16_r<16>(c, scores, bias, idx, w, st); break;
      default: goto general;
    }
    return launch_status();
  }
general:
  if (c->E <= 16) launch_topk<1, 16>(c, scores, bias, idx, w, st);
  else if (c->E <= 32) launch_topk<1, 32>(c, scores, bias, idx, w, st);
  else if (c->E <= 64) launch_topk<1, 64>(c, scores, bias, idx, w, st);
  else if (c->E <= 128) launch_topk<2, 64>(c, scores, bias, idx, w, st);
  else if (c->E <= 256) launch_topk<4, 64>(c, scores, bias, idx, w, st);
  else launch_topk<8, 64>(c, scores, bias, idx, w, st);
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const moe_cfg* cfg, const void* x, const void* w_router,
                                const float* logit_offset, const float* bias, float* scores,
                                uint32_t flags, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                                void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (flags & ~MOE_SCORES_IN) return MOE_ERR_UNSUPPORTED;
  const bool scores_in = flags & MOE_SCORES_IN;
  if (!bias || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (scores_in && !scores) return MOE_ERR_NULL;
  if (!scores_in && (!x || !w_router)) return MOE_ERR_NULL;
  // without `scores` the affinities are staged in the workspace, unless the
  // fused kernel keeps them in LDS (the workspace is still required, so that a
  // caller's arguments are valid on every device)
  if (!scores && (!ws || ws_bytes < route_ws_bytes(cfg))) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  if (!scores_in && router_topk_fusable(cfg))
    return launch_router_topk_bf16(cfg, (const bf16_t*)x, (const bf16_t*)w_router, logit_offset, bias, scores,
                                   topk_idx, topk_w, s);
  float* sc = scores ? scores : static_cast<float*>(ws);
  if (!scores_in) {
    if (cfg->act == MOE_F32) {
      const int64_t n = (int64_t)cfg->T * cfg->E;
      hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                         (const float*)x, (const float*)w_router, logit_offset, sc, cfg->T,
                         cfg->H, cfg->E);
      if ((st = launch_status()) != MOE_OK) return st;
    } else {
      st = launch_router_bf16(cfg, (const bf16_t*)x, (const bf16_t*)w_router, logit_offset, sc, s);
      if (st != MOE_OK) return st;
    }
  }
  return launch_route_topk(cfg, sc, bias, topk_idx, topk_w, s);
}
