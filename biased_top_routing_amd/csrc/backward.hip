// Backward of the layer: the bandwidth-bound steps (combine, slot sum), the
// gate and balance-loss gradient of the router, and the four C entry points.
// The expert and router GEMMs are in gemm_bwd.hip.
//
// With the expert choice fixed, y_t = y_shared_t + sum_j w_tj y_perm[inv_tj] and
// w_tj = scale * s_{t,e_tj} / sum_j' s_{t,e_tj'} (DeepSeek-V3 Technical
// Report：中英对照解读, §2 and §3; the bias only ranks experts: reading notes,
// Method §1).  The sequence-wise balance loss follows the reading stated in
// moe.h (the pages keep such a loss with a very small weight but print no
// formula).  Every reduction below runs in a fixed order, so repeated calls
// give identical bits.
#include <math.h>

#include <algorithm>

#include "bwd_layout.h"
#include "common.h"
#include "ffn_layout.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 f32_to_bf16x8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

constexpr int kMaxTopK = 32;   // validate_cfg bounds k

// One workgroup per token, one lane per 16-byte chunk of the row (up to 1024
// lanes): for each slot j, d_topk_w[t,j] = <dy_t, y_perm[inv_tj]> (fp32,
// per-wave shuffle sums, then the waves in order) and dy_perm[inv_tj] =
// topk_w[t,j] * dy_t.
constexpr int kMaxWaves = 16;
__global__ __launch_bounds__(1024) void combine_bwd_kernel(const uint4* __restrict__ dy,
                                                          const uint4* __restrict__ y_perm,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ topk_w, int k,
                                                          int64_t nchunk, uint4* __restrict__ dy_perm,
                                                          float* __restrict__ d_w) {
  __shared__ float red[kMaxWaves][kMaxTopK];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = 0; j < k; ++j) {
    const int64_t p = inv[t * k + j];
    const float wj = topk_w[t * k + j];
    float s = 0.f;
    for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
      float d[8], y[8], o[8];
      bf16x8_to_f32(dy[t * nchunk + c], d);
      bf16x8_to_f32(y_perm[p * nchunk + c], y);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s = fmaf(d[i], y[i], s);
        o[i] = wj * d[i];
      }
      dy_perm[p * nchunk + c] = f32_to_bf16x8(o);
    }
    s = wave_sum(s);
    if (lane == 0) red[wave][j] = s;
  }
  __syncthreads();
  if ((int)threadIdx.x < k) {
    const int j = threadIdx.x, nw = (int)(blockDim.x / kWave);
    float v = red[0][j];
    for (int w = 1; w < nw; ++w) v += red[w][j];
    d_w[t * k + j] = v;
  }
}

// dx_t = sum_j dx_perm[inv_tj] + dx_shared_t + dx_router_t (fp32, in that order), bf16 out;
// one lane per 16-byte chunk of the row.
__global__ __launch_bounds__(1024) void dispatch_bwd_kernel(const uint4* __restrict__ dx_perm,
                                                           const uint4* __restrict__ dx_shared,
                                                           const float4* __restrict__ dx_router,
                                                           const int32_t* __restrict__ inv, int k,
                                                           int64_t nchunk, uint4* __restrict__ dx) {
  const int64_t t = blockIdx.x;
  for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, v[8];
    for (int j = 0; j < k; ++j) {
      bf16x8_to_f32(dx_perm[(int64_t)inv[t * k + j] * nchunk + c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (dx_shared) {
      bf16x8_to_f32(dx_shared[t * nchunk + c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (dx_router) {
      const float4 a = dx_router[(t * nchunk + c) * 2], b = dx_router[(t * nchunk + c) * 2 + 1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    dx[t * nchunk + c] = f32_to_bf16x8(acc);
  }
}

constexpr int kMaxEPL = 8;   // experts per lane: E <= 512

// Statistics of one chunk of kSeqChunk tokens of one sequence: per expert, how
// often it was selected and the sum of its normalised affinity s_te / sum_e' s_te'.
// Each wave takes every fourth token; the waves' sums are added in order.
__global__ __launch_bounds__(256) void seq_stats_kernel(const float* __restrict__ s, const int32_t* __restrict__ idx,
                                                        int T, int E, int k, int L, int nchunk,
                                                        int32_t* __restrict__ cnt, float* __restrict__ psum) {
  __shared__ int32_t c_lds[512];
  __shared__ float p_lds[4][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x / nchunk, ch = blockIdx.x % nchunk;
  const int t0 = b * L + ch * kSeqChunk, t1 = min(b * L + L, t0 + kSeqChunk);
  for (int e = threadIdx.x; e < E; e += blockDim.x) c_lds[e] = 0;
  __syncthreads();
  float acc[kMaxEPL];
#pragma unroll
  for (int i = 0; i < kMaxEPL; ++i) acc[i] = 0.f;
  for (int t = t0 + wave; t < t1; t += 4) {
    float v[kMaxEPL], rs = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxEPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? s[(int64_t)t * E + e] : 0.f;
      rs += v[i];
    }
    rs = wave_sum(rs);
#pragma unroll
    for (int i = 0; i < kMaxEPL; ++i) acc[i] += v[i] / rs;
    if (lane < k) atomicAdd(&c_lds[idx[(int64_t)t * k + lane]], 1);   // integer counts: order-free
  }
#pragma unroll
  for (int i = 0; i < kMaxEPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) p_lds[wave][e] = acc[i];
  }
  __syncthreads();
  const int64_t out = (int64_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    cnt[out + e] = c_lds[e];
    psum[out + e] = ((p_lds[0][e] + p_lds[1][e]) + p_lds[2][e]) + p_lds[3][e];
  }
}

// Per (sequence, expert): f = E / (k L) * count, P = psum / L; the coefficient
// alpha / nseq * f / L of d L_bal / d s' and the loss alpha / nseq * sum f P.
// One workgroup; every thread sums its (b, e) pairs in a fixed order, then a
// fixed tree over the threads.
__global__ __launch_bounds__(256) void seq_coef_kernel(const int32_t* __restrict__ cnt, const float* __restrict__ psum,
                                                       int E, int k, int L, int nseq, int nchunk, float alpha,
                                                       float* __restrict__ coef, float* __restrict__ loss) {
  __shared__ float red[256];
  float mine = 0.f;
  for (int q = threadIdx.x; q < nseq * E; q += blockDim.x) {
    const int b = q / E, e = q % E;
    int c = 0;
    float ps = 0.f;
    for (int ch = 0; ch < nchunk; ++ch) {
      c += cnt[((int64_t)b * nchunk + ch) * E + e];
      ps += psum[((int64_t)b * nchunk + ch) * E + e];
    }
    const float f = (float)E / ((float)k * (float)L) * (float)c;
    coef[q] = alpha / (float)nseq * f / (float)L;
    mine += f * (ps / (float)L);
  }
  red[threadIdx.x] = mine;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = nseq > 0 ? alpha / (float)nseq * red[0] : 0.0f;
}

// One wavefront per token: ds_e from the gates (selected experts) and from the
// balance loss (every expert, through s' = s / sum s), dlogit = ds s (1 - s),
// stored bf16 for the router GEMMs.
__global__ __launch_bounds__(256) void route_grad_kernel(const float* __restrict__ s, const int32_t* __restrict__ idx,
                                                         const float* __restrict__ d_w, const float* __restrict__ coef,
                                                         int T, int E, int k, int L, float scale,
                                                         bf16_t* __restrict__ dlogit) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int b = t / L;
  float v[kMaxEPL], ds[kMaxEPL], rs = 0.f, gs = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxEPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? s[(int64_t)t * E + e] : 0.f;
    ds[i] = coef && e < E ? coef[(int64_t)b * E + e] : 0.f;   // d L_bal / d s'_te
    rs += v[i];
    gs += ds[i] * v[i];
  }
  rs = wave_sum(rs);
  gs = wave_sum(gs);
#pragma unroll
  for (int i = 0; i < kMaxEPL; ++i) ds[i] = ds[i] / rs - gs / (rs * rs);
  // gates over the selected experts
  const int sel = lane < k ? idx[(int64_t)t * k + lane] : 0;
  const float ss = lane < k ? s[(int64_t)t * E + sel] : 0.f;
  const float dwj = lane < k ? d_w[(int64_t)t * k + lane] : 0.f;
  const float S = wave_sum(ss);
  const float B1 = wave_sum(dwj * ss);
  const float dsel = scale / S * (dwj - B1 / S);
  for (int j = 0; j < k; ++j) {
    const int ej = __shfl(sel, j);
    const float dj = __shfl(dsel, j);
#pragma unroll
    for (int i = 0; i < kMaxEPL; ++i)
      if (ej == lane + 64 * i) ds[i] += dj;
  }
#pragma unroll
  for (int i = 0; i < kMaxEPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) dlogit[(int64_t)t * E + e] = f32_to_bf16(ds[i] * v[i] * (1.0f - v[i]));
  }
}

bool bwd_dtypes_ok(const moe_cfg* c) { return c->act == MOE_BF16 && c->wgt == MOE_BF16; }

// one lane per 16-byte chunk of a row, whole wavefronts, at most 1024 lanes
dim3 row_block(int64_t nchunk) {
  return dim3((unsigned)std::min<int64_t>(align_up((size_t)nchunk, kWave), kMaxWaves * kWave));
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine_backward(const moe_cfg* cfg, const void* dy, const void* y_perm,
                                           const int32_t* inv, const float* topk_w, void* dy_perm,
                                           float* d_topk_w, void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bwd_dtypes_ok(cfg)) return MOE_ERR_UNSUPPORTED;
  if (!dy || !y_perm || !inv || !topk_w || !dy_perm || !d_topk_w) return MOE_ERR_NULL;
  if (cfg->T == 0) return MOE_OK;
  const int64_t nchunk = (int64_t)cfg->H * 2 / 16;
  hipLaunchKernelGGL(combine_bwd_kernel, dim3((unsigned)cfg->T), row_block(nchunk), 0, as_stream(stream), (const uint4*)dy,
                     (const uint4*)y_perm, inv, topk_w, cfg->k, nchunk, (uint4*)dy_perm, d_topk_w);
  return launch_status();
}

namespace {

// Both expert backward entry points; saved == nullptr: recompute g, u.
moe_status expert_ffn_backward(const moe_cfg* cfg, const void* x_perm, const void* x, const int32_t* offsets,
                               const moe_expert_weights* w, const moe_ffn_saved* saved, const void* dy_perm,
                               const void* dy, void* dx_perm, void* dx_shared, const moe_expert_grads* grads,
                               void* ws, size_t ws_bytes, void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bwd_dtypes_ok(cfg)) return MOE_ERR_UNSUPPORTED;
  if (!x_perm || !x || !offsets || !w || !dy_perm || !dy || !dx_perm || !grads || !ws) return MOE_ERR_NULL;
  if (!w->w_gate_up || !w->w_down || !grads->w_gate_up || !grads->w_down) return MOE_ERR_NULL;
  if (cfg->S > 0 && (!w->ws_gate_up || !w->ws_down || !dx_shared || !grads->ws_gate_up || !grads->ws_down))
    return MOE_ERR_NULL;
  const int64_t widest = std::max<int64_t>(cfg->H, 2LL * std::max(cfg->S, 1) * cfg->I);
  if ((int64_t)cfg->T * widest * 2 > INT32_MAX || 2LL * cfg->S * cfg->I * cfg->H * 2 > INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  if (saved && (!saved->g || !saved->u || (cfg->S > 0 && (!saved->gs || !saved->us)))) return MOE_ERR_NULL;
  if (ws_bytes < FfnBwdLayout(cfg).total) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return launch_ffn_bwd_bf16(cfg, (const bf16_t*)x_perm, (const bf16_t*)x, offsets, w, saved,
                             (const bf16_t*)dy_perm, (const bf16_t*)dy, (bf16_t*)dx_perm, (bf16_t*)dx_shared, grads,
                             ws, as_stream(stream));
}

}  // namespace

extern "C" moe_status moe_expert_ffn_backward(const moe_cfg* cfg, const void* x_perm, const void* x,
                                              const int32_t* offsets, const moe_expert_weights* w,
                                              const void* dy_perm, const void* dy, void* dx_perm, void* dx_shared,
                                              const moe_expert_grads* grads, void* ws, size_t ws_bytes,
                                              void* stream) {
  return expert_ffn_backward(cfg, x_perm, x, offsets, w, nullptr, dy_perm, dy, dx_perm, dx_shared, grads, ws,
                             ws_bytes, stream);
}

extern "C" moe_status moe_expert_ffn_backward_saved(const moe_cfg* cfg, const void* x_perm, const void* x,
                                                    const int32_t* offsets, const moe_expert_weights* w,
                                                    const moe_ffn_saved* saved, const void* dy_perm, const void* dy,
                                                    void* dx_perm, void* dx_shared, const moe_expert_grads* grads,
                                                    void* ws, size_t ws_bytes, void* stream) {
  if (!saved) return MOE_ERR_NULL;
  return expert_ffn_backward(cfg, x_perm, x, offsets, w, saved, dy_perm, dy, dx_perm, dx_shared, grads, ws,
                             ws_bytes, stream);
}

extern "C" moe_status moe_route_backward(const moe_cfg* cfg, const void* x, const void* w_router,
                                         const float* scores, const int32_t* topk_idx, const float* d_topk_w,
                                         float alpha, int32_t seq_len, float* dx_router, float* dw_router,
                                         float* loss, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bwd_dtypes_ok(cfg)) return MOE_ERR_UNSUPPORTED;
  if (!x || !w_router || !scores || !topk_idx || !d_topk_w || !dw_router || !loss || !ws) return MOE_ERR_NULL;
  if (!(alpha >= 0.0f) || !isfinite(alpha)) return MOE_ERR_SHAPE;
  if (seq_len < 0 || (seq_len > 0 && cfg->T % seq_len != 0)) return MOE_ERR_SHAPE;
  const RouteBwdLayout L(cfg, seq_len);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  char* base = static_cast<char*>(ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + L.off_cnt);
  float* psum = reinterpret_cast<float*>(base + L.off_psum);
  float* coef = reinterpret_cast<float*>(base + L.off_coef);
  bf16_t* dlogit = reinterpret_cast<bf16_t*>(base + L.off_dlogit);
  float* part = reinterpret_cast<float*>(base + L.off_part);
  if (cfg->T == 0) {
    hipLaunchKernelGGL(seq_coef_kernel, dim3(1), dim3(256), 0, s, cnt, psum, cfg->E, cfg->k, 1, 0, 0, 0.0f, coef,
                       loss);
    return launch_status();
  }
  const bool bal = alpha > 0.0f;
  if (bal) {
    hipLaunchKernelGGL(seq_stats_kernel, dim3((unsigned)(L.nseq * L.nchunk)), dim3(256), 0, s, scores, topk_idx,
                       cfg->T, cfg->E, cfg->k, L.seq_len, L.nchunk, cnt, psum);
    if ((st = launch_status()) != MOE_OK) return st;
  }
  hipLaunchKernelGGL(seq_coef_kernel, dim3(1), dim3(256), 0, s, cnt, psum, cfg->E, cfg->k, L.seq_len,
                     bal ? L.nseq : 0, L.nchunk, alpha, coef, loss);
  if ((st = launch_status()) != MOE_OK) return st;
  hipLaunchKernelGGL(route_grad_kernel, dim3((unsigned)((cfg->T + 3) / 4)), dim3(256), 0, s, scores, topk_idx,
                     d_topk_w, bal ? coef : nullptr, cfg->T, cfg->E, cfg->k, L.seq_len, cfg->route_scale, dlogit);
  if ((st = launch_status()) != MOE_OK) return st;
  return launch_router_bwd_gemms(cfg, (const bf16_t*)x, (const bf16_t*)w_router, dlogit, part, L.nsplit, dw_router,
                                 dx_router, s);
}

extern "C" moe_status moe_dispatch_backward(const moe_cfg* cfg, const void* dx_perm, const void* dx_shared,
                                            const float* dx_router, const int32_t* inv, void* dx, void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bwd_dtypes_ok(cfg)) return MOE_ERR_UNSUPPORTED;
  if (!dx_perm || !inv || !dx || (cfg->S > 0 && !dx_shared)) return MOE_ERR_NULL;
  if (cfg->T == 0) return MOE_OK;
  const int64_t nchunk = (int64_t)cfg->H * 2 / 16;
  hipLaunchKernelGGL(dispatch_bwd_kernel, dim3((unsigned)cfg->T), row_block(nchunk), 0, as_stream(stream),
                     (const uint4*)dx_perm, cfg->S > 0 ? (const uint4*)dx_shared : nullptr,
                     (const float4*)dx_router, inv, cfg->k, nchunk, (uint4*)dx);
  return launch_status();
}
