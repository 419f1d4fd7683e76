// moe_combine: gated gather of the routed expert outputs plus the shared output.
// moe_update_bias: the per-step +-gamma balancing rule.
//
// Combine weights each routed output by its gate, which comes from the raw
// affinity (DeepSeek-V3 Technical Report：中英对照解读, §2.2 and §3).  The bias
// update follows the reading notes (Method §1 "Auxiliary-loss-free 负载均衡")
// and the qwbw.cn essay's load-balancing section: after each step an
// overloaded expert's bias falls by gamma and an underloaded one's rises.
#include <algorithm>

#include "common.h"

namespace moe {

// One workgroup per token with one lane per 16-byte chunk of the row (8 bf16 or
// 4 fp32 values; up to 1024 lanes, whole wavefronts): every routed row of a
// token is in flight at once (measured at 7168 bf16 columns: 896 lanes 9%
// faster than 256 lanes looping over 3.5 chunks each).
// y = y_shared + sum_j w_j * y_perm[inv_j], fp32 accumulation, j ascending.
// The k routed rows of a chunk are loaded in batches of 8 before they are
// accumulated, so that a lane keeps up to 9 loads in flight.  Each output row
// is read once and written once: the loads and stores are non-temporal.
#ifndef MOE_COMBINE_NT
#define MOE_COMBINE_NT 1
#endif
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
#if MOE_COMBINE_NT
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
#if MOE_COMBINE_NT
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
#else
  *p = v;
#endif
}

template <bool BF16>
__device__ __forceinline__ void accum_chunk(float* acc, uint4 r, float g) {
  const uint32_t w4[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (BF16) {
      acc[2 * i] = fmaf(g, bf16_to_f32((bf16_t)(w4[i] & 0xFFFF)), acc[2 * i]);
      acc[2 * i + 1] = fmaf(g, bf16_to_f32((bf16_t)(w4[i] >> 16)), acc[2 * i + 1]);
    } else {
      acc[i] = fmaf(g, __uint_as_float(w4[i]), acc[i]);
    }
  }
}

constexpr int kMaxCombineK = 32;   // validate_cfg bounds k

template <bool BF16>
__global__ __launch_bounds__(1024) void combine_kernel(const uint4* __restrict__ y_perm,
                                                      const uint4* __restrict__ y_shared,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int64_t nchunk,
                                                      uint4* __restrict__ y) {
  constexpr int KB = 8;   // routed rows loaded per batch
  // The token's slot rows and gates, read once into LDS while every lane is
  // active: the chunk loop below is divergent in its last wavefront (nchunk
  // need not be a multiple of 64), so the slot values must not come from
  // cross-lane moves inside it (a lane that left the loop supplies nothing).
  __shared__ int32_t slot_row[kMaxCombineK];
  __shared__ float slot_w[kMaxCombineK];
  const int64_t t = blockIdx.x;          // the whole workgroup on one token
  const int c0 = threadIdx.x, cstep = blockDim.x;
  if (t >= T) return;
  if ((int)threadIdx.x < k) {
    slot_row[threadIdx.x] = inv[t * k + threadIdx.x];
    slot_w[threadIdx.x] = topk_w[t * k + threadIdx.x];
  }
  __syncthreads();
  constexpr int V = BF16 ? 8 : 4;
  for (int64_t c = c0; c < nchunk; c += cstep) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    if (y_shared) accum_chunk<BF16>(acc, ld_stream(&y_shared[t * nchunk + c]), 1.0f);
    for (int j0 = 0; j0 < k; j0 += KB) {
      uint4 r[KB];
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        // slots past k reload slot j0's row (kept in range, weight 0 below)
        const int j = j0 + jj < k ? j0 + jj : j0;
        const int64_t p = slot_row[j];
        r[jj] = ld_stream(&y_perm[p * nchunk + c]);
      }
#pragma unroll
      for (int jj = 0; jj < KB; ++jj) {
        if (j0 + jj < k) accum_chunk<BF16>(acc, r[jj], slot_w[j0 + jj]);
      }
    }
    uint4 o;
    if (BF16) {
      o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    } else {
      o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3]));
    }
    st_stream(&y[t * nchunk + c], o);
  }
}

// One thread per expert; fp32 adds with round-to-nearest-even.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          float* __restrict__ bias, int E,
                                                          int64_t total, float gamma, int eq_mode) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t load = (int64_t)counts[e] * E;
  const float b = bias[e];
  if (load > total) bias[e] = b - gamma;
  else if (load < total || eq_mode == 0) bias[e] = b + gamma;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const moe_cfg* cfg, const void* y_perm, const void* y_shared,
                                  const int32_t* inv, const float* topk_w, void* y, void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!y_perm || !inv || !topk_w || !y) return MOE_ERR_NULL;
  if (cfg->S > 0 && !y_shared) return MOE_ERR_NULL;
  if (cfg->T == 0) return MOE_OK;
  const int64_t nchunk = (int64_t)cfg->H * act_bytes(cfg) / 16;
  const dim3 grid((unsigned)cfg->T);
  const dim3 block((unsigned)std::min<int64_t>(align_up((size_t)nchunk, kWave), 1024));
  const uint4* ysh = cfg->S > 0 ? (const uint4*)y_shared : nullptr;
  if (cfg->act == MOE_F32)
    hipLaunchKernelGGL((combine_kernel<false>), grid, block, 0, as_stream(stream), (const uint4*)y_perm,
                       ysh, inv, topk_w, cfg->T, cfg->k, nchunk, (uint4*)y);
  else
    hipLaunchKernelGGL((combine_kernel<true>), grid, block, 0, as_stream(stream), (const uint4*)y_perm,
                       ysh, inv, topk_w, cfg->T, cfg->k, nchunk, (uint4*)y);
  return launch_status();
}

extern "C" moe_status moe_update_bias(const moe_cfg* cfg, const int32_t* counts, float* bias, float gamma,
                                      void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!counts || !bias) return MOE_ERR_NULL;
  if (!(gamma == gamma)) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(bias_update_kernel, dim3((cfg->E + 255) / 256), dim3(256), 0, as_stream(stream), counts,
                     bias, cfg->E, pairs(cfg), gamma, cfg->bias_eq_mode);
  return launch_status();
}
