// moe_dispatch: per-expert load count, expert-sorted stable permutation of the
// (token, slot) pairs, and the permuted activation rows.
//
// Tokens are dispatched to the experts they selected and combined back later
// (DeepSeek-V3 Technical Report：中英对照解读, §2.2); each expert's load is
// counted over the whole batch (qwbw.cn essay on the DeepSeek-V3 report,
// load-balancing section).  On one GPU dispatch is a permutation.
//
// Design: no atomics.  Flat pair ids f = t*k + j are cut into segments of
// kSegPairs, one wavefront each.  Inside a wavefront the lanes holding the same
// expert find each other with ballots over the bits of the expert id, so each
// pair learns how many earlier pairs of its segment share its expert, and one
// leader lane per expert updates the segment's LDS counter.  A column scan over
// segments turns the per-segment counts into stable destinations.
#include <mutex>

#include "common.h"
#include "ffn_layout.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Lanes of this wavefront whose (valid) expert id equals mine.
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t on = __ballot(valid && bit);
    m &= bit ? on : ~on;
  }
  return m;
}

// The expert ids of segment `seg` held by this lane (pair lo + 64 it + lane),
// all loaded before any is used; -1 past the last pair.
__device__ __forceinline__ void load_segment(const int32_t* __restrict__ idx, int64_t seg, int64_t N,
                                             int (&ev)[kSegPairs / kWave]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t lo = seg * kSegPairs;
#pragma unroll
  for (int it = 0; it < kSegPairs / kWave; ++it) {
    const int64_t f = lo + it * kWave + lane;
    ev[it] = f < N ? idx[f] : -1;
  }
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int64_t N,
                                                    int E, int nbits, int64_t nseg,
                                                    int32_t* __restrict__ segcounts) {
  extern __shared__ int32_t cnt_all[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t* cnt = cnt_all + wave * E;
  const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __syncthreads();
  int ev[kSegPairs / kWave];
  load_segment(idx, seg, N, ev);
#pragma unroll
  for (int it = 0; it < kSegPairs / kWave; ++it) {
    const bool valid = (unsigned)ev[it] < (unsigned)E;   // (an id outside [0, E) is not counted)
    const int e = valid ? ev[it] : 0;
    const uint64_t m = same_expert_lanes(e, valid, nbits);
    if (valid && (m & lanes_below()) == 0) cnt[e] += __popcll(m);
  }
  __syncthreads();
  if (seg < nseg)
    for (int e = lane; e < E; e += kWave) segcounts[seg * E + e] = cnt[e];
}

// Column scan over segments: segcounts[s][e] becomes the number of pairs of
// expert e in segments before s; counts[e] the total; offsets the exclusive
// prefix of counts over experts.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ segcounts, int64_t nseg,
                                                    int E, int Ep2, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  extern __shared__ int32_t sm[];
  const int P = 1024 / Ep2;                 // parts per expert column
  int32_t* part_sum = sm;                   // [P][Ep2]
  int32_t* tot = sm + P * Ep2;              // [Ep2]
  const int tid = threadIdx.x;
  const int e = tid % Ep2, part = tid / Ep2;
  const int64_t chunk = (nseg + P - 1) / P;
  const int64_t s0 = part * chunk;
  const int64_t s1 = s0 + chunk < nseg ? s0 + chunk : nseg;
  // (the column is walked in batches of kScanBatch segments whose loads are all
  // issued before any is added)
  constexpr int kScanBatch = 16;
  int32_t acc = 0;
  if (e < E)
    for (int64_t b = s0; b < s1; b += kScanBatch) {
      int32_t c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = b + i < s1 ? segcounts[(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) acc += c[i];
    }
  part_sum[part * Ep2 + e] = acc;
  __syncthreads();
  int32_t run = 0;
  for (int p = 0; p < part; ++p) run += part_sum[p * Ep2 + e];
  if (e < E)
    for (int64_t b = s0; b < s1; b += kScanBatch) {
      int32_t c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = b + i < s1 ? segcounts[(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (b + i < s1) {
          segcounts[(b + i) * E + e] = run;
          run += c[i];
        }
    }
  if (part == 0) {
    int32_t total = 0;
    for (int p = 0; p < P; ++p) total += part_sum[p * Ep2 + e];
    tot[e] = e < E ? total : 0;
    if (e < E) counts[e] = total;
  }
  __syncthreads();
  for (int d = 1; d < Ep2; d <<= 1) {     // inclusive scan of tot over experts
    int32_t v = 0;
    if (part == 0 && e >= d) v = tot[e - d];
    __syncthreads();
    if (part == 0) tot[e] += v;
    __syncthreads();
  }
  if (part == 0 && e < E) offsets[e + 1] = tot[e];
  if (tid == 0) offsets[0] = 0;
}

__global__ __launch_bounds__(256) void rank_kernel(const int32_t* __restrict__ idx, int64_t N, int E,
                                                   int nbits, int64_t nseg,
                                                   const int32_t* __restrict__ segprefix,
                                                   const int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ perm,
                                                   int32_t* __restrict__ inv) {
  extern __shared__ int32_t cnt_all[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t* cnt = cnt_all + wave * E;
  const int64_t seg = (int64_t)blockIdx.x * 4 + wave;
  if (seg < nseg)
    for (int e = lane; e < E; e += kWave) cnt[e] = offsets[e] + segprefix[seg * E + e];
  __syncthreads();
  const int64_t lo = seg * kSegPairs;
  int ev[kSegPairs / kWave];
  load_segment(idx, seg, N, ev);
#pragma unroll
  for (int it = 0; it < kSegPairs / kWave; ++it) {
    const int64_t f = lo + it * kWave + lane;
    const bool valid = (unsigned)ev[it] < (unsigned)E;   // (an id outside [0, E) is not counted)
    const int e = valid ? ev[it] : 0;
    const uint64_t m = same_expert_lanes(e, valid, nbits);
    const int32_t base = valid ? cnt[e] : 0;
    const int32_t pos = base + __popcll(m & lanes_below());
    if (valid && (m & lanes_below()) == 0) cnt[e] = base + __popcll(m);
    if (valid) {
      perm[pos] = (int32_t)f;
      inv[f] = pos;
    }
  }
}

// One wavefront per token: load the token's row once, store it to each of its
// k destination rows.  16-byte chunks; CPL chunks per lane per pass.  Plain
// stores: with x read from HBM (the Infinity Cache flushed before the launch)
// non-temporal ones were 11% slower, and a training step, which reads the
// permuted rows back, ran at the same speed with either.
#ifndef MOE_PERMUTE_NT
#define MOE_PERMUTE_NT 0
#endif
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
#if MOE_PERMUTE_NT
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
#else
  *p = v;
#endif
}
template <int CPL>
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint4* __restrict__ src,
                                                           const int32_t* __restrict__ inv, int T,
                                                           int k, int64_t nchunk,
                                                           uint4* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int32_t myp = lane < k ? inv[t * k + lane] : 0;
  for (int64_t c0 = 0; c0 < nchunk; c0 += (int64_t)CPL * kWave) {
    uint4 v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t c = c0 + i * kWave + lane;
      v[i] = src[t * nchunk + (c < nchunk ? c : nchunk - 1)];   // tail lanes reload the last chunk
    }
    for (int j = 0; j < k; ++j) {
      const int64_t p = __shfl(myp, j);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int64_t c = c0 + i * kWave + lane;
        if (c < nchunk) st_stream(&dst[p * nchunk + c], v[i]);
      }
    }
  }
}

// 1 x 128 E4M3 quantisation of a chunk of 8 bf16 values held by this lane;
// 16 consecutive lanes hold one tile.  Returns the 8 codes packed and the
// tile's scale (sc = amax / 448, or 1 for an all-zero tile).
__device__ __forceinline__ uint2 quant_chunk_1x128(uint4 raw, float* sc_out) {
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32((bf16_t)(w[i] & 0xFFFF));
    v[2 * i + 1] = bf16_to_f32((bf16_t)(w[i] >> 16));
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float sc = amax == 0.f ? 1.0f : __fdiv_rn(amax, 448.0f);
  const float y = __fdiv_rn(1.0f, sc);
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = div_by_scale(v[i], sc, y);   // fl32(v / sc)
  *sc_out = sc;
  return make_uint2(e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7]));
}

// fp8 dispatch: quantise the token's bf16 row per 1x128 tile once, then store
// the codes and scales to each of its k destination rows.
template <int CPL>
__global__ __launch_bounds__(256) void permute_rows_fp8_kernel(const uint4* __restrict__ src,
                                                               const int32_t* __restrict__ inv,
                                                               int T, int k, int H,
                                                               uint2* __restrict__ dst,
                                                               float* __restrict__ dst_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;      // whole wavefront exits together
  const int64_t nchunk = H / 8, ntile = H / 128;
  const int32_t myp = lane < k ? inv[t * k + lane] : 0;
  for (int64_t c0 = 0; c0 < nchunk; c0 += (int64_t)CPL * kWave) {
    uint2 q[CPL];
    float sc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t c = c0 + i * kWave + lane;
      // a 16-lane tile group is wholly inside or outside the row (H % 128 == 0)
      const uint4 raw = c < nchunk ? src[t * nchunk + c] : make_uint4(0, 0, 0, 0);
      q[i] = quant_chunk_1x128(raw, &sc[i]);
    }
    for (int j = 0; j < k; ++j) {
      const int64_t p = __shfl(myp, j);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int64_t c = c0 + i * kWave + lane;
        if (c < nchunk) {
          dst[p * nchunk + c] = q[i];
          if ((lane & 15) == 0) dst_scale[p * ntile + c / 16] = sc[i];
        }
      }
    }
  }
}

// Row quantisation without permutation (shared-expert input, tests).
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint4* __restrict__ src,
                                                            int64_t rows, int cols,
                                                            uint2* __restrict__ dst,
                                                            float* __restrict__ dst_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int64_t nchunk = cols / 8, ntile = cols / 128;
  for (int64_t c0 = 0; c0 < nchunk; c0 += kWave) {
    const int64_t c = c0 + lane;
    float sc;
    const uint4 raw = c < nchunk ? src[r * nchunk + c] : make_uint4(0, 0, 0, 0);
    const uint2 q = quant_chunk_1x128(raw, &sc);
    if (c < nchunk) {
      dst[r * nchunk + c] = q;
      if ((lane & 15) == 0) dst_scale[r * ntile + c / 16] = sc;
    }
  }
}

moe_status launch_quantize_rows(const bf16_t* src, int64_t rows, int cols, fp8_t* dst, float* scales,
                                hipStream_t st) {
  if (rows == 0) return MOE_OK;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                     (const uint4*)src, rows, cols, (uint2*)dst, scales);
  return launch_status();
}

// 128 x 128 weight blocks: one workgroup per block.
__global__ __launch_bounds__(256) void quantize_blocks_kernel(const bf16_t* __restrict__ src,
                                                              int rows, int cols,
                                                              uint8_t* __restrict__ dst,
                                                              float* __restrict__ scales) {
  __shared__ float red[4];
  const int nbc = cols / 128, nbr = rows / 128;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / ((int64_t)nbr * nbc);
  const int br = (int)((blk / nbc) % nbr), bc = (int)(blk % nbc);
  const bf16_t* s = src + mat * (int64_t)rows * cols;
  uint8_t* d = dst + mat * (int64_t)rows * cols;
  float v[64];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = threadIdx.x + 256 * i;          // 2048 chunks of 8 values
    const int r = q >> 4, cc = q & 15;
    const uint4 raw = *reinterpret_cast<const uint4*>(s + (int64_t)(br * 128 + r) * cols + bc * 128 + cc * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[8 * i + 2 * h] = bf16_to_f32((bf16_t)(w[h] & 0xFFFF));
      v[8 * i + 2 * h + 1] = bf16_to_f32((bf16_t)(w[h] >> 16));
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) amax = fmaxf(amax, fabsf(v[8 * i + h]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax == 0.f ? 1.0f : __fdiv_rn(amax, 448.0f);
  const float y = __fdiv_rn(1.0f, sc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q >> 4, cc = q & 15;
    float t[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) t[h] = div_by_scale(v[8 * i + h], sc, y);   // fl32(v / sc)
    *reinterpret_cast<uint2*>(d + (int64_t)(br * 128 + r) * cols + bc * 128 + cc * 8) =
        make_uint2(e4m3x4(t[0], t[1], t[2], t[3]), e4m3x4(t[4], t[5], t[6], t[7]));
  }
  if (threadIdx.x == 0) scales[(mat * nbr + br) * nbc + bc] = sc;
}

// The kernels of moe_dispatch, with the per-segment counts in `segc`
// (dispatch_segments(cfg) * E int32, no contents required).  Arguments checked.
static moe_status dispatch_launch(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, int32_t* inv, void* x_perm, float* x_perm_scale,
                                  int32_t* segc, hipStream_t s) {
  moe_status st;
  const bool fp8 = cfg->wgt == MOE_FP8_E4M3;
  const int64_t N = pairs(cfg);
  const int64_t nseg = dispatch_segments(cfg);
  const int E = cfg->E;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  int Ep2 = 1;
  while (Ep2 < E) Ep2 <<= 1;
  const unsigned blocks = (unsigned)((nseg + 3) / 4);
  if (nseg > 0) {
    hipLaunchKernelGGL(count_kernel, dim3(blocks), dim3(256), 4 * E * sizeof(int32_t), s, topk_idx, N,
                       E, nbits, nseg, segc);
    if ((st = launch_status()) != MOE_OK) return st;
  }
  const int P = 1024 / Ep2;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), (size_t)(P + 1) * Ep2 * sizeof(int32_t), s, segc,
                     nseg, E, Ep2, counts, offsets);
  if ((st = launch_status()) != MOE_OK) return st;
  if (nseg == 0) return MOE_OK;
  hipLaunchKernelGGL(rank_kernel, dim3(blocks), dim3(256), 4 * E * sizeof(int32_t), s, topk_idx, N, E,
                     nbits, nseg, segc, offsets, perm, inv);
  if ((st = launch_status()) != MOE_OK) return st;
  if (!x_perm) return MOE_OK;
  const unsigned tblocks = (unsigned)((cfg->T + 3) / 4);
  if (fp8) {
    hipLaunchKernelGGL((permute_rows_fp8_kernel<8>), dim3(tblocks), dim3(256), 0, s, (const uint4*)x, inv,
                       cfg->T, cfg->k, cfg->H, (uint2*)x_perm, x_perm_scale);
  } else {
    const int64_t nchunk = (int64_t)cfg->H * act_bytes(cfg) / 16;
    hipLaunchKernelGGL((permute_rows_kernel<16>), dim3(tblocks), dim3(256), 0, s, (const uint4*)x, inv,
                       cfg->T, cfg->k, nchunk, (uint4*)x_perm);
  }
  return launch_status();
}

static moe_status dispatch_check(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                                 int32_t* offsets, int32_t* perm, int32_t* inv, void* x_perm, float* x_perm_scale) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  const bool fp8 = cfg->wgt == MOE_FP8_E4M3;
  // x_perm == nullptr: indices only (the expert FFN gathers the rows itself)
  if (!topk_idx || !counts || !offsets || !perm || !inv) return MOE_ERR_NULL;
  if (x_perm && (!x || (fp8 && !x_perm_scale))) return MOE_ERR_NULL;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_dispatch(const moe_cfg* cfg, const int32_t* topk_idx, const void* x,
                                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                   void* x_perm, float* x_perm_scale, void* ws, size_t ws_bytes,
                                   void* stream) {
  moe_status st = dispatch_check(cfg, topk_idx, x, counts, offsets, perm, inv, x_perm, x_perm_scale);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < dispatch_ws_bytes(cfg)) return MOE_ERR_WORKSPACE;
  return dispatch_launch(cfg, topk_idx, x, counts, offsets, perm, inv, x_perm, x_perm_scale,
                         static_cast<int32_t*>(ws), as_stream(stream));
}

// ------------------------------------------------ dispatch without a workspace
// The per-segment counts live in a fixed array of device memory that belongs
// to the library (one copy per GPU, held until the process ends).  Host code
// never passes the array's name to a kernel: on the host it only stands for
// the symbol; the array's device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current.
namespace moe {
namespace {
__device__ __align__(256) int32_t scratch[kDispatchScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
int32_t* scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once known

moe_status scratch_on_current_device(int32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_LAUNCH;
    scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace
}  // namespace moe

extern "C" moe_status moe_dispatch_noalloc(const moe_cfg* cfg, const int32_t* topk_idx, const void* x,
                                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                           void* x_perm, float* x_perm_scale, void* stream) {
  moe_status st = dispatch_check(cfg, topk_idx, x, counts, offsets, perm, inv, x_perm, x_perm_scale);
  if (st != MOE_OK) return st;
  if ((size_t)dispatch_segments(cfg) * cfg->E * sizeof(int32_t) > kDispatchScratchBytes) return MOE_ERR_SCRATCH;
  int32_t* segc = nullptr;
  if ((st = scratch_on_current_device(&segc)) != MOE_OK) return st;
  return dispatch_launch(cfg, topk_idx, x, counts, offsets, perm, inv, x_perm, x_perm_scale, segc,
                         as_stream(stream));
}

extern "C" moe_status moe_quantize_fp8(const void* src_bf16, int32_t n_mat, int32_t rows, int32_t cols,
                                       int32_t block_rows, uint8_t* dst, float* scales, void* stream) {
  if (!src_bf16 || !dst || !scales) return MOE_ERR_NULL;
  if (n_mat < 0 || rows < 0 || cols <= 0 || cols % 128) return MOE_ERR_SHAPE;
  if (block_rows != 1 && block_rows != 128) return MOE_ERR_UNSUPPORTED;
  if (rows % block_rows) return MOE_ERR_SHAPE;
  if (n_mat == 0 || rows == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  if (block_rows == 1)
    return launch_quantize_rows((const bf16_t*)src_bf16, (int64_t)n_mat * rows, cols, dst, scales, s);
  const int64_t nblk = (int64_t)n_mat * (rows / 128) * (cols / 128);
  if (nblk >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(quantize_blocks_kernel, dim3((unsigned)nblk), dim3(256), 0, s, (const bf16_t*)src_bf16,
                     rows, cols, dst, scales);
  return launch_status();
}
