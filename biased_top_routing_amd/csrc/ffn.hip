// moe_expert_ffn: the routed experts on their segments of the permuted rows and
// the shared experts on every token, each a SwiGLU FFN
// (DeepSeek-V3 Technical Report：中英对照解读, §2 Architecture: shared experts
// every token passes through plus routed experts picked by top-k).
//
// This file holds the entry point, the device-side tile-table builder of the
// grouped GEMMs, and the fp32 expert kernels of the small fp32 configuration.
#include <algorithm>

#include "common.h"
#include "ffn_layout.h"
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------ tile tables
// Segments 0..E-1 are the routed experts (rows offsets[e]..offsets[e+1] of the
// permuted rows); segment E is the shared experts over all T tokens.  Each
// segment contributes ceil(rows / bm) row tiles times its column tiles, with
// the row height bm of the GEMM the table is for.
// Inside a segment the row tiles are cut into groups of kGroupRowTiles; a
// group's tiles are listed column-tile-major.  Tiles that run at the same time
// on one XCD (consecutive entries, or runs of them: grouped_tile_at) then cover
// a few row tiles times a few column tiles, so both their activation rows and
// their weight rows are shared in that XCD's L2, also for segments far larger
// than the number of tiles in flight.  Every workgroup computes the prefix sums over segments in LDS
// (at most 513 segments) and writes its own share of the entries.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int S, int T, int bm1, int bm1_alt, int bm2,
                                                           int bm2_alt, int nt1, int nt1s,
                                                           int nt2,
                                                           TileDesc* __restrict__ t1,
                                                           TileDesc* __restrict__ t2,
                                                           int32_t* __restrict__ hdr) {
  __shared__ int32_t pre1[1024], pre2[1024], mt1_s[1024], mt2_s[1024], row0_s[1024], rows_s[1024], hb1_s[1024],
      hb2_s[1024];
  const int tid = threadIdx.x;
  const int nseg = E + (S > 0 ? 1 : 0);
  int c1 = 0, c2 = 0;
  if (tid < nseg) {
    const int rows = tid < E ? offsets[tid + 1] - offsets[tid] : T;
    const int row0 = tid < E ? offsets[tid] : 0;
    const int mt1 = (rows + bm1 - 1) / bm1, mt2 = (rows + bm2 - 1) / bm2;
    // as many tiles of bm1_alt rows cover the segment: use that height
    hb1_s[tid] = bm1_alt > 0 && (int64_t)mt1 * bm1_alt >= rows ? bm1_alt : bm1;
    hb2_s[tid] = bm2_alt > 0 && (int64_t)mt2 * bm2_alt >= rows ? bm2_alt : bm2;
    c1 = mt1 * (tid < E ? nt1 : nt1s);
    c2 = mt2 * nt2;
    mt1_s[tid] = mt1;
    mt2_s[tid] = mt2;
    row0_s[tid] = row0;
    rows_s[tid] = rows;
  }
  pre1[tid] = c1;
  pre2[tid] = c2;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {   // inclusive scans
    const int v1 = tid >= d ? pre1[tid - d] : 0;
    const int v2 = tid >= d ? pre2[tid - d] : 0;
    __syncthreads();
    pre1[tid] += v1;
    pre2[tid] += v2;
    __syncthreads();
  }
  // turn into exclusive prefixes: ex[g] = inc[g] - c[g]
  const int inc1 = pre1[tid], inc2 = pre2[tid];
  const int total1 = pre1[nseg - 1], total2 = pre2[nseg - 1];
  __syncthreads();
  pre1[tid] = inc1 - c1;
  pre2[tid] = inc2 - c2;
  __syncthreads();
  if (tid == 0 && blockIdx.x == 0) {
    hdr[0] = total1;
    hdr[1] = t2 ? total2 : 0;
    // tiles of the routed segments (they come first; the shared ones follow)
    hdr[4] = S > 0 ? pre1[E] : total1;
    hdr[5] = t2 ? (S > 0 ? pre2[E] : total2) : 0;
  }
  for (int pass = 0; pass < (t2 ? 2 : 1); ++pass) {   // t2 == nullptr: the first table only
    const int* pre = pass == 0 ? pre1 : pre2;
    const int total = pass == 0 ? total1 : total2;
    TileDesc* out = pass == 0 ? t1 : t2;
    for (int L = blockIdx.x * 1024 + tid; L < total; L += gridDim.x * 1024) {
      int lo = 0, hi = nseg;           // last g with pre[g] <= L and a non-empty segment
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= L) lo = mid;
        else hi = mid;
      }
      int g = lo;
      // skip empty segments that share the same prefix value
      while (g + 1 < nseg && pre[g + 1] <= L) ++g;
      const int local = L - pre[g];
      const int mt = pass == 0 ? mt1_s[g] : mt2_s[g];
      const int bm = pass == 0 ? hb1_s[g] : hb2_s[g];
      const int ncol = (pass == 0 ? (g < E ? nt1 : nt1s) : nt2);
      const int q = local / (kGroupRowTiles * ncol);             // row-tile group (all earlier ones full)
      const int idx = local - q * kGroupRowTiles * ncol;
      const int gs = min(kGroupRowTiles, mt - q * kGroupRowTiles);
      const int nt = idx / gs, rt = q * kGroupRowTiles + idx % gs;
      TileDesc d;
      d.seg = g;
      d.row0 = row0_s[g] + rt * bm;
      d.rows = min(bm, rows_s[g] - rt * bm);
      d.nt = nt;
      out[L] = d;
    }
  }
}

moe_status launch_build_tile_tables(const moe_cfg* c, const int32_t* offsets, int bm1, int bm1_alt, int nt1,
                                    int nt1s, TileDesc* t1, int64_t max1, int bm2, int bm2_alt, int nt2, TileDesc* t2,
                                    int64_t max2, int32_t* hdr, hipStream_t st) {
  const int64_t most = max1 > max2 ? max1 : max2;
  const unsigned blocks = (unsigned)std::min<int64_t>(std::max<int64_t>((most + 1023) / 1024, 1), 64);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(blocks), dim3(1024), 0, st, offsets, c->E, c->S, c->T, bm1, bm1_alt,
                     bm2, bm2_alt, nt1, nt1s, nt2, t1, t2, hdr);
  return launch_status();
}

moe_status launch_build_tiles(const moe_cfg* c, const int32_t* offsets, void* ws, hipStream_t st) {
  const FfnLayout L(c);
  char* base = static_cast<char*>(ws);
  return launch_build_tile_tables(c, offsets, L.bm1, L.bm1_alt, (int)L.nt1, (int)L.nt1s,
                                  reinterpret_cast<TileDesc*>(base + L.off_t1), L.max1, L.bm2, L.bm2_alt, (int)L.nt2,
                                  reinterpret_cast<TileDesc*>(base + L.off_t2), L.max2,
                                  reinterpret_cast<int32_t*>(base + L.off_hdr), st);
}

// ------------------------------------------------------------ fp32 experts
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int64_t row) {
  int lo = 0, hi = E;                  // last e with offsets[e] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  while (lo + 1 < E && offsets[lo + 1] <= row) ++lo;
  return lo;
}

// h[row, c] = silu(<a_row, Wg_c>) * <a_row, Wu_c>; one thread per (row, c).
// offsets == nullptr: shared experts (h width S*I, column c -> expert c / I).
// rowmap != nullptr: operand row `row` is row rowmap[row] / k of a (the
// expert-sorted order gathered from x).
__global__ __launch_bounds__(256) void gateup_f32_kernel(const float* __restrict__ a, int64_t nrows,
                                                         const int32_t* __restrict__ rowmap, int k,
                                                         const int32_t* __restrict__ offsets, int E,
                                                         const float* __restrict__ W, int H, int I,
                                                         int hw, float* __restrict__ h) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= nrows * hw) return;
  const int64_t row = id / hw;
  const int c = (int)(id % hw);
  const int ex = offsets ? expert_of_row(offsets, E, row) : c / I;
  const int cc = c % I;
  const float* wg = W + ((int64_t)ex * 2 * I + cc) * H;
  const float* wu = wg + (int64_t)I * H;
  const int64_t arow = rowmap ? (int64_t)(rowmap[row] / k) : row;
  const float4* ar = reinterpret_cast<const float4*>(a + arow * H);
  float g = 0.f, u = 0.f;
  for (int i = 0; i < H / 4; ++i) {
    const float4 x = ar[i];
    const float4 p = reinterpret_cast<const float4*>(wg)[i];
    const float4 q = reinterpret_cast<const float4*>(wu)[i];
    g = fmaf(x.x, p.x, g); g = fmaf(x.y, p.y, g); g = fmaf(x.z, p.z, g); g = fmaf(x.w, p.w, g);
    u = fmaf(x.x, q.x, u); u = fmaf(x.y, q.y, u); u = fmaf(x.z, q.z, u); u = fmaf(x.w, q.w, u);
  }
  h[row * hw + c] = g / (1.0f + expf(-g)) * u;
}

// y[row, n] = sum_k h[row, k] * W_d[k / I][n][k % I]; one thread per (row, n).
__global__ __launch_bounds__(256) void down_f32_kernel(const float* __restrict__ h, int64_t nrows,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       const float* __restrict__ W, int H, int I,
                                                       int kw, float* __restrict__ y) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= nrows * H) return;
  const int64_t row = id / H;
  const int n = (int)(id % H);
  const float* Wb = offsets ? W + (int64_t)expert_of_row(offsets, E, row) * H * I : W;
  const float* hr = h + row * kw;
  float acc = 0.f;
  for (int k0 = 0; k0 < kw; k0 += I) {
    const float4* wr = reinterpret_cast<const float4*>(Wb + (int64_t)(k0 / I) * H * I + (int64_t)n * I);
    const float4* hq = reinterpret_cast<const float4*>(hr + k0);
    for (int i = 0; i < I / 4; ++i) {
      const float4 x = hq[i], w = wr[i];
      acc = fmaf(x.x, w.x, acc); acc = fmaf(x.y, w.y, acc);
      acc = fmaf(x.z, w.z, acc); acc = fmaf(x.w, w.w, acc);
    }
  }
  y[row * H + n] = acc;
}

moe_status launch_ffn_f32(const moe_cfg* c, const float* x_perm, const int32_t* perm,
                          const int32_t* offsets, const moe_expert_weights* w, const float* x,
                          float* y_perm, float* y_shared, void* ws, int phase, hipStream_t st) {
  const FfnLayout L(c);
  char* base = static_cast<char*>(ws);
  float* hp = reinterpret_cast<float*>(base + L.off_hp);
  float* hs = reinterpret_cast<float*>(base + L.off_hs);
  const int64_t P = pairs(c);
  auto blocks = [](int64_t n) { return dim3((unsigned)((n + 255) / 256)); };
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_GATE_UP) {
    hipLaunchKernelGGL(gateup_f32_kernel, blocks(P * c->I), dim3(256), 0, st, perm ? x : x_perm, P, perm,
                       c->k, offsets, c->E, (const float*)w->w_gate_up, c->H, c->I, c->I, hp);
    if (c->S > 0)
      hipLaunchKernelGGL(gateup_f32_kernel, blocks((int64_t)c->T * c->S * c->I), dim3(256), 0, st, x,
                         (int64_t)c->T, (const int32_t*)nullptr, 1, (const int32_t*)nullptr, c->E,
                         (const float*)w->ws_gate_up, c->H, c->I, c->S * c->I, hs);
  }
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_DOWN) {
    hipLaunchKernelGGL(down_f32_kernel, blocks(P * c->H), dim3(256), 0, st, hp, P, offsets, c->E,
                       (const float*)w->w_down, c->H, c->I, c->I, y_perm);
    if (c->S > 0)
      hipLaunchKernelGGL(down_f32_kernel, blocks((int64_t)c->T * c->H), dim3(256), 0, st, hs, (int64_t)c->T,
                         (const int32_t*)nullptr, c->E, (const float*)w->ws_down, c->H, c->I,
                         c->S * c->I, y_shared);
  }
  return launch_status();
}

}  // namespace moe

using namespace moe;

namespace {

// Both FFN entry points: routed gate/up rows from x_perm (perm == nullptr) or
// gathered from x through perm.
moe_status expert_ffn(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                      const int32_t* perm, const int32_t* offsets, const moe_expert_weights* w,
                      const void* x, void* y_perm, void* y_shared, const moe_ffn_saved* saved, void* ws,
                      size_t ws_bytes, int phase, void* stream) {
  moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (phase != MOE_FFN_ALL && phase != MOE_FFN_GATE_UP && phase != MOE_FFN_DOWN)
    return MOE_ERR_UNSUPPORTED;
  const bool gate_up = phase != MOE_FFN_DOWN;
  if (!w || !offsets || !y_perm || !ws || !w->w_gate_up || !w->w_down) return MOE_ERR_NULL;
  if (!perm && !x_perm) return MOE_ERR_NULL;
  if (perm && gate_up && !x) return MOE_ERR_NULL;
  if (cfg->S > 0 && (!x || !y_shared || !w->ws_gate_up || !w->ws_down)) return MOE_ERR_NULL;
  const bool fp8 = cfg->wgt == MOE_FP8_E4M3;
  if (fp8 && ((!perm && !x_perm_scale) || !w->w_gate_up_scale || !w->w_down_scale)) return MOE_ERR_NULL;
  if (fp8 && cfg->S > 0 && (!w->ws_gate_up_scale || !w->ws_down_scale)) return MOE_ERR_NULL;
  if (saved) {
    if (cfg->act != MOE_BF16 || cfg->wgt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (!saved->g || !saved->u || (cfg->S > 0 && (!saved->gs || !saved->us))) return MOE_ERR_NULL;
  }
  // gathered rows are addressed by 32-bit byte offsets into x (one row past
  // the end marks a dropped row)
  if (perm && cfg->act != MOE_F32 &&
      ((int64_t)cfg->T + 1) * cfg->H * (fp8 ? 1 : (int64_t)act_bytes(cfg)) > INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < FfnLayout(cfg).total) return MOE_ERR_WORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  if (cfg->act == MOE_F32)
    return launch_ffn_f32(cfg, (const float*)x_perm, perm, offsets, w, (const float*)x, (float*)y_perm,
                          (float*)y_shared, ws, phase, s);
  if (!fp8)
    return launch_ffn_bf16(cfg, (const bf16_t*)x_perm, perm, offsets, w, (const bf16_t*)x,
                           (bf16_t*)y_perm, (bf16_t*)y_shared, phase == MOE_FFN_DOWN ? nullptr : saved, ws,
                           phase, s);
  return launch_ffn_fp8(cfg, (const fp8_t*)x_perm, x_perm_scale, perm, offsets, w, (const bf16_t*)x,
                        (bf16_t*)y_perm, (bf16_t*)y_shared, ws, phase, s);
}

}  // namespace

extern "C" moe_status moe_expert_ffn(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                                     const int32_t* offsets, const moe_expert_weights* w, const void* x,
                                     void* y_perm, void* y_shared, void* ws, size_t ws_bytes, int phase,
                                     void* stream) {
  if (!x_perm) return MOE_ERR_NULL;
  return expert_ffn(cfg, x_perm, x_perm_scale, nullptr, offsets, w, x, y_perm, y_shared, nullptr, ws, ws_bytes,
                    phase, stream);
}

extern "C" moe_status moe_expert_ffn_gather(const moe_cfg* cfg, const void* x, const int32_t* perm,
                                            const int32_t* offsets, const moe_expert_weights* w,
                                            void* y_perm, void* y_shared, void* ws, size_t ws_bytes,
                                            int phase, void* stream) {
  if (!perm) return MOE_ERR_NULL;
  return expert_ffn(cfg, nullptr, nullptr, perm, offsets, w, x, y_perm, y_shared, nullptr, ws, ws_bytes, phase,
                    stream);
}

extern "C" moe_status moe_expert_ffn_save(const moe_cfg* cfg, const void* x_perm, const int32_t* perm,
                                          const int32_t* offsets, const moe_expert_weights* w, const void* x,
                                          void* y_perm, void* y_shared, const moe_ffn_saved* saved, void* ws,
                                          size_t ws_bytes, int phase, void* stream) {
  if (!saved || (!x_perm && !perm)) return MOE_ERR_NULL;
  return expert_ffn(cfg, x_perm, nullptr, x_perm ? nullptr : perm, offsets, w, x, y_perm, y_shared, saved, ws,
                    ws_bytes, phase, stream);
}
