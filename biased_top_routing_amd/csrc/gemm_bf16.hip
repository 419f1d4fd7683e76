// bf16 MFMA GEMMs of the layer on gfx950 (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   router   scores[T,E] = sigmoid(x W_r^T + o)
//   gate/up  h = silu(X W_g^T) * (X W_u^T) per expert segment (routed) and over all
//            tokens for the shared experts; h stored as bf16
//   down     Y = h W_d^T per segment; Y stored as bf16
// The layer's experts are SwiGLU FFNs of shared and routed experts (DeepSeek-V3
// Technical Report：中英对照解读, §2 Architecture); the router stays in bf16
// with fp32 accumulation (qwbw.cn essay, FP8 part of the infrastructure section,
// keeps MoE gating in BF16/FP32).
//
// Tiling: a workgroup of WM x WN wavefronts computes a (WM*MI*32) x (WN*NI*32)
// tile; each wavefront owns MI x NI MFMA 32x32 blocks.  A and B K-slices of BK
// columns are staged through LDS by direct-to-LDS buffer loads (a ring of
// STAGES slices, one barrier per slice) with an XOR swizzle of the 16-byte
// chunks so that the MFMA operand reads (32 rows x 16 bytes per half wave) hit
// distinct banks.  For gate/up, the tile's weight rows are BN/2 gate rows and
// the BN/2 up rows of the same intermediate columns, each wavefront holding
// matching gate and up blocks, so SwiGLU is applied in registers.
// Grouped tiles come from a device-built table (segment, first row, rows,
// column tile); each XCD (workgroup id mod 8) takes a contiguous share of the
// shared-expert tiles, then its routed tiles: runs of 8 consecutive entries
// dealt to the XCDs in turn for gate/up, one contiguous share for down
// (grouped_tile_at), so tiles sharing operands run together in one XCD's L2
// and neighbouring XCDs read the same rows close in time.  A gate/up tile
// whose rows fit fewer padded MFMA rows with MI_ALT row blocks per wavefront
// runs that body instead.
// Small batches route through a separate split-K router kernel (no LDS ring).
#include "common.h"
#include "ffn_layout.h"
#include "gemm_common.h"
#include "kernels.h"
#include "route_topk.h"

namespace moe {

// kGateUpGU: the gate/up GEMM storing the gate and up outputs themselves
// (recomputed for the backward pass) instead of h; kGateUpSave: storing h and
// the gate and up outputs (a forward pass that keeps them for the backward).
// kRouterTopk: the router GEMM whose epilogue leaves the tile's affinities in
// LDS (and in `scores` when given) for the workgroup's top-k.
enum { kRouter = 0, kGateUp = 1, kDown = 2, kGateUpGU = 3, kGateUpSave = 4, kRouterTopk = 5 };
constexpr bool is_router(int mode) { return mode == kRouter || mode == kRouterTopk; }
constexpr bool is_gate_up(int mode) { return mode == kGateUp || mode == kGateUpGU || mode == kGateUpSave; }


struct GemmParams {
  const bf16_t* a_routed;   // gate/up: x_perm [P,H]; down: h_perm [P,I]
  const bf16_t* a_shared;   // gate/up and router: x [T,H]; down: h_shared [T,S*I]
  const bf16_t* w_routed;   // gate/up: w_gate_up; down: w_down; router: w_router
  const bf16_t* w_shared;   // gate/up: ws_gate_up; down: ws_down
  const float* offset;      // router logit offset (nullable)
  void* out_routed;         // gate/up: h_perm; down: y_perm; router: scores (fp32)
  void* out_shared;         // gate/up: h_shared; down: y_shared
  bf16_t* g_routed;         // gate/up GU and save: gate outputs [rows, I]
  bf16_t* u_routed;         //   up outputs
  bf16_t* g_shared;         //   shared experts' [T, S*I]
  bf16_t* u_shared;
  const TileDesc* tiles;
  const int32_t* ntiles;
  const int32_t* perm;      // gate/up: non-null -> routed rows gathered from a_shared
  const float* bias;        // router top-k: routing bias [E]
  int32_t* topk_idx;        // router top-k: [T, k] out
  float* topk_w;            //   [T, k] out
  int G, M;                 //   expert groups, groups per token
  float route_scale;
  int T, H, E, S, I, k;
};

// Row pitches (bf16 elements) of the output staging: down 64 columns + 8,
// gate/up 128 h columns + 8.
constexpr int kDownStagePitch = 72;
constexpr int kGateUpStagePitch = 136;

// bf16 elements of LDS a tile's ring needs: STAGES slices of (BM + BN) x BK,
// plus a spare 1 KB when the slice's loads do not divide evenly over the NW
// wavefronts (the short ones issue a dropped load there).
constexpr int ring_elems(int BM, int BN, int BK, int STAGES, int NW) {
  return STAGES * (BM + BN) * BK + (((BM + BN) * (BK / 8) / 64) % NW ? 512 : 0);
}

// Tile of (WM*MI*32) token rows x (WN*NI*32) weight rows; wave (wm, wn) owns
// MI x NI MFMA 32x32 blocks.  K advances BK columns per slice through a ring of
// STAGES LDS stages filled by direct-to-LDS loads.  `lds` holds STAGES stages.
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
template <int MODE, int WM, int WN, int MI, int NI, int BK, int STAGES>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, bf16_t* lds, int seg, int row0, int rows, int nt) {
  constexpr int NW = WM * WN;             // wavefronts per workgroup
  constexpr int NT = 64 * NW;             // threads
  static_assert(NW == 4 || NW == 8 || NW == 16, "4, 8 or 16 wavefronts per workgroup");
  constexpr int BM = WM * MI * 32;
  constexpr int BN = WN * NI * 32;
  constexpr int CPR = BK / 8;             // 16-byte chunks per LDS row
  constexpr int NA = BM * CPR / 64;       // direct-to-LDS instructions of a slice: A rows
  constexpr int NB = BN * CPR / 64;       //   weight rows
  constexpr int PER = (NA + NB + NW - 1) / NW;   // per wave (a short wave's last one is a dropped dummy)
  constexpr int STAGE = (BM + BN) * BK;   // bf16 elements per LDS stage
  static_assert(BM * CPR % 64 == 0 && BN * CPR % 64 == 0, "whole 64-lane instructions");
  // (the wavefront index is uniform: kept in an SGPR, so are the load slots below)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool shared = !is_router(MODE) && seg == p.E;
  // Routed gate/up rows gathered straight from x: row row0 + r of the
  // expert-sorted order is token perm[row0 + r] / k (dispatch's row copy
  // folded into the operand loads).
  const bool gather = is_gate_up(MODE) && !shared && p.perm != nullptr;

  // ------------------------------------------------------------ operand bases
  const bf16_t* A;
  int lda;
  if constexpr (MODE == kDown) {
    A = shared ? p.a_shared : p.a_routed;
    lda = shared ? p.S * p.I : p.I;
  } else {
    A = (is_router(MODE) || shared || gather) ? p.a_shared : p.a_routed;
    lda = p.H;
  }
  const int K = lda;
  if (!gather) A += (int64_t)row0 * lda;
  const int a_rows = gather ? p.T : rows;   // rows covered by the A descriptor

  const bf16_t* W;
  int ldw;
  int64_t seg_kstride = 0;   // down, shared: next shared expert's W_d every I columns of K
  int ncols;                 // valid output columns of this GEMM (h columns for gate/up)
  if constexpr (is_router(MODE)) {
    W = p.w_routed;
    ldw = p.H;
    ncols = p.E;
  } else if constexpr (is_gate_up(MODE)) {
    W = shared ? p.w_shared : p.w_routed + (int64_t)seg * 2 * p.I * p.H;
    ldw = p.H;
    ncols = shared ? p.S * p.I : p.I;
  } else {
    W = shared ? p.w_shared : p.w_routed + (int64_t)seg * p.H * p.I;
    ldw = p.I;
    seg_kstride = (int64_t)p.H * p.I;
    ncols = p.H;
  }

  // Direct-to-LDS loads: one buffer_load_dwordx4 ... lds fills 1 KB of LDS,
  // lane l at +16*l.  The slice's instructions are numbered A first (NA of
  // them), then B (NB); instruction i of wave w is number i*NW + w and covers
  // chunks [64 n, 64 n + 64) of its region; the lane loads the logical chunk
  // that the XOR swizzle places at its physical position.  Token rows past the
  // tile's valid rows get an offset outside the A descriptor, so the hardware
  // drops them without a memory request (their LDS rows feed only outputs that
  // are never stored); weight rows past the valid columns are clamped.  When
  // NA + NB is not a multiple of NW, the waves left short issue one more load
  // with such an out-of-range offset into a spare 1 KB of LDS past the ring,
  // so that every wave has PER loads per slice to wait on.
  int ld_off[PER], ld_pos[PER];
  bool ld_a[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int n = i * NW + wave;          // wave-uniform
    if (n < NA) {
      const int q = n * 64 + lane, r = q / CPR, pc = q % CPR;
      int src = r < rows ? r : a_rows + 1;
      if constexpr (is_gate_up(MODE))
        if (gather && r < rows) src = p.perm[row0 + r] / p.k;
      ld_off[i] = src * lda + swz<CPR>(r, pc) * 8;
      ld_pos[i] = n * 512;
      ld_a[i] = true;
    } else if (n < NA + NB) {
      const int q = (n - NA) * 64 + lane, r = q / CPR, pc = q % CPR;
      int wrow;
      if constexpr (is_gate_up(MODE)) {
        // rows [0, BN/2) gate, [BN/2, BN) up, of h columns nt*BN/2 + j
        const bool up = r >= BN / 2;
        const int c = min(nt * (BN / 2) + (up ? r - BN / 2 : r), ncols - 1);
        wrow = (c / p.I) * 2 * p.I + (up ? p.I : 0) + c % p.I;
      } else {
        wrow = min(nt * BN + r, ncols - 1);
      }
      ld_off[i] = wrow * ldw + swz<CPR>(r, pc) * 8;
      ld_pos[i] = BM * BK + (n - NA) * 512;
      ld_a[i] = false;
    } else {
      ld_off[i] = (a_rows + 1) * lda;     // past the A descriptor: dropped
      ld_pos[i] = -1;                      // the spare LDS past the ring
      ld_a[i] = true;
    }
  }
  // Buffer descriptors over this tile's A rows and this segment's weights: the
  // per-lane part of every address is a 32-bit byte offset, the K advance an
  // SGPR offset.  Accesses past the described range read as zero.
  // (the host checks that a segment's weights stay below 2 GiB)
  int w_bytes;
  if constexpr (is_router(MODE)) w_bytes = p.E * p.H * 2;
  else if constexpr (is_gate_up(MODE)) w_bytes = (shared ? p.S : 1) * 2 * p.I * p.H * 2;
  else w_bytes = (shared ? p.S : 1) * p.H * p.I * 2;
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(A, a_rows * lda * 2);
  const __amdgpu_buffer_rsrc_t rsrc_w = make_rsrc(W, w_bytes);
#pragma unroll
  for (int i = 0; i < PER; ++i) ld_off[i] *= 2;
  typedef __attribute__((address_space(3))) void lds_void_t;
#define MOE_ISSUE(stage_, k0_)                                                                       \
  {                                                                                                  \
    const int k0v = (k0_);                                                                           \
    const int wk = MODE == kDown ? (int)((k0v / p.I) * seg_kstride) + (k0v % p.I) : k0v;             \
    bf16_t* sb = lds + (stage_) * STAGE;                                                             \
    _Pragma("unroll") for (int i = 0; i < PER; ++i) {                                                \
      bf16_t* dst = ld_pos[i] < 0 ? lds + STAGES * STAGE : sb + ld_pos[i];                           \
      if (ld_a[i])                                                                                   \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_void_t*)dst, 16, ld_off[i], k0v * 2, 0, 0); \
      else                                                                                           \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, (lds_void_t*)dst, 16, ld_off[i], wk * 2, 0, 0); \
    }                                                                                                \
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // LDS rows this lane reads for its MFMA operands
  int a_rd[MI], b_rd[NI];
  const int lr = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_rd[mi] = wm * MI * 32 + mi * 32 + lr;
  // A wavefront whose token rows all lie past the tile's valid rows skips its
  // operand reads and MFMAs (one wave-uniform branch per slice: a small tile,
  // e.g. at decode size, then costs little more than its loads).
  const bool has_rows = wm * MI * 32 < rows;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int brow;
    if constexpr (is_gate_up(MODE)) {
      constexpr int HALF = NI / 2;   // gate blocks, then the matching up blocks
      brow = (ni < HALF ? 0 : BN / 2) + wn * HALF * 32 + (ni % HALF) * 32;
    } else {
      brow = wn * NI * 32 + ni * 32;
    }
    b_rd[ni] = brow + lr;
  }

  // Ring: slices kt+1 .. kt+STAGES-2 are in flight while slice kt is multiplied.
  const int nk = K / BK;
  // Down GEMM: each tile starts its K walk at its own slice (3 per column
  // tile, 1 per row tile) and wraps around, so that tiles sharing a weight or
  // h panel do not all wait on the same cache misses at once (measured 2-3%
  // faster).  Only the fp32 summation order of the slices depends on it.
  const int rot = MODE == kDown ? (int)(((unsigned)nt * 3u + (unsigned)(row0 / BM)) % (unsigned)nk) : 0;
  auto kslice = [&](int kt_) { const int q = kt_ + rot; return q >= nk ? q - nk : q; };
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) MOE_ISSUE(s, kslice(s) * BK);
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of slice kt have landed once only the later slices remain
    wait_slices<PER>(min(nk - 1, kt + STAGES - 2) - kt);
    // ... and every wave's; the stage of slice kt-1 is free again.  A bare
    // barrier that is also a compiler memory fence: __syncthreads would drain
    // the loads still in flight (vmcnt(0)).
    asm volatile("s_barrier" ::: "memory");
    if (kt + STAGES - 1 < nk) {
      const int st = cur == 0 ? STAGES - 1 : cur - 1;   // (kt + STAGES - 1) % STAGES
      MOE_ISSUE(st, kslice(kt + STAGES - 1) * BK);
    }
    const bf16_t* base = lds + cur * STAGE;
    // Operand fragments are double-buffered across the BK/16 MFMA k-steps: the
    // reads of step kk+1 are interleaved with the MFMAs of step kk.
    constexpr int KK = BK / 16;
    if (has_rows) {
    bf16x8_t fa[2][MI], fb[2][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      fa[0][mi] = *reinterpret_cast<const bf16x8_t*>(base + a_rd[mi] * BK + swz<CPR>(a_rd[mi], kh) * 8);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      fb[0][ni] = *reinterpret_cast<const bf16x8_t*>(base + BM * BK + b_rd[ni] * BK + swz<CPR>(b_rd[ni], kh) * 8);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cb = kk & 1, nb = cb ^ 1;
      if (kk + 1 < KK) {
        const int c = (kk + 1) * 2 + kh;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          fa[nb][mi] = *reinterpret_cast<const bf16x8_t*>(base + a_rd[mi] * BK + swz<CPR>(a_rd[mi], c) * 8);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          fb[nb][ni] = *reinterpret_cast<const bf16x8_t*>(base + BM * BK + b_rd[ni] * BK +
                                                          swz<CPR>(b_rd[ni], c) * 8);
      }
      // the reads above stay ahead of this step's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][mi], fb[cb][ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    }   // has_rows
    cur = cur == STAGES - 1 ? 0 : cur + 1;
  }
#undef MOE_ISSUE

  // ------------------------------------------------------------ epilogue
  // acc[mi][ni][r] holds C[i][j] with j = lane % 32 and
  // i = 8 * (r / 4) + 4 * (lane / 32) + r % 4 inside the 32 x 32 block.
  if constexpr (is_gate_up(MODE)) {
    // The tile's outputs over BM rows x BN/2 columns -- h = silu(g) * u, and the
    // gate and up outputs g, u themselves where the mode keeps them -- are
    // assembled in LDS one after the other over the finished ring (rows padded to
    // kGateUpStagePitch elements) and stored as whole 256-byte row segments, 16
    // bytes per lane.
    constexpr int HALF = NI / 2;
    constexpr int HC = BN / 2;                      // h columns of the tile
    static_assert(HC * 2 == 256 && BM * kGateUpStagePitch <= STAGES * STAGE, "output tile staging");
    constexpr int NOUT = MODE == kGateUp ? 1 : MODE == kGateUpGU ? 2 : 3;
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
      // output o: kGateUp h; kGateUpGU g, u; kGateUpSave h, g, u
      const int what = MODE == kGateUpGU ? o + 1 : o;   // 0 h, 1 g, 2 u
      __syncthreads();   // the ring (o == 0), or the previous output's stores, are done with the stage
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = wm * MI * 32 + mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
#pragma unroll
          for (int ni = 0; ni < HALF; ++ni) {
            const float g = acc[mi][ni][r], u = acc[mi][ni + HALF][r];
            const float v = what == 0 ? g * gate_sigmoid(g) * u : what == 1 ? g : u;
            lds[i * kGateUpStagePitch + wn * HALF * 32 + ni * 32 + lr] = f32_to_bf16(v);
          }
        }
      __syncthreads();
      bf16_t* out = what == 0 ? static_cast<bf16_t*>(shared ? p.out_shared : p.out_routed)
                  : what == 1 ? (shared ? p.g_shared : p.g_routed)
                              : (shared ? p.u_shared : p.u_routed);
      if (nt * HC < ncols) {   // ncols (I or S*I) is a multiple of 128: the tile's columns are all valid or none
        for (int q = threadIdx.x; q < BM * (HC / 8); q += NT) {
          const int rr = q / (HC / 8), ch = q % (HC / 8);
          if (rr < rows)
            *reinterpret_cast<uint4*>(out + (row0 + rr) * (int64_t)ncols + nt * HC + ch * 8) =
                *reinterpret_cast<const uint4*>(lds + rr * kGateUpStagePitch + ch * 8);
        }
      }
    }
    return;
  }
  if constexpr (MODE == kDown) {
    // A lane holds single values of 16 rows; the wavefront's (MI*32) x (NI*32)
    // outputs pass through LDS (rows padded to kDownStagePitch elements against bank
    // conflicts, over the finished ring) and go out as whole 128-byte row
    // segments, 16 bytes per lane.
    static_assert(NI * 32 * 2 == 128, "a wavefront's columns are one 128-byte row segment");
    __syncthreads();   // every wavefront is done with the ring
    bf16_t* stg = lds + wave * (MI * 32 * kDownStagePitch);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stg[(mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3)) * kDownStagePitch + ni * 32 + lr] =
              f32_to_bf16(acc[mi][ni][r]);
    // (the wavefront reads back only what it wrote; its LDS operations complete in order)
    __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);
    __builtin_amdgcn_wave_barrier();
    bf16_t* out = static_cast<bf16_t*>(shared ? p.out_shared : p.out_routed);
    const int col = nt * BN + wn * NI * 32 + (lane & 7) * 8;   // H is a multiple of 64: whole segment or none
#pragma unroll
    for (int it = 0; it < MI * 32 / 8; ++it) {
      const int lr2 = it * 8 + (lane >> 3);
      const int i = wm * MI * 32 + lr2;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + lr2 * kDownStagePitch + (lane & 7) * 8);
      if (i < rows && col < ncols) *reinterpret_cast<uint4*>(out + (row0 + i) * (int64_t)ncols + col) = v;
    }
    return;
  }
  // kRouterTopk reuses the LDS ring for the [BM][BN] fp32 affinities: every
  // wavefront must be done with its last slice first.
  if constexpr (MODE == kRouterTopk) __syncthreads();
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = wm * MI * 32 + mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (i >= rows) continue;
      const int64_t row = row0 + i;
      if constexpr (MODE == kRouterTopk) {
        // the tile holds every expert of its tokens (nt == 0, BN >= E)
        float* sl = reinterpret_cast<float*>(lds);
        float* out = static_cast<float*>(p.out_routed);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = wn * NI * 32 + ni * 32 + lr;
          float sv = 0.f;
          if (col < ncols) {
            const float l = acc[mi][ni][r] + (p.offset ? p.offset[col] : 0.f);
            sv = 1.0f / (1.0f + expf(-l));
            if (out) out[row * ncols + col] = sv;
          }
          sl[i * BN + col] = sv;
        }
      } else {
        float* out = static_cast<float*>(p.out_routed);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = nt * BN + wn * NI * 32 + ni * 32 + lr;
          if (col < ncols) {
            const float l = acc[mi][ni][r] + (p.offset ? p.offset[col] : 0.f);
            out[row * ncols + col] = 1.0f / (1.0f + expf(-l));
          }
        }
      }
    }
  }
}
#endif

// One workgroup per tile.  Grouped GEMMs (MI_ALT > 0): a tile whose valid rows
// fit fewer MFMA rows with MI_ALT blocks per wavefront (e.g. 161..256 rows:
// 256 with MI_ALT = 4 against 320 with MI = 5) runs the MI_ALT body; both
// bodies share the LDS ring (sized for MI).
template <int MODE, int WM, int WN, int MI, int NI, int BK, int STAGES, int OCC, int MI_ALT = 0>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_bf16_kernel(GemmParams p) {
  static_assert(MI_ALT >= 0 && MI_ALT < MI, "the alternative body has fewer row blocks");
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = WM * MI * 32;
  constexpr int RING = ring_elems(BM, WN * NI * 32, BK, STAGES, WM * WN);
  constexpr int STG = MODE == kDown ? WM * WN * MI * 32 * kDownStagePitch : 0;   // down: output staging
  __shared__ __attribute__((aligned(16))) bf16_t lds[RING > STG ? RING : STG];
  // ------------------------------------------------------------ which tile
  int seg = 0, row0, rows, nt;
  if constexpr (MODE == kRouter) {
    row0 = blockIdx.x * BM;
    rows = min(BM, p.T - row0);
    nt = blockIdx.y;
  } else {
    const int L = grouped_tile<is_gate_up(MODE) ? kStripeGateUp : kStripeDown>(p.ntiles);
    if (L < 0) return;
    const TileDesc d = p.tiles[L];
    // the descriptor is the same for the whole workgroup: keep it in SGPRs
    seg = __builtin_amdgcn_readfirstlane(d.seg);
    row0 = __builtin_amdgcn_readfirstlane(d.row0);
    rows = __builtin_amdgcn_readfirstlane(d.rows);
    nt = __builtin_amdgcn_readfirstlane(d.nt);
  }
  if constexpr (MI_ALT > 0) {
    // MFMA rows computed: whole wavefront row bands of MI*32 (or MI_ALT*32) rows
    constexpr int HM = MI * 32, HA = MI_ALT * 32;
    if (rows <= WM * HA && (rows + HA - 1) / HA * HA < (rows + HM - 1) / HM * HM) {
      gemm_tile<MODE, WM, WN, MI_ALT, NI, BK, STAGES>(p, lds, seg, row0, rows, nt);
      return;
    }
  }
  gemm_tile<MODE, WM, WN, MI, NI, BK, STAGES>(p, lds, seg, row0, rows, nt);
#endif
}

// Router GEMM for small batches, whose token-tile grid would leave most CUs
// idle (decode: T = 128 gives two 64-token tiles, each walking all of K):
// a workgroup computes a TM x TN tile of (tokens, experts) with MFMA blocks of
// TM x TN (32 x 32 x 16 or 16 x 16 x 32 bf16), each of its 16 wavefronts takes
// one sixteenth of K straight from memory into operand registers (no operand is
// shared between wavefronts, so nothing is staged in LDS), and the 16 partial
// tiles are added through LDS in wavefront order (a fixed order: repeated calls
// give identical bits; the summation order, and so the last bits of the
// affinities, differ from the large-batch tiles).  Token and expert rows past
// the ends are clamped to the last valid row and their results not stored.
constexpr int kRsWaves = 16;
template <int TM>   // 32: 32 x 32 x 16 blocks; 16: 16 x 16 x 32 blocks
__global__ __launch_bounds__(64 * kRsWaves) void router_splitk_kernel(const bf16_t* __restrict__ x,
                                                                     const bf16_t* __restrict__ w,
                                                                     const float* __restrict__ offset,
                                                                     float* __restrict__ scores, int T, int H,
                                                                     int E) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NR = TM * TM / 64;       // accumulator values per lane
  constexpr int KS = 512 / TM;           // K per MFMA step (16 or 32)
  __shared__ float red[kRsWaves][NR][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane % TM, kg = lane / TM;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TM;
  // operand lane l: row l % TM, K elements 8 (l / TM) .. + 7 of each step
  const bf16_t* xa = x + (int64_t)min(t0 + lr, T - 1) * H + 8 * kg;
  const bf16_t* wb = w + (int64_t)min(e0 + lr, E - 1) * H + 8 * kg;
  const int nks = H / KS;
  const int ks0 = wave * nks / kRsWaves, ks1 = (wave + 1) * nks / kRsWaves;
  typedef float accv_t __attribute__((ext_vector_type(NR)));
  accv_t acc;
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll 4
  for (int ks = ks0; ks < ks1; ++ks) {
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xa + ks * KS);
    const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(wb + ks * KS);
    if constexpr (TM == 32) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  for (int q = threadIdx.x; q < NR * 64; q += 64 * kRsWaves) {
    const int r = q >> 6, l = q & 63;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < kRsWaves; ++v) sum += red[v][r][l];
    // acc[r] of lane l: 32 x 32 blocks row 8 (r / 4) + 4 (l / 32) + r % 4;
    // 16 x 16 blocks row 4 (l / 16) + r; column l % TM
    const int i = TM == 32 ? 8 * (r >> 2) + 4 * (l >> 5) + (r & 3) : 4 * (l >> 4) + r;
    const int t = t0 + i, e = e0 + l % TM;
    if (t < T && e < E) {
      const float lg = sum + (offset ? offset[e] : 0.f);
      scores[(int64_t)t * E + e] = 1.0f / (1.0f + expf(-lg));
    }
  }
#endif
}

// Router GEMM with the whole routing step in its epilogue, for tiles that hold
// every expert of their tokens (BN >= E): the tile's affinities
// s = sigmoid(x W_r^T + o) go to LDS (and to `scores` when given), then the
// workgroup's 16-lane slices run the biased group-limited top-k of its tokens
// from LDS (topk16_token, the per-token code of the standalone top-k kernel),
// so the [T, E] affinities need not be written and read back.  The GEMM part
// adds the K slices in the order of the standalone router GEMM, so its
// affinities, and with them the selection, are the same bit for bit.
template <int EPL, int TOPR, int WM, int WN, int MI, int NI, int BK, int STAGES>
__global__ __launch_bounds__(64 * WM * WN) void router_topk_kernel(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = WM * MI * 32, BN = WN * NI * 32;
  constexpr int RING = ring_elems(BM, BN, BK, STAGES, WM * WN), SCO = 2 * BM * BN;   // in bf16 elements
  constexpr int TPP = 64 * WM * WN / 16;                            // tokens per pass
  static_assert(16 * EPL <= BN && BM % TPP == 0, "a tile holds every expert; whole passes");
  __shared__ __attribute__((aligned(16))) bf16_t lds[RING > SCO ? RING : SCO];
  const int row0 = blockIdx.x * BM;
  const int rows = min(BM, p.T - row0);
  gemm_tile<kRouterTopk, WM, WN, MI, NI, BK, STAGES>(p, lds, 0, row0, rows, 0);
  __syncthreads();
  const float* sl = reinterpret_cast<const float*>(lds);
  const int l16 = threadIdx.x & 15;
  float b[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) b[j] = p.bias[l16 * EPL + j];
  for (int tt = threadIdx.x / 16; tt < BM; tt += TPP) {   // the same trip count on every lane
    const bool valid = tt < rows;
    const int64_t t = row0 + (valid ? tt : 0);
    topk16_token<EPL, TOPR>(sl + tt * BN, b, valid, p.G, p.M, p.k, p.route_scale, p.topk_idx + t * p.k,
                            p.topk_w + t * p.k);
  }
#endif
}

// CUs of the device current at the first call (a thread-safe one-time query).
static int cu_count() {
  static const int n_cu = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return n_cu;
}

// Router kernel and tile by batch size.  Small batches: the split-K kernel with
// 16 x 16 tiles while there are at most two per CU, else with 32 x 32 tiles
// while there are at most two per CU (route stage with a cache flush, against
// 64 x 256 tiles: E = 256, T = 128 100 -> 27 us, T = 2048 99 -> 82 us; E = 64,
// T = 4096 33 -> 23 us).  Larger batches: every token tile re-reads its columns
// of the router weight from L2, so the tile is as large as the batch allows
// while the grid still covers every CU: 256 x 256 and 128 x 256 for large
// batches, 128 x 128 at T = 16384 with E = 256 (two column tiles of 128
// experts: 3.5 instead of 4.6 MB of operand loads per tile against 64 x 256,
// measured 14% faster), else 64 x 256.
enum RouterTile { kRtSplit16, kRtSplit32, kRt256, kRt128, kRt128N, kRt64 };
using RT256 = TileCfg<MOE_RT256_TILE>;
using RT128 = TileCfg<MOE_RT128_TILE>;
using RT128N = TileCfg<MOE_RT128N_TILE>;
using RT64 = TileCfg<MOE_RT_TILE>;

static RouterTile router_tile(const moe_cfg* c) {
  const int64_t n_cu = cu_count();
  auto tiles = [&](int bm, int bn) { return ((int64_t)c->T + bm - 1) / bm * (((int64_t)c->E + bn - 1) / bn); };
  if (tiles(16, 16) <= 2 * n_cu) return kRtSplit16;
  if (tiles(32, 32) <= 2 * n_cu) return kRtSplit32;
  if (tiles(RT256::BM, RT256::BN) >= n_cu) return kRt256;
  if (tiles(RT128::BM, RT128::BN) >= n_cu) return kRt128;
  if (tiles(RT128N::BM, RT128N::BN) >= n_cu) return kRt128N;
  return kRt64;
}

// The fused kernel runs where the two-kernel path would use 64-token tiles
// anyway (mid-size batches: E = 256 from T = 2049 to 16383); there it saves the
// affinities' round trip and a launch.  Larger batches keep the larger tiles of
// the two-kernel path: with a cache flush, the fused 64 x 256 tiles took
// 0.143 / 0.439 / 1.60 ms against 0.133 / 0.319 / 1.18 ms at T = 16384 / 65536
// / 262144 (every tile re-reads the whole 3.7 MB router weight).
#ifndef MOE_ROUTE_FUSED
#define MOE_ROUTE_FUSED 1
#endif
bool router_topk_fusable(const moe_cfg* c) {
  if (!MOE_ROUTE_FUSED || c->act != MOE_BF16 || !topk16_fits(c) || c->E > 256) return false;
  const int epl = c->E / 16;
  return (epl == 1 || epl == 2 || epl == 4 || epl == 8 || epl == 16) && router_tile(c) == kRt64;
}

template <int EPL, int TOPR>
static void launch_router_topk_r(const moe_cfg* c, const GemmParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((c->T + 63) / 64));
  if constexpr (EPL <= 8)   // 64 tokens x 128 experts
    hipLaunchKernelGGL((router_topk_kernel<EPL, TOPR, 2, 4, 1, 1, 64, 3>), grid, dim3(512), 0, st, p);
  else                      // 64 tokens x 256 experts
    hipLaunchKernelGGL((router_topk_kernel<EPL, TOPR, 2, 4, 1, 2, 64, 3>), grid, dim3(512), 0, st, p);
}

template <int EPL>
static void launch_router_topk_e(const moe_cfg* c, const GemmParams& p, hipStream_t st) {
  switch (c->group_topr) {
    case 1: launch_router_topk_r<EPL, 1>(c, p, st); break;
    case 2: launch_router_topk_r<EPL, 2>(c, p, st); break;
    case 3: launch_router_topk_r<EPL, 3>(c, p, st); break;
    default: launch_router_topk_r<EPL, 4>(c, p, st); break;
  }
}

moe_status launch_router_topk_bf16(const moe_cfg* c, const bf16_t* x, const bf16_t* w_router, const float* offset,
                                   const float* bias, float* scores, int32_t* idx, float* w, hipStream_t st) {
  if (!router_topk_fusable(c)) return MOE_ERR_UNSUPPORTED;
  GemmParams p{};
  p.a_shared = x;
  p.w_routed = w_router;
  p.offset = offset;
  p.out_routed = scores;
  p.bias = bias;
  p.topk_idx = idx;
  p.topk_w = w;
  p.G = c->G; p.M = c->M; p.route_scale = c->route_scale;
  p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I; p.k = c->k;
  switch (c->E / 16) {
    case 1: launch_router_topk_e<1>(c, p, st); break;
    case 2: launch_router_topk_e<2>(c, p, st); break;
    case 4: launch_router_topk_e<4>(c, p, st); break;
    case 8: launch_router_topk_e<8>(c, p, st); break;
    default: launch_router_topk_e<16>(c, p, st); break;
  }
  return launch_status();
}

moe_status launch_router_bf16(const moe_cfg* c, const bf16_t* x, const bf16_t* w_router,
                              const float* offset, float* scores, hipStream_t st) {
  GemmParams p{};
  p.a_shared = x;
  p.w_routed = w_router;
  p.offset = offset;
  p.out_routed = scores;
  p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I;
  auto launch = [&](auto cfg) {
    using RT = decltype(cfg);
    const dim3 grid((unsigned)((c->T + RT::BM - 1) / RT::BM), (unsigned)((c->E + RT::BN - 1) / RT::BN));
    hipLaunchKernelGGL((gemm_bf16_kernel<kRouter, RT::WM, RT::WN, RT::MI, RT::NI, RT::BK, RT::STAGES, RT::OCC>), grid,
                       dim3(64 * RT::WM * RT::WN), 0, st, p);
  };
  switch (router_tile(c)) {
    case kRtSplit16:
      hipLaunchKernelGGL(router_splitk_kernel<16>, dim3((unsigned)((c->T + 15) / 16), (unsigned)((c->E + 15) / 16)),
                         dim3(64 * kRsWaves), 0, st, x, w_router, offset, scores, c->T, c->H, c->E);
      break;
    case kRtSplit32:
      hipLaunchKernelGGL(router_splitk_kernel<32>, dim3((unsigned)((c->T + 31) / 32), (unsigned)((c->E + 31) / 32)),
                         dim3(64 * kRsWaves), 0, st, x, w_router, offset, scores, c->T, c->H, c->E);
      break;
    case kRt256: launch(RT256{}); break;
    case kRt128: launch(RT128{}); break;
    case kRt128N: launch(RT128N{}); break;
    default: launch(RT64{}); break;
  }
  return launch_status();
}

moe_status launch_ffn_bf16(const moe_cfg* c, const bf16_t* x_perm, const int32_t* perm,
                           const int32_t* offsets, const moe_expert_weights* w, const bf16_t* x,
                           bf16_t* y_perm, bf16_t* y_shared, const moe_ffn_saved* saved, void* ws, int phase,
                           hipStream_t st) {
  const FfnLayout L(c);
  char* base = static_cast<char*>(ws);
  const int32_t* hdr = reinterpret_cast<const int32_t*>(base + L.off_hdr);
  bf16_t* hp = reinterpret_cast<bf16_t*>(base + L.off_hp);
  bf16_t* hs = reinterpret_cast<bf16_t*>(base + L.off_hs);
  moe_status s;
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_GATE_UP) {
    if ((s = launch_build_tiles(c, offsets, ws, st)) != MOE_OK) return s;
    GemmParams p{};
    p.a_routed = x_perm; p.a_shared = x;
    p.w_routed = (const bf16_t*)w->w_gate_up; p.w_shared = (const bf16_t*)w->ws_gate_up;
    p.out_routed = hp; p.out_shared = hs;
    p.tiles = reinterpret_cast<const TileDesc*>(base + L.off_t1);
    p.ntiles = hdr;
    p.perm = perm;
    if (saved) {
      p.g_routed = static_cast<bf16_t*>(saved->g); p.u_routed = static_cast<bf16_t*>(saved->u);
      p.g_shared = static_cast<bf16_t*>(saved->gs); p.u_shared = static_cast<bf16_t*>(saved->us);
    }
    p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I; p.k = c->k;
    const int64_t grid = grouped_grid(L.max1, kStripeGateUp);
    if (grid > 0) {
      const dim3 dg((unsigned)grid), bd(64 * DecGateUpTile::WM * DecGateUpTile::WN),
          bg(64 * GateUpTile::WM * GateUpTile::WN);
      if (L.dec && saved) hipLaunchKernelGGL((gemm_bf16_kernel<kGateUpSave, MOE_DEC_GU_TILE>), dg, bd, 0, st, p);
      else if (L.dec) hipLaunchKernelGGL((gemm_bf16_kernel<kGateUp, MOE_DEC_GU_TILE>), dg, bd, 0, st, p);
      else if (saved)
        hipLaunchKernelGGL((gemm_bf16_kernel<kGateUpSave, MOE_GU_TILE, MOE_GU_MI_ALT>), dg, bg, 0, st, p);
      else hipLaunchKernelGGL((gemm_bf16_kernel<kGateUp, MOE_GU_TILE, MOE_GU_MI_ALT>), dg, bg, 0, st, p);
      if ((s = launch_status()) != MOE_OK) return s;
    }
  }
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_DOWN) {
    GemmParams p{};
    p.a_routed = hp; p.a_shared = hs;
    p.w_routed = (const bf16_t*)w->w_down; p.w_shared = (const bf16_t*)w->ws_down;
    p.out_routed = y_perm; p.out_shared = y_shared;
    p.tiles = reinterpret_cast<const TileDesc*>(base + L.off_t2);
    p.ntiles = hdr + 1;
    p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I;
    const int64_t grid = grouped_grid(L.max2, kStripeDown);
    if (grid > 0) {
      if (L.dec)
        hipLaunchKernelGGL((gemm_bf16_kernel<kDown, MOE_DEC_DN_TILE>), dim3((unsigned)grid),
                           dim3(64 * DecDownTile::WM * DecDownTile::WN), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<kDown, MOE_DN_TILE>), dim3((unsigned)grid),
                           dim3(64 * DownTile::WM * DownTile::WN), 0, st, p);
      if ((s = launch_status()) != MOE_OK) return s;
    }
  }
  return MOE_OK;
}

moe_status launch_gateup_recompute_bf16(const moe_cfg* c, const bf16_t* x_perm, const bf16_t* x,
                                        const moe_expert_weights* w, const TileDesc* tiles,
                                        const int32_t* ntiles, int64_t max_tiles, bf16_t* g, bf16_t* u,
                                        bf16_t* gs, bf16_t* us, hipStream_t st) {
  GemmParams p{};
  p.a_routed = x_perm; p.a_shared = x;
  p.w_routed = (const bf16_t*)w->w_gate_up; p.w_shared = (const bf16_t*)w->ws_gate_up;
  p.g_routed = g; p.u_routed = u;
  p.g_shared = gs; p.u_shared = us;
  p.tiles = tiles;
  p.ntiles = ntiles;
  p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I; p.k = c->k;
  const int64_t grid = grouped_grid(max_tiles, kStripeGateUp);
  if (grid > 0)
    hipLaunchKernelGGL((gemm_bf16_kernel<kGateUpGU, MOE_GU_TILE, MOE_GU_MI_ALT>), dim3((unsigned)grid),
                       dim3(64 * GateUpTile::WM * GateUpTile::WN), 0, st, p);
  return launch_status();
}

}  // namespace moe
