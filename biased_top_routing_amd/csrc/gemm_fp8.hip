// FP8 (E4M3) expert GEMMs of the layer on gfx950 with fine-grained scaling:
// one fp32 scale per 1 x 128 tile of an activation row (x and h) and per
// 128 x 128 block of a weight, E4M3 for every FP8 tensor, and the low-precision
// products promoted to fp32 accumulation every 128 elements of K (qwbw.cn
// essay, FP8 part of the training-infrastructure section; DeepSeek-V3
// Technical Report：中英对照解读, §6 FP8 Training).
//
// On gfx950 one v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-wide K
// chunk, so the promotion is: P = A_c B_c^T of the chunk from a zero
// accumulator, then acc += P * sa[row, c] * sw[block, c] in fp32 registers.
// The MFMA takes the weight fragment as its first operand, so a lane's four
// results are four adjacent weight columns of one token row: they share one
// scale product sa * sw, and the epilogue stores them as one word.
// (The FP8 MFMA's own sum of a chunk's products is not exact for codes of a
// wide exponent range; starting every chunk from zero keeps that error from
// growing with K.)
//   gate/up  h = silu(X W_g^T) * (X W_u^T), quantised per 1 x 128 tile of h in
//            the epilogue (codes + one fp32 scale per tile)
//   down     Y = h W_d^T, stored as bf16
//
// Tiling: a workgroup of WM x WN wavefronts computes a (WM*MI*16) x (WN*NI*16)
// tile; each wavefront owns MI x NI MFMA 16 x 16 blocks.  K advances 128 bytes
// per slice through a ring of LDS stages filled by direct-to-LDS buffer loads
// (16-byte chunks, XOR swizzle per row); the tile's activation scales of the
// slice ride in the same stage (one 4-byte load per lane; wavefronts without
// scale rows issue an equal load that the range check drops, so every
// wavefront waits on the same count).  Weight-block scales of all chunks are
// staged once per tile.  The gate/up tile's 256 weight rows are the 128 gate
// rows and the 128 up rows of 128 h columns, so SwiGLU and the 1 x 128
// quantisation of h stay inside the workgroup.  All LDS is one array: with
// several LDS objects the compiler makes every LDS read wait for the
// direct-to-LDS loads in flight.
#include "common.h"
#include "ffn_layout.h"
#include "kernels.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4v_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

enum { kGateUp8 = 1, kDown8 = 2 };

// FP8 tile: 2 x 4 wavefronts of 10 x 4 blocks (160 x 64 each) -> 320 x 256
constexpr int kWM8 = 2, kWN8 = 4, kMI8 = kFp8BM / (kWM8 * 16), kNI8 = 4;
static_assert(kWM8 * kMI8 * 16 == kFp8BM, "row tiles of the fp8 tile table");
static_assert(kWN8 * kNI8 * 16 == 2 * kFp8BNH && kWN8 * kNI8 * 16 == kFp8BN2, "column tiles");

struct Fp8Params {
  const fp8_t* a_routed;    // gate/up: x_perm codes [P,H]; down: h codes [P,I]
  const float* sa_routed;   // their 1 x 128 scales
  const fp8_t* a_shared;    // gate/up: x codes [T,H]; down: h_shared codes [T,S*I]
  const float* sa_shared;
  const fp8_t* w_routed;    // gate/up: w_gate_up; down: w_down (codes)
  const float* sw_routed;   // their 128 x 128 block scales
  const fp8_t* w_shared;
  const float* sw_shared;
  void* out_routed;         // gate/up: h codes; down: y_perm (bf16)
  float* out_routed_scale;  // gate/up: h scales
  void* out_shared;         // gate/up: h_shared codes; down: y_shared (bf16)
  float* out_shared_scale;
  const TileDesc* tiles;
  const int32_t* ntiles;
  const int32_t* perm;      // gate/up: non-null -> routed rows gathered from a_shared / sa_shared
  int T, H, E, S, I, k;
};

__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

template <int N>
constexpr int vm_wait_imm() {
  return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vm_wait_imm<N>());
}

// Waits until at most n slices' loads (PER each) of this wave are outstanding.
template <int PER>
__device__ __forceinline__ void wait_slices(int n) {
  if (n <= 0) wait_vm<0>();
  else if (n == 1) wait_vm<PER>();
  else wait_vm<2 * PER>();
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
#endif

// The 32 K bytes of lane group g in an LDS row: its two 16-byte chunks sit at
// swizzled positions that depend only on the row's low four bits, so every
// fragment a lane reads (rows l16 + 16 j) uses the same two byte offsets lo, hi.
__device__ __forceinline__ i32x8_t frag(const uint8_t* rowp, int lo, int hi) {
  const i32x4v_t a = *reinterpret_cast<const i32x4v_t*>(rowp + lo);
  const i32x4v_t b = *reinterpret_cast<const i32x4v_t*>(rowp + hi);
  return i32x8_t{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

// SB = 1: every slice's loads carry the tile's activation scales of that chunk
// (one 4-byte load per tile row).  SB = 4 (K a multiple of 4 chunks, 2-stage
// ring): each scale-loading wavefront brings its 64 rows' scales of 4 chunks
// at once (16 bytes per lane) into a 2-group scale buffer, once every 4 slices,
// so a slice issues a quarter as many scale requests; the scales themselves,
// and so every output bit, are the same.
template <int MODE, int WM, int WN, int MI, int NI, int STAGES, int SB>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_fp8_kernel(Fp8Params p) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int BM = WM * MI * 16, BN = WN * NI * 16;
  constexpr int BK = 128, CPR = BK / 16;
  constexpr int A_CH = BM * CPR / NT, B_CH = BN * CPR / NT;
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "whole loads per thread");
  constexpr int SA_W = BM / 64;                       // wavefronts that load activation scales
  static_assert(BM % 64 == 0 && SA_W <= NW, "64 scale rows per loading wavefront");
  constexpr int PER = A_CH + B_CH + 1;                // loads per thread per slice
  constexpr bool BATCH = SB == 4;
  static_assert(SB == 1 || (SB == 4 && STAGES == 2), "scale groups of 4 chunks need the 2-stage ring");
  static_assert(MODE != kGateUp8 || BN == 256, "a gate/up tile is one 1 x 128 tile of h");
  static_assert(MODE != kDown8 || (128 % (NI * 16) == 0), "a wavefront's columns in one weight block");
  // LDS layout (bytes): STAGES x [A rows | B rows | sa[BM] | dummy scale rows]
  // (SB = 4: STAGES x [A rows | B rows], then the scale groups sg[2][BM][4]),
  // then sw[2][kFp8MaxKC], then red[BM][WN] (SB = 4: also the target of the
  // slices' dropped scale loads, which write zeros there before the epilogue
  // uses it)
  constexpr int SA_OFF = (BM + BN) * BK;
  constexpr int DUMMY_OFF = SA_OFF + BM * 4;
  constexpr int STAGE = BATCH ? SA_OFF : DUMMY_OFF + (NW - SA_W) * 256;
  static_assert(STAGE % 16 == 0, "stage alignment");
  constexpr int SG_OFF = STAGES * STAGE;
  constexpr int SW_OFF = SG_OFF + (BATCH ? 2 * BM * 16 : 0);
  constexpr int RED_OFF = SW_OFF + 2 * kFp8MaxKC * 4;
  static_assert(!BATCH || BM * WN * 4 >= NW * 256, "dropped scale loads fit in red");
  constexpr int SA_STRIDE = BATCH ? 4 : 1;            // floats per row of the slice's scales
  // down epilogue: each wavefront stages its (MI*16) x (NI*16) bf16 outputs in LDS
  // (rows padded to STG_PITCH bytes against bank conflicts) over the finished ring
  constexpr int STG_PITCH = NI * 16 * 2 + 16;
  // row blocks staged per round (the whole wavefront tile when it fits in 144 KB)
  constexpr int STG_MI = NW * MI * 16 * STG_PITCH <= 147456 ? MI : MI / 2;
  static_assert(MI % STG_MI == 0, "whole staging rounds");
  constexpr int STG_BYTES = MODE == kDown8 ? NW * STG_MI * 16 * STG_PITCH : 0;
  constexpr int LDS_BYTES = RED_OFF + BM * WN * 4 > STG_BYTES ? RED_OFF + BM * WN * 4 : STG_BYTES;
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  float* sw_lds = reinterpret_cast<float*>(lds + SW_OFF);
  float* red = reinterpret_cast<float*>(lds + RED_OFF);

  // (the wavefront index is uniform: kept in an SGPR, so are the load choices below)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, g = lane >> 4;

  // ------------------------------------------------------------ which tile
  const int L = grouped_tile<kStripeFp8>(p.ntiles);
  if (L < 0) return;
  const TileDesc d = p.tiles[L];
  const int seg = __builtin_amdgcn_readfirstlane(d.seg);
  const int row0 = __builtin_amdgcn_readfirstlane(d.row0);
  const int rows = __builtin_amdgcn_readfirstlane(d.rows);
  const int nt = __builtin_amdgcn_readfirstlane(d.nt);
  const bool shared = seg == p.E;
  // Routed gate/up rows gathered from the quantised x: row row0 + r of the
  // expert-sorted order is token perm[row0 + r] / k (codes and scales).
  const bool gather = MODE == kGateUp8 && !shared && p.perm != nullptr;

  // ------------------------------------------------------------ operands
  const int lda = MODE == kDown8 ? (shared ? p.S * p.I : p.I) : p.H;   // = K
  const int KC = lda / 128;
  const int64_t a_base = gather ? 0 : (int64_t)row0;
  const fp8_t* A = (shared || gather ? p.a_shared : p.a_routed) + a_base * lda;
  const float* SA = (shared || gather ? p.sa_shared : p.sa_routed) + a_base * KC;
  const int a_rows = gather ? p.T : rows;   // rows covered by the A and scale descriptors
  const fp8_t* W;
  int ldw, w_bytes, ncols;
  if constexpr (MODE == kGateUp8) {
    W = shared ? p.w_shared : p.w_routed + (int64_t)seg * 2 * p.I * p.H;
    ldw = p.H;
    w_bytes = (shared ? p.S : 1) * 2 * p.I * p.H;
    ncols = shared ? p.S * p.I : p.I;
  } else {
    W = shared ? p.w_shared : p.w_routed + (int64_t)seg * p.H * p.I;
    ldw = p.I;
    w_bytes = (shared ? p.S : 1) * p.H * p.I;
    ncols = p.H;
  }

  // ------------------------------------------------------------ weight scales -> LDS
  // [2][KC]: gate/up: the gate block and the up block of this tile's 128 h
  // columns; down: the tile's two 128-column output blocks
  if (tid < 2 * KC) {
    const int h = tid / KC, c = tid % KC;
    float v;
    if constexpr (MODE == kGateUp8) {
      const int hc = nt * 128;                           // first h column (one expert, one block)
      const int wrow = (hc / p.I) * 2 * p.I + (h ? p.I : 0) + hc % p.I;
      const float* base = shared ? p.sw_shared : p.sw_routed + (int64_t)seg * (2 * p.I / 128) * (p.H / 128);
      v = base[(wrow / 128) * (p.H / 128) + c];
    } else {
      const int J = min(nt * 2 + h, p.H / 128 - 1);
      if (shared) {
        const int ic = p.I / 128, s = c / ic, cl = c % ic;
        v = p.sw_shared[((int64_t)s * (p.H / 128) + J) * ic + cl];
      } else {
        v = p.sw_routed[((int64_t)seg * (p.H / 128) + J) * (p.I / 128) + c];
      }
    }
    sw_lds[h * kFp8MaxKC + c] = v;
  }

  // ------------------------------------------------------------ load offsets
  // Token rows past the valid ones get offsets outside the A (and scale)
  // descriptors: the range check drops them without a memory request.
  int a_off[A_CH], b_off[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int q = (i * NW + wave) * 64 + lane, r = q / CPR, pc = q % CPR;
    int src = r < rows ? r : a_rows + 1;
    if constexpr (MODE == kGateUp8)
      if (gather && r < rows) src = p.perm[row0 + r] / p.k;
    a_off[i] = src * lda + swz8(r, pc) * 16;
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int q = (i * NW + wave) * 64 + lane, r = q / CPR, pc = q % CPR;
    int wrow;
    if constexpr (MODE == kGateUp8) {
      const bool up = r >= BN / 2;
      const int c = min(nt * (BN / 2) + (up ? r - BN / 2 : r), ncols - 1);
      wrow = (c / p.I) * 2 * p.I + (up ? p.I : 0) + c % p.I;
    } else {
      wrow = min(nt * BN + r, ncols - 1);
    }
    b_off[i] = wrow * ldw + swz8(r, pc) * 16;
  }
  const int sa_row = wave * 64 + lane;                 // scale row of this lane (SA_W waves)
  int sa_src = (wave < SA_W && sa_row < rows) ? sa_row : a_rows + 1;
  if constexpr (MODE == kGateUp8)
    if (gather && wave < SA_W && sa_row < rows) sa_src = p.perm[row0 + sa_row] / p.k;
  const int sa_off = sa_src * KC * 4;
  const int sa_dst = wave < SA_W ? SA_OFF + wave * 256 : DUMMY_OFF + (wave - SA_W) * 256;
  const int sa_drop = (a_rows + 1) * KC * 4;           // SB = 4: past the scale descriptor (dropped)
  const __amdgpu_buffer_rsrc_t rsrc_a = rsrc_of(A, a_rows * lda);
  const __amdgpu_buffer_rsrc_t rsrc_w = rsrc_of(W, w_bytes);
  const __amdgpu_buffer_rsrc_t rsrc_s = rsrc_of(SA, a_rows * KC * 4);
  const int64_t seg_kstride = (int64_t)p.H * p.I;   // down, shared: next expert's W_d every I of K
  typedef __attribute__((address_space(3))) void lds_void_t;
#define MOE_ISSUE8(stage_, kc_)                                                                      \
  {                                                                                                  \
    const int kcv = (kc_), k0v = kcv * BK;                                                           \
    const int wk = MODE == kDown8 ? (int)((k0v / p.I) * seg_kstride) + (k0v % p.I) : k0v;            \
    uint8_t* sb = lds + (stage_) * STAGE;                                                            \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                                 \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_void_t*)(sb + (i * NW + wave) * 1024), \
                                                 16, a_off[i], k0v, 0, 0);                          \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                                                 \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                    \
            rsrc_w, (lds_void_t*)(sb + BM * BK + (i * NW + wave) * 1024), 16, b_off[i], wk, 0, 0);   \
    if constexpr (!BATCH) {                                                                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_s, (lds_void_t*)(sb + sa_dst), 4, sa_off, kcv * 4, \
                                               0, 0);                                                \
    } else {                                                                                         \
      /* group G = (kc + 3) / 4 of chunks [4G, 4G + 4): its quarter from wavefront */                 \
      /* w = kc mod 4 (and 4 with 0), so slices 4G-3 .. 4G bring the whole group */                  \
      const int grp = (kcv + 3) >> 2;                                                                \
      if (wave < SA_W && (wave & 3) == (kcv & 3) && 4 * grp < KC)                                    \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                    \
            rsrc_s, (lds_void_t*)(lds + SG_OFF + (grp & 1) * BM * 16 + wave * 1024), 16, sa_off,     \
            grp * 16, 0, 0);                                                                         \
      else                                                                                           \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_s, (lds_void_t*)(lds + RED_OFF + wave * 256), 4, \
                                                 sa_drop, 0, 0, 0);                                  \
    }                                                                                                \
  }

  const int nk = KC;
  // SB = 4: scale group 0 before the ring (the first slice's wait covers it)
  if constexpr (BATCH)
    if (wave < SA_W)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_s, (lds_void_t*)(lds + SG_OFF + wave * 1024), 16, sa_off, 0,
                                               0, 0);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) MOE_ISSUE8(s, s);
  // the weight-scale stores above are complete before any wavefront reads them
  __syncthreads();

  f32x4_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LDS rows of this lane's operands; lane group g supplies K bytes [32g, 32g+32)
  const int arow0 = wm * MI * 16 + l16;
  int b_rd[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int brow;
    if constexpr (MODE == kGateUp8) {
      // blocks [0, NI/2): gate rows of h columns wn*NI/2*16 + ...; [NI/2, NI): the matching up rows
      constexpr int HALF = NI / 2;
      brow = (ni < HALF ? 0 : BN / 2) + wn * HALF * 16 + (ni % HALF) * 16;
    } else {
      brow = wn * NI * 16 + ni * 16;
    }
    b_rd[ni] = brow + l16;
  }
  const int c_lo = swz8(l16, 2 * g) * 16, c_hi = swz8(l16, 2 * g + 1) * 16;
  // this lane's accumulators: token row arow0 + 16 mi, weight columns 4g + r of each 16-column block
  const int wsel = MODE == kDown8 ? (wn * NI * 16) / 128 : 0;   // down: output block of this wavefront
  const bool has_rows = wm * MI * 16 < rows;

  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_slices<PER>(min(nk - 1, kt + STAGES - 2) - kt);
    asm volatile("s_barrier" ::: "memory");
    if (kt + STAGES - 1 < nk) {
      const int st = cur == 0 ? STAGES - 1 : cur - 1;
      MOE_ISSUE8(st, kt + STAGES - 1);
    }
    if (has_rows) {
      const uint8_t* base = lds + cur * STAGE;
      // this slice's scale of each tile row (SB = 4: entry kt mod 4 of group kt / 4)
      const float* sa_st = BATCH ? reinterpret_cast<const float*>(lds + SG_OFF) + ((kt >> 2) & 1) * BM * 4 + (kt & 3)
                                 : reinterpret_cast<const float*>(base + SA_OFF);
      const float w0 = sw_lds[wsel * kFp8MaxKC + kt];
      const float w1 = sw_lds[kFp8MaxKC + kt];
      i32x8_t fb[NI];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) fb[ni] = frag(base + BM * BK + b_rd[ni] * BK, c_lo, c_hi);
      // row blocks one at a time (short live ranges); the next block's operand
      // and scale reads are issued before this block's MFMAs, and the previous
      // block's chunk products are promoted (VALU) under this block's MFMAs
      const uint8_t* pa = base + arow0 * BK;   // this lane's A row in block 0; block mi is 16 mi rows further
      const float* psa = sa_st + arow0 * SA_STRIDE;
      i32x8_t fa = frag(pa, c_lo, c_hi);
      float sa = psa[0];
      f32x4_t prev[NI];
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        i32x8_t fa_n;
        float sa_n = 0.f;
        if (mi + 1 < MI) {
          fa_n = frag(pa + (mi + 1) * 16 * BK, c_lo, c_hi);
          sa_n = psa[(mi + 1) * 16 * SA_STRIDE];
        }
        __builtin_amdgcn_sched_barrier(0);
        const float s0 = sa * w0, s1 = sa * w1;
        f32x4_t part[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          part[ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[ni], fa, z, 0, 0, 0, 0, 0, 0);
          if (mi > 0) {
            const float sp = MODE == kGateUp8 && ni >= NI / 2 ? p1 : p0;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mi - 1][ni][r] = fmaf(prev[ni][r], sp, acc[mi - 1][ni][r]);
          }
        }
        // one MFMA, then the previous block's 4 promotion FMAs of that column block
        if (mi > 0) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) prev[ni] = part[ni];
        p0 = s0;
        p1 = s1;
        if (mi + 1 < MI) {
          fa = fa_n;
          sa = sa_n;
        }
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const float sp = MODE == kGateUp8 && ni >= NI / 2 ? p1 : p0;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[MI - 1][ni][r] = fmaf(prev[ni][r], sp, acc[MI - 1][ni][r]);
      }
    }
    cur = cur == STAGES - 1 ? 0 : cur + 1;
  }
#undef MOE_ISSUE8

  // ------------------------------------------------------------ epilogue
  // acc[mi][ni][r] holds C[i][j] with i = arow0 + 16 mi (token row), j = 16 ni + 4 (lane / 16) + r
  if constexpr (MODE == kGateUp8) {
    constexpr int HALF = NI / 2;
    // per row: SwiGLU in registers, amax over this wavefront's HALF*16 columns
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      float m = 0.f;
#pragma unroll
      for (int b = 0; b < HALF; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = acc[mi][b][r], uv = acc[mi][b + HALF][r];
          const float h = gv * gate_sigmoid(gv) * uv;
          acc[mi][b][r] = h;     // h replaces the gate accumulator
          m = fmaxf(m, fabsf(h));
        }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (g == 0) red[(arow0 + mi * 16) * WN + wn] = m;
    }
    __syncthreads();
    fp8_t* out = static_cast<fp8_t*>(shared ? p.out_shared : p.out_routed);
    float* out_s = shared ? p.out_shared_scale : p.out_routed_scale;
    const int ntile = ncols / 128;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int i = arow0 + mi * 16;
      if (i >= rows) continue;
      float amax = red[i * WN];
#pragma unroll
      for (int w2 = 1; w2 < WN; ++w2) amax = fmaxf(amax, red[i * WN + w2]);
      const float sc = amax == 0.f ? 1.0f : __fdiv_rn(amax, 448.0f);
      const float y = __fdiv_rn(1.0f, sc);
      const int64_t row = row0 + i;
#pragma unroll
      for (int b = 0; b < HALF; ++b) {
        // four adjacent h columns; ncols is a multiple of 128, so all four are in range or none
        const int col = nt * 128 + wn * HALF * 16 + b * 16 + 4 * g;
        if (col < ncols)
          *reinterpret_cast<uint32_t*>(out + row * ncols + col) =
              e4m3x4(div_by_scale(acc[mi][b][0], sc, y), div_by_scale(acc[mi][b][1], sc, y),
                     div_by_scale(acc[mi][b][2], sc, y), div_by_scale(acc[mi][b][3], sc, y));
      }
      if (wn == 0 && g == 0) out_s[row * ntile + nt] = sc;
    }
  } else {
    // A lane holds 4 adjacent columns of a row (8 bytes); the stores go out as
    // whole 128-byte row segments instead: the wavefront's outputs pass through
    // LDS and each lane then stores 16 bytes, 8 lanes per row.  (Stored straight
    // from the accumulators, in 32-byte pieces per row, the down GEMM spent ~20%
    // of its time in the epilogue.)
    static_assert(NI * 16 * 2 == 128, "a wavefront's columns are one 128-byte row segment");
    __syncthreads();   // every wavefront is done with the ring
    uint8_t* stg = lds + wave * (STG_MI * 16 * STG_PITCH);
    bf16_t* out = static_cast<bf16_t*>(shared ? p.out_shared : p.out_routed);
    const int col = nt * BN + wn * NI * 16 + (lane & 7) * 8;   // ncols is a multiple of 128: the segment is whole or absent
#pragma unroll
    for (int m0 = 0; m0 < MI; m0 += STG_MI) {
#pragma unroll
      for (int mi = m0; mi < m0 + STG_MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          *reinterpret_cast<uint2*>(stg + ((mi - m0) * 16 + l16) * STG_PITCH + (ni * 16 + 4 * g) * 2) =
              uint2{pack_bf16x2(acc[mi][ni][0], acc[mi][ni][1]), pack_bf16x2(acc[mi][ni][2], acc[mi][ni][3])};
      // (the wavefront reads back only what it wrote; its LDS operations complete in order)
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < STG_MI * 16 / 8; ++it) {
        const int lr = it * 8 + (lane >> 3);
        const int i = wm * MI * 16 + m0 * 16 + lr;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + lr * STG_PITCH + (lane & 7) * 16);
        if (i < rows && col < ncols) *reinterpret_cast<uint4*>(out + (row0 + i) * (int64_t)ncols + col) = v;
      }
      // (the next round's stage writes come after these reads in this wavefront's LDS order)
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
    }
  }
#endif
}

}  // namespace

moe_status launch_ffn_fp8(const moe_cfg* c, const fp8_t* x_perm, const float* x_perm_scale,
                          const int32_t* perm, const int32_t* offsets, const moe_expert_weights* w,
                          const bf16_t* x, bf16_t* y_perm, bf16_t* y_shared, void* ws, int phase,
                          hipStream_t st) {
  const FfnLayout L(c);
  char* base = static_cast<char*>(ws);
  const int32_t* hdr = reinterpret_cast<const int32_t*>(base + L.off_hdr);
  fp8_t* hp = reinterpret_cast<fp8_t*>(base + L.off_hp);
  float* hps = reinterpret_cast<float*>(base + L.off_hps);
  fp8_t* hs = reinterpret_cast<fp8_t*>(base + L.off_hs);
  float* hss = reinterpret_cast<float*>(base + L.off_hss);
  fp8_t* xq = reinterpret_cast<fp8_t*>(base + L.off_xq);
  float* xqs = reinterpret_cast<float*>(base + L.off_xqs);
  constexpr int kThreads8 = 64 * kWM8 * kWN8;
  moe_status s;
  Fp8Params p{};
  p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I; p.k = c->k;
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_GATE_UP) {
    if ((s = launch_build_tiles(c, offsets, ws, st)) != MOE_OK) return s;
    // x once in E4M3 (1 x 128 scales): the shared experts' operand, and the
    // routed one when its rows are gathered
    if ((c->S > 0 || perm) && (s = launch_quantize_rows(x, c->T, c->H, xq, xqs, st)) != MOE_OK) return s;
    p.perm = perm;
    p.a_routed = x_perm; p.sa_routed = x_perm_scale;
    p.a_shared = xq; p.sa_shared = xqs;
    p.w_routed = (const fp8_t*)w->w_gate_up; p.sw_routed = w->w_gate_up_scale;
    p.w_shared = (const fp8_t*)w->ws_gate_up; p.sw_shared = w->ws_gate_up_scale;
    p.out_routed = hp; p.out_routed_scale = hps;
    p.out_shared = hs; p.out_shared_scale = hss;
    p.tiles = reinterpret_cast<const TileDesc*>(base + L.off_t1);
    p.ntiles = hdr;
    const int64_t grid = grouped_grid(L.max1, kStripeFp8);
    if (grid > 0) {
      if ((c->H / 128) % 4 == 0)   // K = H in whole groups of 4 chunks
        hipLaunchKernelGGL((gemm_fp8_kernel<kGateUp8, kWM8, kWN8, kMI8, kNI8, 2, 4>), dim3((unsigned)grid),
                           dim3(kThreads8), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_fp8_kernel<kGateUp8, kWM8, kWN8, kMI8, kNI8, 2, 1>), dim3((unsigned)grid),
                           dim3(kThreads8), 0, st, p);
      if ((s = launch_status()) != MOE_OK) return s;
    }
  }
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_DOWN) {
    p.perm = nullptr;
    p.a_routed = hp; p.sa_routed = hps;
    p.a_shared = hs; p.sa_shared = hss;
    p.w_routed = (const fp8_t*)w->w_down; p.sw_routed = w->w_down_scale;
    p.w_shared = (const fp8_t*)w->ws_down; p.sw_shared = w->ws_down_scale;
    p.out_routed = y_perm; p.out_routed_scale = nullptr;
    p.out_shared = y_shared; p.out_shared_scale = nullptr;
    p.tiles = reinterpret_cast<const TileDesc*>(base + L.off_t2);
    p.ntiles = hdr + 1;
    const int64_t grid = grouped_grid(L.max2, kStripeFp8);
    if (grid > 0) {
      if ((c->I / 128) % 4 == 0)   // K = I (routed) and S * I (shared) in whole groups of 4 chunks
        hipLaunchKernelGGL((gemm_fp8_kernel<kDown8, kWM8, kWN8, kMI8, kNI8, 2, 4>), dim3((unsigned)grid),
                           dim3(kThreads8), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_fp8_kernel<kDown8, kWM8, kWN8, kMI8, kNI8, 2, 1>), dim3((unsigned)grid),
                           dim3(kThreads8), 0, st, p);
      if ((s = launch_status()) != MOE_OK) return s;
    }
  }
  return MOE_OK;
}

}  // namespace moe
