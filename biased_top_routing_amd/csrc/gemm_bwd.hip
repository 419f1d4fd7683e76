// Backward GEMMs of the layer on gfx950 (v_mfma_f32_32x32x16_bf16, fp32
// accumulate).  With the expert choice fixed, the layer's gradient is plain
// calculus on y = sum_s FFN_s(x) + sum_j w_j FFN_{e_j}(x) (DeepSeek-V3
// Technical Report：中英对照解读, §2): per expert and for the shared experts
//   dh   = dY W_d                      (dY: gated output gradient rows)
//   dg   = dh * u * silu'(g),  du = dh * silu(g)     (g, u recomputed)
//   dX   = [dg du] W_gu
//   dW_gu = [dg du]^T X,   dW_d = dY^T h
// and for the router dx += dlogit W_r, dW_r = dlogit^T x.
//
// One engine, six kinds.  Tiles are 256 x 256 outputs, 8 wavefronts (2 per
// SIMD) of 128 x 64, K slices of 64 staged by direct-to-LDS loads in a 2-slice
// ring.  An operand is either K-contiguous (rows along M, K inside a row: the
// forward's layout, read with ds_read_b128) or M-contiguous (rows along K,
// M inside a row: the weights of dh / dx, and both operands of the weight
// gradients, whose K is the token rows).  An M-contiguous slice sits in LDS
// as [64 K rows][256] with its 16-byte chunks XOR-swizzled by the row, and an
// MFMA fragment (8 consecutive K of one M index per lane) is assembled by two
// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4r + q points at K row
// k0 + r, columns m0 + 4q .. m0 + 4q + 3, and lane j receives column m0 + j of
// rows k0 .. k0 + 3.
//   kDh   row-segmented (expert segments of the permuted rows; shared = all T
//         rows): A = output-gradient rows (K-contiguous, K = H), B = W_d
//         (M-contiguous); epilogue: SwiGLU backward from the recomputed g, u,
//         stores dgu and h.
//   kDx   row-segmented: A = dgu rows (K = 2I, or S*2I shared), B = W_gu; stores dX.
//   kDxR  all T rows: A = dlogit (K = E), B = W_r; stores fp32.
//   kDwGu / kDwD  K-segmented: one 256 x 256 tile of one expert's weight
//         gradient reduces over that expert's token rows (both operands
//         M-contiguous; rows past the segment's end read as zero); fp32 stores.
//   kDwR  K-segmented over fixed splits of the T tokens (fp32 partial sums,
//         reduced in order afterwards, so the result does not depend on timing).
#include "bwd_layout.h"
#include "common.h"
#include "ffn_layout.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

enum { kDh = 0, kDx = 1, kDxR = 2, kDwGu = 3, kDwD = 4, kDwR = 5 };
constexpr int dw_stripe(int kind) { return kind == kDwGu ? kStripeDwGu : kStripeDwD; }
constexpr bool kseg_kind(int kind) { return kind >= kDwGu; }

struct BwdParams {
  const bf16_t* a_routed;   // kDh: dy_perm; kDx: dgu; kDwGu: dgu; kDwD: dy_perm
  const bf16_t* a_shared;   // kDh: dy; kDx: dgu_s; kDxR, kDwR: dlogit; kDwGu: dgu_s; kDwD: dy
  const bf16_t* b_routed;   // kDh: w_down; kDx: w_gate_up; kDwGu: x_perm; kDwD: h
  const bf16_t* b_shared;   // kDh: ws_down; kDx: ws_gate_up; kDxR: w_router; kDwGu, kDwR: x; kDwD: h_s
  const bf16_t* g_routed;   // kDh: recomputed gate outputs
  const bf16_t* g_shared;
  const bf16_t* u_routed;   // kDh: recomputed up outputs
  const bf16_t* u_shared;
  void* out_routed;         // kDh: dgu; kDx: dx_perm; kDw*: fp32 gradient (kDwR: partials)
  void* out_shared;         // kDh: dgu_s; kDx: dx_shared; kDxR: dx_router; kDw*: shared gradient
  bf16_t* h_routed;         // kDh: h recomputed
  bf16_t* h_shared;
  const TileDesc* tiles;    // row-segmented kinds
  const int32_t* ntiles;
  const int32_t* offsets;   // K-segmented kinds: the experts' token-row segments
  int T, H, E, S, I;
  int ksplit;               // kDwR: token rows per split
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// XOR key of the 16-byte chunks of K row r of an M-contiguous LDS slice: the
// 8 rows (r, r+1, r+2, r+3, r+8, ..) one transposing read touches spread over
// all banks.
__device__ __forceinline__ int mc_key(int r) { return (r & 3) << 2; }

#if defined(__HIP_DEVICE_COMPILE__)
// MFMA 32x32x16 operand fragment of M block [mb, mb + 32) and K step kk from an
// M-contiguous slice [64][R]: lane l holds M index mb + l % 32, K 8 (l / 32) .. + 7.
template <int R>
__device__ __forceinline__ bf16x8_t mc_frag(const bf16_t* tile, int kk, int mb, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int krow = 16 * kk + 8 * (g >> 1) + (i >> 2);
  const int m = mb + 16 * (g & 1) + 4 * (i & 3);
  const bf16_t* p0 = tile + krow * R + (((m >> 3) ^ mc_key(krow)) << 3) + (m & 7);
  const bf16_t* p1 = p0 + 4 * R;   // K rows + 4 (same key)
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p0);
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p1);
  return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
#endif

template <int KIND, int WM, int WN, int MI, int NI, int STAGES, int BK, int OCC>
__global__ __launch_bounds__(64 * WM * WN, OCC) void gemm_bwd_kernel(BwdParams p) {
  constexpr bool KSEG = kseg_kind(KIND);
  constexpr bool A_MC = KSEG;          // A is M-contiguous exactly for the weight gradients
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int BM = WM * MI * 32, BN = WN * NI * 32;
  constexpr int CPK = BK / 8;          // 16-byte chunks per K-contiguous row of a slice
  constexpr int A_CH = BM * CPK / NT, B_CH = BN * CPK / NT, PER = A_CH + B_CH;
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(BK == 32 || BK == 64, "K slices of 32 or 64");
  static_assert(BM * CPK % NT == 0 && BN * CPK % NT == 0, "whole loads per thread");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "M-contiguous slices of at least 16 chunks per row");
#if defined(__HIP_DEVICE_COMPILE__)
  // kDx, kDh: each wavefront's (MI*32) x (NI*32) outputs are staged in LDS for
  // the epilogue (rows padded to DX_PITCH elements), over the finished ring
  constexpr int DX_PITCH = NI * 32 + 8;
  constexpr bool STAGED = KIND == kDx || KIND == kDh;
  constexpr int LDS_ELEMS = STAGED && NW * MI * 32 * DX_PITCH > STAGES * STAGE ? NW * MI * 32 * DX_PITCH
                                                                              : STAGES * STAGE;
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, kh = lane >> 5;

  // ------------------------------------------------------------ tile
  int seg = 0, m0 = 0, mvalid = 0, n0 = 0, N = 0, K = 0, split = 0;
  bool shared = false, b_split = false;
  const bf16_t* A = nullptr;
  const bf16_t* B = nullptr;
  int lda = 0, ldb = 0, a_bytes = 0, b_bytes = 0;
  if constexpr (KIND == kDxR) {
    const int ntn = (p.H + BN - 1) / BN;
    const int rt = blockIdx.x / ntn, nt = blockIdx.x % ntn;
    m0 = rt * BM;
    mvalid = min(BM, p.T - m0);
    if (mvalid <= 0) return;
    n0 = nt * BN;
    N = p.H;
    A = p.a_shared + (int64_t)m0 * p.E;
    lda = p.E;
    K = p.E;
    B = p.b_shared;
    ldb = p.H;
    b_bytes = p.E * p.H * 2;
  } else if constexpr (!KSEG) {
    const int L = grouped_tile<0>(p.ntiles);
    if (L < 0) return;
    const TileDesc d = p.tiles[L];
    seg = __builtin_amdgcn_readfirstlane(d.seg);
    m0 = __builtin_amdgcn_readfirstlane(d.row0);
    mvalid = __builtin_amdgcn_readfirstlane(d.rows);
    n0 = __builtin_amdgcn_readfirstlane(d.nt) * BN;
    shared = seg == p.E;
    if constexpr (KIND == kDh) {
      lda = p.H;
      K = p.H;
      A = (shared ? p.a_shared : p.a_routed) + (int64_t)m0 * lda;
      N = shared ? p.S * p.I : p.I;
      B = shared ? p.b_shared : p.b_routed + (int64_t)seg * p.H * p.I;
      ldb = p.I;
      b_bytes = (shared ? p.S : 1) * p.H * p.I * 2;
      b_split = shared && p.S > 1;   // column n of shared expert n / I, W_d rows at stride H * I
    } else {
      lda = (shared ? p.S : 1) * 2 * p.I;
      K = lda;
      A = (shared ? p.a_shared : p.a_routed) + (int64_t)m0 * lda;
      N = p.H;
      B = shared ? p.b_shared : p.b_routed + (int64_t)seg * 2 * p.I * p.H;
      ldb = p.H;
      b_bytes = K * p.H * 2;
    }
  } else {
    // K-segmented: one tile of one gradient; M x N and the token rows it reduces over
    int M, local, ntn;
    int64_t krow0 = 0;
    if constexpr (KIND == kDwR) {
      M = p.E;
      N = p.H;
      const int mtn = (M + BM - 1) / BM;
      ntn = (N + BN - 1) / BN;
      split = blockIdx.x / (mtn * ntn);
      local = blockIdx.x % (mtn * ntn);
      krow0 = (int64_t)split * p.ksplit;
      K = min(p.ksplit, p.T - (int)krow0);
      if (K < 0) return;
      A = p.a_shared + krow0 * p.E;
      lda = p.E;
      B = p.b_shared + krow0 * p.H;
      ldb = p.H;
    } else {
      const int Mr = KIND == kDwGu ? 2 * p.I : p.H, Nr = KIND == kDwGu ? p.H : p.I;
      const int Ms = KIND == kDwGu ? p.S * 2 * p.I : p.H, Ns = KIND == kDwGu ? p.H : p.S * p.I;
      const int mtr = (Mr + BM - 1) / BM, ntr = (Nr + BN - 1) / BN;
      const int n_sh = p.S > 0 ? ((Ms + BM - 1) / BM) * ((Ns + BN - 1) / BN) : 0;
      const int nrt = p.E * mtr * ntr;
      const int q = dw_tile_at(blockIdx.x, n_sh, nrt, dw_stripe(KIND));
      if (q < 0) return;
      if (q < n_sh) {
        shared = true;
        seg = p.E;
        M = Ms;
        N = Ns;
        ntn = (Ns + BN - 1) / BN;
        local = q;
        K = p.T;
      } else {
        const int L = q - n_sh;
        seg = L / (mtr * ntr);
        local = L % (mtr * ntr);
        M = Mr;
        N = Nr;
        ntn = ntr;
        krow0 = p.offsets[seg];
        K = p.offsets[seg + 1] - (int)krow0;
      }
      if constexpr (KIND == kDwGu) {
        lda = (shared ? p.S : 1) * 2 * p.I;
        A = (shared ? p.a_shared : p.a_routed) + krow0 * lda;
        ldb = p.H;
        B = (shared ? p.b_shared : p.b_routed) + krow0 * ldb;
      } else {
        lda = p.H;
        A = (shared ? p.a_shared : p.a_routed) + krow0 * lda;
        ldb = shared ? p.S * p.I : p.I;
        B = (shared ? p.b_shared : p.b_routed) + krow0 * ldb;
      }
    }
    m0 = (local / ntn) * BM;
    n0 = (local % ntn) * BN;
    mvalid = min(BM, M - m0);
    a_bytes = K * lda * 2;
    b_bytes = K * ldb * 2;
  }
  seg = __builtin_amdgcn_readfirstlane(seg);
  K = __builtin_amdgcn_readfirstlane(K);

  // ------------------------------------------------------------ load offsets
  // Instruction i of wave w fills LDS chunks [(i*NW + w)*64, +64) of the A (B)
  // region.  K-contiguous A: lane chunk -> (row, logical K chunk) as in the
  // forward GEMMs; rows past the tile's valid rows are pushed out of the
  // descriptor's range (the hardware then writes zeros).  M-contiguous
  // operands: lane chunk -> (K row r, logical column chunk); the K advance
  // moves the descriptor's base, whose range ends at the segment's last row.
  int a_off[A_CH], b_off[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int q = (i * NW + wave) * 64 + lane;
    if constexpr (A_MC) {
      constexpr int CPR = BM / 8;
      const int r = q / CPR, pc = q % CPR;
      a_off[i] = (r * lda + m0 + ((pc ^ mc_key(r)) << 3)) * 2;
    } else {
      const int r = q / CPK, pc = q % CPK;
      a_off[i] = ((r < mvalid ? r : mvalid + 1) * lda + (swz<CPK>(r, pc) << 3)) * 2;
    }
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    constexpr int CPR = BN / 8;
    const int q = (i * NW + wave) * 64 + lane;
    const int r = q / CPR, pc = q % CPR;
    const int col = n0 + ((pc ^ mc_key(r)) << 3);
    const int cmap = b_split ? (col / p.I) * p.H * p.I + col % p.I : col;
    b_off[i] = (r * ldb + cmap) * 2;
  }
  const __amdgpu_buffer_rsrc_t rsrc_a_kc = make_rsrc(A, A_MC ? 0 : mvalid * lda * 2);
#define MOE_ISSUE_BWD(stage_, k0_)                                                                    \
  {                                                                                                   \
    const int k0v = (k0_);                                                                            \
    bf16_t* sb = lds + (stage_) * STAGE;                                                              \
    if constexpr (A_MC) {                                                                             \
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)k0v * lda, max(0, a_bytes - k0v * lda * 2)); \
      _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                                \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(sb + (i * NW + wave) * 512), 16,  \
                                                   a_off[i], 0, 0, 0);                                \
    } else {                                                                                          \
      _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                                \
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a_kc, (lds_void_t*)(sb + (i * NW + wave) * 512), \
                                                   16, a_off[i], k0v * 2, 0, 0);                      \
    }                                                                                                 \
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)k0v * ldb, max(0, b_bytes - k0v * ldb * 2)); \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                                                  \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(sb + BM * BK + (i * NW + wave) * 512), \
                                                 16, b_off[i], 0, 0, 0);                              \
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  int a_rd[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) a_rd[mi] = wm * MI * 32 + mi * 32 + lr;
  const bool has_rows = wm * MI * 32 < mvalid;

  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) MOE_ISSUE_BWD(s, s * BK);
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_slices<PER>(min(nk - 1, kt + STAGES - 2) - kt);
    asm volatile("s_barrier" ::: "memory");
    const bf16_t* base = lds + cur * STAGE;
    const bf16_t* bbase = base + BM * BK;
    constexpr int KK = BK / 16;
    // Every transposing read of this slice is issued before the next slice's
    // direct-to-LDS loads: issued after them, the compiler makes the first one
    // wait for those loads (vmcnt(0)), which serialises loads and MFMAs.
    bf16x8_t fbs[KK][NI];
    bf16x8_t fas[A_MC ? KK : 1][MI];
    if (has_rows) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) fbs[kk][ni] = mc_frag<BN>(bbase, kk, wn * NI * 32 + ni * 32, lane);
        if constexpr (A_MC) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) fas[kk][mi] = mc_frag<BM>(base, kk, wm * MI * 32 + mi * 32, lane);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + STAGES - 1 < nk) {
      const int st = cur == 0 ? STAGES - 1 : cur - 1;
      MOE_ISSUE_BWD(st, (kt + STAGES - 1) * BK);
    }
    if (has_rows) {
      if constexpr (A_MC) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fas[kk][mi], fbs[kk][ni], acc[mi][ni], 0, 0, 0);
        }
      } else {
        // K-contiguous A: ds_read_b128 fragments, double-buffered across the k-steps
        bf16x8_t fa[2][MI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          fa[0][mi] = *reinterpret_cast<const bf16x8_t*>(base + a_rd[mi] * BK + (swz<CPK>(a_rd[mi], kh) << 3));
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int cb = kk & 1;
          if (kk + 1 < KK) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
              fa[cb ^ 1][mi] = *reinterpret_cast<const bf16x8_t*>(base + a_rd[mi] * BK +
                                                                  (swz<CPK>(a_rd[mi], 2 * (kk + 1) + kh) << 3));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cb][mi], fbs[kk][ni], acc[mi][ni], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    cur = cur == STAGES - 1 ? 0 : cur + 1;
  }
#undef MOE_ISSUE_BWD

  // ------------------------------------------------------------ epilogue
  // acc[mi][ni][r] = C[i][j], j = lane % 32, i = 8 (r / 4) + 4 (lane / 32) + r % 4.
  if constexpr (KIND == kDh) {
    // SwiGLU backward from the recomputed g, u: dg = dh u silu'(g), du = dh silu(g),
    // and h = silu(g) u.  The three outputs go out one after the other as whole
    // 128-byte row segments through LDS; du and h wait, rounded to bf16, in the
    // accumulator registers.
    static_assert(NI * 32 * 2 == 128, "a wavefront's columns are one 128-byte row segment");
    const bf16_t* G = shared ? p.g_shared : p.g_routed;
    const bf16_t* U = shared ? p.u_shared : p.u_routed;
    const int c0 = n0 + wn * NI * 32;   // first column of this wavefront (in one I block: I % 128 == 0)
    __syncthreads();   // every wavefront is done with the ring
    bf16_t* stg = lds + wave * (MI * 32 * DX_PITCH);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      // this row block's g and u: all loads issued before any is used
      float gv[16][NI], uv[16][NI];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = wm * MI * 32 + mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        const int64_t row = m0 + (i < mvalid ? i : 0);    // rows past the tile's end read row 0 (never stored)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = min(c0 + ni * 32 + lr, N - 1);
          gv[r][ni] = bf16_to_f32(G[row * N + col]);
          uv[r][ni] = bf16_to_f32(U[row * N + col]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const float v = acc[mi][ni][r], g = gv[r][ni], u = uv[r][ni];
          const float sg = gate_sigmoid(g);
          const float silu = g * sg;
          stg[(mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3)) * DX_PITCH + ni * 32 + lr] =
              f32_to_bf16(v * u * (sg + g * sg * (1.0f - sg)));
          uint32_t duh = pack_bf16x2(v * silu, silu * u);   // (du, h), kept here: an opaque
          asm volatile("" : "+v"(duh));                      // copy so that it is not recomputed later
          acc[mi][ni][r] = __uint_as_float(duh);
        }
    }
    bf16_t* dgu = static_cast<bf16_t*>(shared ? p.out_shared : p.out_routed);
    bf16_t* hh = shared ? p.h_shared : p.h_routed;
    const int64_t dcol = (c0 / p.I) * 2 * p.I + c0 % p.I;   // dg of column c0 in a row of [g | u] blocks
#pragma unroll
    for (int o = 0; o < 3; ++o) {   // 0 dg, 1 du, 2 h
      if (o > 0) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t w = __float_as_uint(acc[mi][ni][r]);
              stg[(mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3)) * DX_PITCH + ni * 32 + lr] =
                  (bf16_t)(o == 1 ? (w & 0xFFFFu) : (w >> 16));
            }
      }
      // (the wavefront reads back only what it wrote; its LDS operations complete in order)
      __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < MI * 32 / 8; ++it) {
        const int lr2 = it * 8 + (lane >> 3);
        const int i = wm * MI * 32 + lr2;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + lr2 * DX_PITCH + (lane & 7) * 8);
        if (i < mvalid && c0 < N) {
          const int64_t row = m0 + i;
          bf16_t* dst = o == 2 ? hh + row * N + c0 : dgu + row * 2 * N + dcol + (o == 1 ? p.I : 0);
          *reinterpret_cast<uint4*>(dst + (lane & 7) * 8) = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);
      __builtin_amdgcn_wave_barrier();
    }
    return;
  }
  if constexpr (KIND == kDx) {
    // dX goes out as whole 128-byte row segments, 16 bytes per lane, through LDS
    // (a lane holds single values of 16 rows)
    static_assert(NI * 32 * 2 == 128, "a wavefront's columns are one 128-byte row segment");
    __syncthreads();   // every wavefront is done with the ring
    bf16_t* stg = lds + wave * (MI * 32 * DX_PITCH);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stg[(mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3)) * DX_PITCH + ni * 32 + lr] = f32_to_bf16(acc[mi][ni][r]);
    // (the wavefront reads back only what it wrote; its LDS operations complete in order)
    __builtin_amdgcn_s_waitcnt(kLgkmWaitZero);
    __builtin_amdgcn_wave_barrier();
    bf16_t* out = static_cast<bf16_t*>(shared ? p.out_shared : p.out_routed);
    const int col = n0 + wn * NI * 32 + (lane & 7) * 8;   // N = H is a multiple of 64: whole segment or none
#pragma unroll
    for (int it = 0; it < MI * 32 / 8; ++it) {
      const int lr2 = it * 8 + (lane >> 3);
      const int i = wm * MI * 32 + lr2;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + lr2 * DX_PITCH + (lane & 7) * 8);
      if (i < mvalid && col < N) *reinterpret_cast<uint4*>(out + (m0 + i) * (int64_t)N + col) = v;
    }
    return;
  }
  // The weight gradients (45 GB of fp32 at the V3-like shape, never re-read by
  // this layer) are stored non-temporally: measured 2-5% faster than plain
  // stores, which also displace the operand panels from the L2.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = wm * MI * 32 + mi * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (i >= mvalid) continue;
      const int64_t row = m0 + i;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = n0 + wn * NI * 32 + ni * 32 + lr;
        if (col >= N) continue;
        const float v = acc[mi][ni][r];
        if constexpr (KIND == kDxR) {
          static_cast<float*>(p.out_shared)[row * N + col] = v;
        } else if constexpr (KIND == kDwGu) {
          float* o = shared ? static_cast<float*>(p.out_shared)
                            : static_cast<float*>(p.out_routed) + (int64_t)seg * 2 * p.I * p.H;
          __builtin_nontemporal_store(v, &o[row * N + col]);
        } else if constexpr (KIND == kDwD) {
          float* o = shared ? static_cast<float*>(p.out_shared) + (int64_t)(col / p.I) * p.H * p.I + col % p.I
                            : static_cast<float*>(p.out_routed) + (int64_t)seg * p.H * p.I + col;
          __builtin_nontemporal_store(v, &o[row * p.I]);
        } else {
          static_cast<float*>(p.out_routed)[(int64_t)split * p.E * p.H + row * N + col] = v;
        }
      }
    }
  }
#endif   // __HIP_DEVICE_COMPILE__
}

// dW_r = sum over the splits of the partial sums, in split order.
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int nsplit,
                                                            int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < nsplit; ++k) s += part[(int64_t)k * n + i];
  out[i] = s;
}

// dh, router: 256 x 256 tiles, 8 wavefronts, 64-deep slices in a 2-slice ring, one workgroup per CU.
#define MOE_BWD_TILE 2, 4, 4, 2, 2, 64, 1
constexpr int kBwdThreads = 64 * 2 * 4;
static_assert(2 * 4 * 32 == kBwdBM && 4 * 2 * 32 == kBwdBN, "backward tile shape");
// Expert weight gradients: the same 256 x 256 tile (measured: 256 x 128 tiles with 32-deep slices and two
// workgroups per CU, one computing while the other drains its fp32 stores, are 5-10% slower).
#ifndef MOE_BWD_WG_TILE
#define MOE_BWD_WG_TILE 2, 4, 4, 2, 2, 64, 1
#endif
template <int WM_, int WN_, int MI_, int NI_, int STAGES_, int BK_, int OCC_>
struct BwdTile {
  static constexpr int WM = WM_, WN = WN_, MI = MI_, NI = NI_, STAGES = STAGES_, BK = BK_, OCC = OCC_;
  static constexpr int BM = WM * MI * 32, BN = WN * NI * 32, THREADS = 64 * WM * WN;
};
using WgTile = BwdTile<MOE_BWD_WG_TILE>;
// dx: the same 256 x 256 tile over 16 wavefronts of 64 x 64 (4 per SIMD, as in the forward down GEMM): 2% faster
// than 8 of 128 x 64, bit-identical (dh keeps 8: its SwiGLU epilogue would spill at 128 registers).
#ifndef MOE_BWD_DX_TILE
#define MOE_BWD_DX_TILE 4, 4, 2, 2, 2, 64, 1
#endif
using DxTile = BwdTile<MOE_BWD_DX_TILE>;
static_assert(DxTile::BM == kBwdBM && DxTile::BN == kBwdBN, "dx tile shape (the tile tables use kBwdBM x kBwdBN)");

moe_status launch_ffn_bwd_bf16(const moe_cfg* c, const bf16_t* x_perm, const bf16_t* x, const int32_t* offsets,
                               const moe_expert_weights* w, const moe_ffn_saved* saved, const bf16_t* dy_perm,
                               const bf16_t* dy, bf16_t* dx_perm, bf16_t* dx_shared, const moe_expert_grads* gr,
                               void* ws, hipStream_t st) {
  const FfnBwdLayout L(c);
  char* base = static_cast<char*>(ws);
  int32_t* hdr = reinterpret_cast<int32_t*>(base + L.off_hdr);
  TileDesc* t_re = reinterpret_cast<TileDesc*>(base + L.off_tre);
  TileDesc* t_dh = reinterpret_cast<TileDesc*>(base + L.off_tdh);
  TileDesc* t_dx = reinterpret_cast<TileDesc*>(base + L.off_tdx);
  // the gate and up outputs: kept by the forward pass, or recomputed here
  bf16_t* g = saved ? static_cast<bf16_t*>(saved->g) : reinterpret_cast<bf16_t*>(base + L.off_g);
  bf16_t* u = saved ? static_cast<bf16_t*>(saved->u) : reinterpret_cast<bf16_t*>(base + L.off_u);
  bf16_t* gs = saved ? static_cast<bf16_t*>(saved->gs) : reinterpret_cast<bf16_t*>(base + L.off_gs);
  bf16_t* us = saved ? static_cast<bf16_t*>(saved->us) : reinterpret_cast<bf16_t*>(base + L.off_us);
  bf16_t* dgu = reinterpret_cast<bf16_t*>(base + L.off_dgu);
  bf16_t* dgus = reinterpret_cast<bf16_t*>(base + L.off_dgus);
  bf16_t* h = reinterpret_cast<bf16_t*>(base + L.off_h);
  bf16_t* hs = reinterpret_cast<bf16_t*>(base + L.off_hs);
  moe_status s;
  // tables: hdr[0] recompute, hdr[1] dx, hdr[2] dh
  if ((s = launch_build_tile_tables(c, offsets, kBM1, kBM1Alt, L.nt_re, L.nts_re, t_re, L.max_re, kBwdBM, 0, L.nt_dx,
                                    t_dx, L.max_dx, hdr, st)) != MOE_OK)
    return s;
  if ((s = launch_build_tile_tables(c, offsets, kBwdBM, 0, L.nt_dh, L.nts_dh, t_dh, L.max_dh, kBwdBM, 0, 1,
                                    nullptr, 0, hdr + 2, st)) != MOE_OK)
    return s;
  if (!saved && (s = launch_gateup_recompute_bf16(c, x_perm, x, w, t_re, hdr, L.max_re, g, u, gs, us, st)) != MOE_OK)
    return s;

  BwdParams p{};
  p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I;
  p.offsets = offsets;
  // dh -> dgu, h
  p.a_routed = dy_perm; p.a_shared = dy;
  p.b_routed = (const bf16_t*)w->w_down; p.b_shared = (const bf16_t*)w->ws_down;
  p.g_routed = g; p.g_shared = gs; p.u_routed = u; p.u_shared = us;
  p.out_routed = dgu; p.out_shared = dgus; p.h_routed = h; p.h_shared = hs;
  p.tiles = t_dh; p.ntiles = hdr + 2;
  hipLaunchKernelGGL((gemm_bwd_kernel<kDh, MOE_BWD_TILE>), dim3((unsigned)grouped_grid(L.max_dh, 0)),
                     dim3(kBwdThreads), 0, st, p);
  if ((s = launch_status()) != MOE_OK) return s;
  // dx
  p.a_routed = dgu; p.a_shared = dgus;
  p.b_routed = (const bf16_t*)w->w_gate_up; p.b_shared = (const bf16_t*)w->ws_gate_up;
  p.out_routed = dx_perm; p.out_shared = dx_shared;
  p.tiles = t_dx; p.ntiles = hdr + 1;
  hipLaunchKernelGGL((gemm_bwd_kernel<kDx, MOE_BWD_DX_TILE>), dim3((unsigned)grouped_grid(L.max_dx, 0)),
                     dim3(DxTile::THREADS), 0, st, p);
  if ((s = launch_status()) != MOE_OK) return s;
  // weight gradients
  auto tiles_of = [](int64_t m, int64_t n) {
    return ((m + WgTile::BM - 1) / WgTile::BM) * ((n + WgTile::BN - 1) / WgTile::BN);
  };
  const int64_t SI = (int64_t)c->S * c->I;
  p.a_routed = dgu; p.a_shared = dgus;
  p.b_routed = x_perm; p.b_shared = x;
  p.out_routed = gr->w_gate_up; p.out_shared = gr->ws_gate_up;
  {
    const int64_t n_sh = c->S > 0 ? tiles_of(2 * SI, c->H) : 0;
    const int64_t n = dw_grid(n_sh, c->E * tiles_of(2 * c->I, c->H), dw_stripe(kDwGu));
    hipLaunchKernelGGL((gemm_bwd_kernel<kDwGu, MOE_BWD_WG_TILE>), dim3((unsigned)n), dim3(WgTile::THREADS), 0, st, p);
    if ((s = launch_status()) != MOE_OK) return s;
  }
  p.a_routed = dy_perm; p.a_shared = dy;
  p.b_routed = h; p.b_shared = hs;
  p.out_routed = gr->w_down; p.out_shared = gr->ws_down;
  {
    const int64_t n_sh = c->S > 0 ? tiles_of(c->H, SI) : 0;
    const int64_t n = dw_grid(n_sh, c->E * tiles_of(c->H, c->I), dw_stripe(kDwD));
    hipLaunchKernelGGL((gemm_bwd_kernel<kDwD, MOE_BWD_WG_TILE>), dim3((unsigned)n), dim3(WgTile::THREADS), 0, st, p);
    if ((s = launch_status()) != MOE_OK) return s;
  }
  return MOE_OK;
}

moe_status launch_router_bwd_gemms(const moe_cfg* c, const bf16_t* x, const bf16_t* w_router,
                                   const bf16_t* dlogit, float* part, int nsplit, float* dw_router,
                                   float* dx_router, hipStream_t st) {
  BwdParams p{};
  p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I;
  p.ksplit = kRouterKSplit;
  p.a_shared = dlogit;
  p.b_shared = x;
  p.out_routed = part;
  const int64_t tiles = (int64_t)((c->E + kBwdBM - 1) / kBwdBM) * ((c->H + kBwdBN - 1) / kBwdBN);
  hipLaunchKernelGGL((gemm_bwd_kernel<kDwR, MOE_BWD_TILE>), dim3((unsigned)(tiles * nsplit)), dim3(kBwdThreads),
                     0, st, p);
  moe_status s;
  if ((s = launch_status()) != MOE_OK) return s;
  const int64_t n = (int64_t)c->E * c->H;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, nsplit, n,
                     dw_router);
  if ((s = launch_status()) != MOE_OK) return s;
  if (dx_router) {
    p.b_shared = w_router;
    p.out_shared = dx_router;
    const int64_t rt = (c->T + kBwdBM - 1) / kBwdBM;
    hipLaunchKernelGGL((gemm_bwd_kernel<kDxR, MOE_BWD_TILE>), dim3((unsigned)(rt * ((c->H + kBwdBN - 1) / kBwdBN))),
                       dim3(kBwdThreads), 0, st, p);
    if ((s = launch_status()) != MOE_OK) return s;
  }
  return MOE_OK;
}

}  // namespace moe
