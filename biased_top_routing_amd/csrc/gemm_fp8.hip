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
//   gate/up  h = silu(X W_g^T) * (X W_u^T), quantised per 1 x 128 tile of h in
//            the epilogue (codes + one fp32 scale per tile)
//   down     Y = h W_d^T, stored as bf16
//
// Tiling: a 512-thread workgroup (8 wavefronts, 2 x 4) computes a 128 x 256
// tile; each wavefront owns 4 x 4 MFMA 16 x 16 blocks (64 x 64).  K advances
// 128 bytes per slice through a ring of LDS stages filled by direct-to-LDS
// buffer loads (16-byte chunks, XOR swizzle per row).  The tile's activation
// scales (all K chunks) and weight scales are staged in LDS once per tile.
// The gate/up tile's 256 weight rows are the 128 gate rows and the 128 up rows
// of 128 h columns, so SwiGLU and the 1 x 128 quantisation of h stay inside
// the workgroup.  Tile tables and the XCD-aware ordering are those of the bf16
// GEMMs.
#include "common.h"
#include "ffn_layout.h"
#include "kernels.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

enum { kGateUp8 = 1, kDown8 = 2 };

constexpr int kWM = 2, kWN = 4;           // wavefront grid
constexpr int kMI = 4, kNI = 4;           // 16 x 16 blocks per wavefront
constexpr int kTM = kWM * kMI * 16;       // 128 token rows
constexpr int kTN = kWN * kNI * 16;       // 256 weight rows
constexpr int kBK = 128;                  // K bytes per slice = one scale chunk
constexpr int kCPR = kBK / 16;            // 16-byte chunks per LDS row
constexpr int kThreads = kWM * kWN * 64;  // 512
constexpr int kACh = kTM * kCPR / kThreads;   // direct-to-LDS loads per thread per slice
constexpr int kBCh = kTN * kCPR / kThreads;
constexpr int kPer = kACh + kBCh;
constexpr int kStage = (kTM + kTN) * kBK;     // bytes per LDS stage
static_assert(kTM == kFp8BM, "row tiles of the tile table");
static_assert(kTN / 2 == kFp8BNH && kTN == kFp8BN2, "column tiles of the fp8 tile tables");

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
  int T, H, E, S, I;
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

__device__ __forceinline__ void wait_slices(int n) {
  if (n <= 0) wait_vm<0>();
  else if (n == 1) wait_vm<kPer>();
  else wait_vm<2 * kPer>();
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

template <int MODE, int STAGES>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(Fp8Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(16))) uint8_t lds[STAGES * kStage];
  __shared__ __attribute__((aligned(16))) float sa_lds[kTM * kFp8MaxKC];   // [row][chunk]
  __shared__ float sw_lds[2 * kFp8MaxKC];                                  // [half][chunk]
  __shared__ float red[kTM][kWN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int l16 = lane & 15, g = lane >> 4;

  // ------------------------------------------------------------ which tile
  const int n_real = __builtin_amdgcn_readfirstlane(*p.ntiles);
  const int per = (n_real + 7) >> 3;
  const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
  if (jj >= per) return;
  const int L = xcd * per + jj;
  if (L >= n_real) return;
  const TileDesc d = p.tiles[L];
  const int seg = __builtin_amdgcn_readfirstlane(d.seg);
  const int row0 = __builtin_amdgcn_readfirstlane(d.row0);
  const int rows = __builtin_amdgcn_readfirstlane(d.rows);
  const int nt = __builtin_amdgcn_readfirstlane(d.nt);
  const bool shared = seg == p.E;

  // ------------------------------------------------------------ operands
  const int lda = MODE == kDown8 ? (shared ? p.S * p.I : p.I) : p.H;   // = K
  const int K = lda, KC = K / 128;
  const fp8_t* A = (shared ? p.a_shared : p.a_routed) + (int64_t)row0 * lda;
  const float* SA = (shared ? p.sa_shared : p.sa_routed) + (int64_t)row0 * KC;
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

  // ------------------------------------------------------------ scales -> LDS
  // activation scales of the tile's rows, all chunks: rows*KC contiguous floats
  {
    const int n = rows * KC;
    for (int i = tid; i < kTM * KC; i += kThreads) sa_lds[i] = i < n ? SA[i] : 0.f;
  }
  // weight scales: [2][KC]; gate/up: gate block, up block; down: the tile's two
  // 128-column output blocks
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
  int a_off[kACh], b_off[kBCh];
#pragma unroll
  for (int i = 0; i < kACh; ++i) {
    const int q = (i * (kThreads / 64) + wave) * 64 + lane, r = q / kCPR, pc = q % kCPR;
    // rows past the valid ones: offset outside the A descriptor (dropped, no request)
    a_off[i] = (r < rows ? r : rows + 1) * lda + swz8(r, pc) * 16;
  }
#pragma unroll
  for (int i = 0; i < kBCh; ++i) {
    const int q = (i * (kThreads / 64) + wave) * 64 + lane, r = q / kCPR, pc = q % kCPR;
    int wrow;
    if constexpr (MODE == kGateUp8) {
      const bool up = r >= kTN / 2;
      const int c = min(nt * (kTN / 2) + (up ? r - kTN / 2 : r), ncols - 1);
      wrow = (c / p.I) * 2 * p.I + (up ? p.I : 0) + c % p.I;
    } else {
      wrow = min(nt * kTN + r, ncols - 1);
    }
    b_off[i] = wrow * ldw + swz8(r, pc) * 16;
  }
  const __amdgpu_buffer_rsrc_t rsrc_a = rsrc_of(A, rows * lda);
  const __amdgpu_buffer_rsrc_t rsrc_w = rsrc_of(W, w_bytes);
  const int64_t seg_kstride = (int64_t)p.H * p.I;   // down, shared: next expert's W_d every I of K
  typedef __attribute__((address_space(3))) void lds_void_t;
#define MOE_ISSUE8(stage_, k0_)                                                                     \
  {                                                                                                 \
    const int k0v = (k0_);                                                                          \
    const int wk = MODE == kDown8 ? (int)((k0v / p.I) * seg_kstride) + (k0v % p.I) : k0v;           \
    uint8_t* sb = lds + (stage_) * kStage;                                                          \
    _Pragma("unroll") for (int i = 0; i < kACh; ++i)                                                \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                   \
            rsrc_a, (lds_void_t*)(sb + (i * (kThreads / 64) + wave) * 1024), 16, a_off[i], k0v, 0, 0); \
    _Pragma("unroll") for (int i = 0; i < kBCh; ++i)                                                \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                   \
            rsrc_w, (lds_void_t*)(sb + kTM * kBK + (i * (kThreads / 64) + wave) * 1024), 16,        \
            b_off[i], wk, 0, 0);                                                                    \
  }

  const int nk = KC;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) MOE_ISSUE8(s, s * kBK);
  // the scale stores above must be complete before any wavefront reads them
  // (this also waits for the first stage, which slice 0 waits for anyway)
  __syncthreads();

  f32x4_t acc[kMI][kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LDS rows of this lane's operands; lane group g supplies K bytes [32g, 32g+32)
  int a_rd[kMI], b_rd[kNI];
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) a_rd[mi] = wm * kMI * 16 + mi * 16 + l16;
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    int brow;
    if constexpr (MODE == kGateUp8) {
      // blocks 0,1: gate rows of h columns wn*32 + [0,32); blocks 2,3: the matching up rows
      brow = (ni < 2 ? 0 : kTN / 2) + wn * 32 + (ni & 1) * 16;
    } else {
      brow = wn * kNI * 16 + ni * 16;
    }
    b_rd[ni] = brow + l16;
  }
  // rows of this lane's accumulators: 4g + r inside each 16-row block
  const int srow0 = wm * kMI * 16 + 4 * g;
  const int wsel = MODE == kDown8 ? (wn >> 1) : 0;   // down: output block of this wavefront

  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_slices(min(nk - 1, kt + STAGES - 2) - kt);
    asm volatile("s_barrier" ::: "memory");
    // All LDS reads of this slice come before the next slice's loads are
    // issued: an LDS read placed after a direct-to-LDS load makes the compiler
    // wait for that load (it cannot tell the stages apart).
    const uint8_t* base = lds + cur * kStage;
    i32x8_t fa[kMI], fb[kNI];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      const uint8_t* rp = base + a_rd[mi] * kBK;
      const int4 lo = *reinterpret_cast<const int4*>(rp + swz8(a_rd[mi], 2 * g) * 16);
      const int4 hi = *reinterpret_cast<const int4*>(rp + swz8(a_rd[mi], 2 * g + 1) * 16);
      fa[mi] = i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const uint8_t* rp = base + kTM * kBK + b_rd[ni] * kBK;
      const int4 lo = *reinterpret_cast<const int4*>(rp + swz8(b_rd[ni], 2 * g) * 16);
      const int4 hi = *reinterpret_cast<const int4*>(rp + swz8(b_rd[ni], 2 * g + 1) * 16);
      fb[ni] = i32x8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    // combined scales of this chunk for the lane's 16 rows (x2 weight halves for gate/up)
    float s0[kMI][4], s1[kMI][4];
    const float w0 = sw_lds[wsel * kFp8MaxKC + kt];
    const float w1 = sw_lds[kFp8MaxKC + kt];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = sa_lds[(srow0 + mi * 16 + r) * KC + kt];
        s0[mi][r] = a * w0;
        s1[mi][r] = a * w1;
      }
    if (kt + STAGES - 1 < nk) {
      const int st = cur == 0 ? STAGES - 1 : cur - 1;
      MOE_ISSUE8(st, (kt + STAGES - 1) * kBK);
    }
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[mi], fb[ni], z, 0, 0, 0, 0, 0, 0);
        const bool second = MODE == kGateUp8 && ni >= 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] = fmaf(part[r], second ? s1[mi][r] : s0[mi][r], acc[mi][ni][r]);
      }
    cur = cur == STAGES - 1 ? 0 : cur + 1;
  }
#undef MOE_ISSUE8

  // ------------------------------------------------------------ epilogue
  // acc[mi][ni][r] holds C[i][j] with j = lane % 16, i = 4 * (lane / 16) + r
  if constexpr (MODE == kGateUp8) {
    float h[kMI][4][2];
    float pmax[kMI][4];
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const float gv = acc[mi][b][r], uv = acc[mi][b + 2][r];
          h[mi][r][b] = gv / (1.0f + expf(-gv)) * uv;
          m = fmaxf(m, fabsf(h[mi][r][b]));
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        pmax[mi][r] = m;
      }
    if (l16 == 0) {
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[srow0 + mi * 16 + r][wn] = pmax[mi][r];
    }
    __syncthreads();
    fp8_t* out = static_cast<fp8_t*>(shared ? p.out_shared : p.out_routed);
    float* out_s = shared ? p.out_shared_scale : p.out_routed_scale;
    const int ntile = ncols / 128;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = srow0 + mi * 16 + r;
        if (i >= rows) continue;
        const float amax = fmaxf(fmaxf(red[i][0], red[i][1]), fmaxf(red[i][2], red[i][3]));
        const float sc = amax == 0.f ? 1.0f : __fdiv_rn(amax, 448.0f);
        const int64_t row = row0 + i;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int col = nt * 128 + wn * 32 + b * 16 + l16;
          if (col < ncols) out[row * ncols + col] = f32_to_e4m3(__fdiv_rn(h[mi][r][b], sc));
        }
        if (wn == 0 && l16 == 0) out_s[row * ntile + nt] = sc;
      }
  } else {
    bf16_t* out = static_cast<bf16_t*>(shared ? p.out_shared : p.out_routed);
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = srow0 + mi * 16 + r;
        if (i >= rows) continue;
        const int64_t row = row0 + i;
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni) {
          const int col = nt * kTN + wn * kNI * 16 + ni * 16 + l16;
          if (col < ncols) out[row * ncols + col] = f32_to_bf16(acc[mi][ni][r]);
        }
      }
  }
#endif
}

}  // namespace

moe_status launch_ffn_fp8(const moe_cfg* c, const fp8_t* x_perm, const float* x_perm_scale,
                          const int32_t* offsets, const moe_expert_weights* w, const bf16_t* x,
                          bf16_t* y_perm, bf16_t* y_shared, void* ws, int phase, hipStream_t st) {
  const FfnLayout L(c);
  char* base = static_cast<char*>(ws);
  const int32_t* hdr = reinterpret_cast<const int32_t*>(base + L.off_hdr);
  fp8_t* hp = reinterpret_cast<fp8_t*>(base + L.off_hp);
  float* hps = reinterpret_cast<float*>(base + L.off_hps);
  fp8_t* hs = reinterpret_cast<fp8_t*>(base + L.off_hs);
  float* hss = reinterpret_cast<float*>(base + L.off_hss);
  fp8_t* xq = reinterpret_cast<fp8_t*>(base + L.off_xq);
  float* xqs = reinterpret_cast<float*>(base + L.off_xqs);
  moe_status s;
  Fp8Params p{};
  p.T = c->T; p.H = c->H; p.E = c->E; p.S = c->S; p.I = c->I;
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_GATE_UP) {
    if ((s = launch_build_tiles(c, offsets, ws, st)) != MOE_OK) return s;
    if (c->S > 0 && (s = launch_quantize_rows(x, c->T, c->H, xq, xqs, st)) != MOE_OK) return s;
    p.a_routed = x_perm; p.sa_routed = x_perm_scale;
    p.a_shared = xq; p.sa_shared = xqs;
    p.w_routed = (const fp8_t*)w->w_gate_up; p.sw_routed = w->w_gate_up_scale;
    p.w_shared = (const fp8_t*)w->ws_gate_up; p.sw_shared = w->ws_gate_up_scale;
    p.out_routed = hp; p.out_routed_scale = hps;
    p.out_shared = hs; p.out_shared_scale = hss;
    p.tiles = reinterpret_cast<const TileDesc*>(base + L.off_t1);
    p.ntiles = hdr;
    const int64_t grid = align_up((size_t)L.max1, 8);
    if (grid > 0) {
      hipLaunchKernelGGL((gemm_fp8_kernel<kGateUp8, 2>), dim3((unsigned)grid), dim3(kThreads), 0, st, p);
      if ((s = launch_status()) != MOE_OK) return s;
    }
  }
  if (phase == MOE_FFN_ALL || phase == MOE_FFN_DOWN) {
    p.a_routed = hp; p.sa_routed = hps;
    p.a_shared = hs; p.sa_shared = hss;
    p.w_routed = (const fp8_t*)w->w_down; p.sw_routed = w->w_down_scale;
    p.w_shared = (const fp8_t*)w->ws_down; p.sw_shared = w->ws_down_scale;
    p.out_routed = y_perm; p.out_routed_scale = nullptr;
    p.out_shared = y_shared; p.out_shared_scale = nullptr;
    p.tiles = reinterpret_cast<const TileDesc*>(base + L.off_t2);
    p.ntiles = hdr + 1;
    const int64_t grid = align_up((size_t)L.max2, 8);
    if (grid > 0) {
      hipLaunchKernelGGL((gemm_fp8_kernel<kDown8, 2>), dim3((unsigned)grid), dim3(kThreads), 0, st, p);
      if ((s = launch_status()) != MOE_OK) return s;
    }
  }
  return MOE_OK;
}

}  // namespace moe
