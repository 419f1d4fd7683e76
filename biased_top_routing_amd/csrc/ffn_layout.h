// Workspace layouts of moe_dispatch and moe_expert_ffn (host + device visible sizes).
#pragma once

#include "common.h"

namespace moe {

// ---- dispatch: one wave owns a contiguous segment of kSegPairs flat pair ids
constexpr int kSegPairs = 1024;

inline int64_t dispatch_segments(const moe_cfg* c) {
  return (pairs(c) + kSegPairs - 1) / kSegPairs;
}

// The fixed scratch of moe_dispatch_noalloc: per-segment counts of at most
// this many bytes (E = 256: up to 4096 segments, 4M (token, slot) pairs).
constexpr size_t kDispatchScratchBytes = (size_t)4 << 20;

inline size_t dispatch_ws_bytes(const moe_cfg* c) {
  size_t b = (size_t)dispatch_segments(c) * c->E * sizeof(int32_t);
  return align_up(b < 256 ? 256 : b, 256);
}

// ---- expert FFN tiling shared by the tile-table builder and the GEMMs

// Tile shapes of the grouped GEMMs (compile-time choices):
// WM, WN wavefronts along tokens / weights; MI, NI MFMA 32x32 blocks per
// wavefront; BK K-depth of an LDS stage; STAGES ring depth; OCC workgroups
// per CU the kernel is built for.  Two or four wavefronts per SIMD (measured:
// a second wavefront per SIMD covers the load and barrier waits that a single
// wavefront exposes).  Gate/up tiles are 320 token rows high so that a
// routed segment of up to 640 rows (balanced loads sit near T*k/E = 512 at the
// V3-like shape) loads its weight panel twice, not three times.
#ifndef MOE_GU_TILE
#define MOE_GU_TILE 2, 4, 5, 2, 64, 2, 1
#endif
#ifndef MOE_DN_TILE
#define MOE_DN_TILE 4, 4, 2, 2, 64, 2, 1
#endif
// Router GEMM tiles (tokens x experts): 64 x 256, 128 x 256, 128 x 128 and
// 256 x 256, 8 wavefronts; the launcher picks the largest whose grid still
// covers every CU (small batches use the split-K router kernel instead)
#ifndef MOE_RT_TILE
#define MOE_RT_TILE 2, 4, 1, 2, 64, 3, 1
#endif
#define MOE_RT128_TILE 2, 4, 2, 2, 64, 3, 1
#define MOE_RT128N_TILE 2, 4, 2, 1, 64, 3, 1
#define MOE_RT256_TILE 2, 4, 4, 2, 64, 2, 1
template <int WM_, int WN_, int MI_, int NI_, int BK_, int STAGES_, int OCC_>
struct TileCfg {
  static constexpr int WM = WM_, WN = WN_, MI = MI_, NI = NI_, BK = BK_, STAGES = STAGES_, OCC = OCC_;
  static constexpr int BM = WM * MI * 32, BN = WN * NI * 32;
};
using GateUpTile = TileCfg<MOE_GU_TILE>;
using DownTile = TileCfg<MOE_DN_TILE>;
constexpr int kBM1 = GateUpTile::BM;      // token rows of a gate/up tile
// A segment's gate/up row tiles are kBM1Alt rows high instead of kBM1 when that
// takes no more tiles: fewer padded MFMA rows (e.g. 512 rows: two tiles of 256
// instead of 320 + 192), run by a kernel body with MOE_GU_MI_ALT row blocks per
// wavefront.  0 turns this off.
#ifndef MOE_GU_MI_ALT
#define MOE_GU_MI_ALT 4
#endif
constexpr int kBM1Alt = GateUpTile::WM * MOE_GU_MI_ALT * 32;
constexpr int kBM2 = DownTile::BM;        // token rows of a down tile
constexpr int kBNH = GateUpTile::BN / 2;   // h columns of a gate/up tile (as many gate as up weight rows)
constexpr int kBN2 = DownTile::BN;         // output columns of a down tile
// Small batches (at most kDecBM routed rows per expert on average, e.g. decode):
// the GEMMs only stream weights, so their tiles are 32 token rows x 256 weight
// rows with a deeper ring (more weight bytes in flight per CU).
#ifndef MOE_DEC_GU_TILE
#define MOE_DEC_GU_TILE 1, 4, 1, 2, 64, 4, 1
#endif
#ifndef MOE_DEC_DN_TILE
#define MOE_DEC_DN_TILE 1, 4, 1, 2, 64, 4, 1
#endif
using DecGateUpTile = TileCfg<MOE_DEC_GU_TILE>;
using DecDownTile = TileCfg<MOE_DEC_DN_TILE>;
constexpr int kDecBM = 32;
static_assert(DecGateUpTile::BM == kDecBM && DecDownTile::BM == kDecBM, "row tiles of the small-batch table");
constexpr int kDecBNH = DecGateUpTile::BN / 2;
constexpr int kDecBN2 = DecDownTile::BN;
static_assert(kDecBNH == kBNH, "h column tiles of both bf16 configurations (I % 128 check)");

inline bool small_batch(const moe_cfg* c) {
  return c->act == MOE_BF16 && c->wgt == MOE_BF16 && pairs(c) <= (int64_t)kDecBM * c->E;
}
// FP8 GEMMs: 320 token rows (10 row blocks of 16 per wavefront, the most that
// 256 registers hold; 4% faster down and 1% faster gate/up than 256 rows at the
// FP8 workload); 128 h columns (one 1 x 128 quantisation tile of h) per gate/up
// tile, 256 output columns per down tile, K at most kFp8MaxKC chunks of 128.
#ifndef MOE_FP8_BM
#define MOE_FP8_BM 320
#endif
constexpr int kFp8BM = MOE_FP8_BM;
constexpr int kFp8BNH = 128;
constexpr int kFp8BN2 = 256;
constexpr int kFp8MaxKC = 64;

// Row tiles per group in the tile order of a segment (see build_tiles_kernel).
#ifndef MOE_GROUP_ROW_TILES
#define MOE_GROUP_ROW_TILES 8
#endif
constexpr int kGroupRowTiles = MOE_GROUP_ROW_TILES;

// One tile of the grouped GEMMs: segment (routed expert e < E, or E = shared),
// first row in the A operand, valid rows, and the column-tile index.
struct TileDesc {
  int32_t seg, row0, rows, nt;
};

// How a grouped launch deals its routed tiles to the XCDs (workgroup id mod 8):
// 0 gives each XCD one contiguous share of the table, so an expert's tiles all
// run in one XCD's L2; P > 0 deals runs of P consecutive table entries to the
// 8 XCDs in turn, so the XCDs work on neighbouring table entries at the same
// time: an expert's column tiles then run on several XCDs together, reading its
// activation rows once from memory and the rest from the memory-side cache,
// and each run of P still shares weight panels in one L2.  Measured at the
// V3-like shapes (alternating libraries on one box): gate/up bf16 runs of 8
// 1-1.5% faster than contiguous shares (2: 1% slower, 32 or more: slower);
// FP8 runs of 2 2-5% (gate/up) and 6-8% (down) faster (1 or 8: 0-3%); the
// bf16 down GEMM is fastest with contiguous shares (runs of 2-64: 1-4% slower).
constexpr int kStripeGateUp = 8;
constexpr int kStripeDown = 0;
constexpr int kStripeFp8 = 2;

// Position j of XCD xcd in runs of P consecutive entries dealt to the 8 XCDs in turn.
__host__ __device__ inline int xcd_run_index(int j, int xcd, int P) {
  return (j / P) * (8 * P) + xcd * P + j % P;
}

// Grouped GEMM launches: one workgroup per tile of a device-built table that
// holds n_rt routed tiles followed by the shared-expert ones (n_real in all).
// Each XCD (workgroup id b mod 8) takes an equal contiguous share of the
// shared tiles first (all full; cut by count alone, the table left them to the
// last XCD, which then finished last), then its routed tiles as P says
// (above).  Returns the table position of workgroup b's tile, or -1 for a
// surplus workgroup.
__host__ __device__ inline int grouped_tile_at(int b, int n_real, int n_rt, int P) {
  const int per_s = (n_real - n_rt + 7) >> 3;
  const int xcd = b & 7, j = b >> 3;
  if (j < per_s) {
    const int L = n_rt + xcd * per_s + j;
    return L < n_real ? L : -1;
  }
  const int jr = j - per_s;
  if (P > 0) {
    const int L = xcd_run_index(jr, xcd, P);
    return L < n_rt ? L : -1;
  }
  const int per_r = (n_rt + 7) >> 3;
  const int L = xcd * per_r + jr;
  return jr < per_r && L < n_rt ? L : -1;
}

#if defined(__HIP_DEVICE_COMPILE__)
// This workgroup's table position (ntiles[0] tiles in all, ntiles[4] routed).
template <int P>
__device__ __forceinline__ int grouped_tile(const int32_t* ntiles) {
  static_assert(P >= 0, "run length");
  return grouped_tile_at(blockIdx.x, __builtin_amdgcn_readfirstlane(ntiles[0]),
                         __builtin_amdgcn_readfirstlane(ntiles[4]), P);
}
#endif

// Workgroups of a grouped launch over a table of at most max_tiles tiles, with
// the kernel's run length P: an XCD takes ceil(shared / 8) shared positions and
// ceil(routed / 8) (P = 0) or P * ceil(routed / 8P) (at most routed / 8 + P)
// routed ones, so P + 2 positions per XCD beyond max_tiles / 8 cover both.
inline int64_t grouped_grid(int64_t max_tiles, int P) {
  return max_tiles > 0 ? (int64_t)align_up((size_t)max_tiles, 8) + 8 * (P + 2) : 0;
}

struct FfnLayout {
  bool dec;                      // small-batch bf16 configuration
  int bm1, bm2;                  // token rows per tile: gate/up, down
  int bm1_alt, bm2_alt;          // rows per tile where that takes no more tiles (0: bm1 / bm2 only)
  int64_t R1, Rs1, R2, Rs2;      // routed row-tile bounds, shared row tiles
  int64_t nt1, nt1s, nt2;        // column tiles: gate/up routed, gate/up shared, down
  int64_t max1, max2;            // tile-table capacities
  size_t off_hdr, off_t1, off_t2, off_hp, off_hps, off_hs, off_hss, off_xq, off_xqs, total;
  int hbytes;                    // bytes per stored h element

  explicit FfnLayout(const moe_cfg* c) {
    const int64_t P = pairs(c);
    const bool f8 = c->wgt == MOE_FP8_E4M3;
    dec = small_batch(c);
    bm1 = f8 ? kFp8BM : dec ? kDecBM : kBM1;
    bm1_alt = f8 || dec ? 0 : kBM1Alt;
    bm2_alt = 0;   // down tiles keep one height (320/256-row tiles of 8 wavefronts measured 1-2% slower)
    bm2 = f8 ? kFp8BM : dec ? kDecBM : kBM2;
    R1 = P / bm1 + c->E;
    Rs1 = c->S > 0 ? (c->T + bm1 - 1) / bm1 : 0;
    R2 = P / bm2 + c->E;
    Rs2 = c->S > 0 ? (c->T + bm2 - 1) / bm2 : 0;
    const int bnh = f8 ? kFp8BNH : dec ? kDecBNH : kBNH, bn2 = f8 ? kFp8BN2 : dec ? kDecBN2 : kBN2;
    nt1 = (c->I + bnh - 1) / bnh;
    nt1s = ((int64_t)c->S * c->I + bnh - 1) / bnh;
    nt2 = (c->H + bn2 - 1) / bn2;
    max1 = R1 * nt1 + Rs1 * nt1s;
    max2 = (R2 + Rs2) * nt2;
    hbytes = c->wgt == MOE_FP8_E4M3 ? 1 : (int)act_bytes(c);
    const bool fp8 = c->wgt == MOE_FP8_E4M3;
    size_t o = 0;
    off_hdr = o; o = align_up(o + 64, 256);
    off_t1 = o; o = align_up(o + (size_t)max1 * sizeof(TileDesc), 256);
    off_t2 = o; o = align_up(o + (size_t)max2 * sizeof(TileDesc), 256);
    off_hp = o; o = align_up(o + (size_t)P * c->I * hbytes, 256);
    off_hps = o; o = align_up(o + (fp8 ? (size_t)P * (c->I / 128) * 4 : 0), 256);
    off_hs = o; o = align_up(o + (size_t)c->T * c->S * c->I * hbytes, 256);
    off_hss = o; o = align_up(o + (fp8 ? (size_t)c->T * c->S * (c->I / 128) * 4 : 0), 256);
    off_xq = o; o = align_up(o + (fp8 ? (size_t)c->T * c->H : 0), 256);
    off_xqs = o; o = align_up(o + (fp8 ? (size_t)c->T * (c->H / 128) * 4 : 0), 256);
    total = o;
  }
};

}  // namespace moe
