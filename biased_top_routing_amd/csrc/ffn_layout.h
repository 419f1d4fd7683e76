// Workspace layouts of moe_dispatch and moe_expert_ffn (host + device visible sizes).
#pragma once

#include "common.h"

namespace moe {

// ---- dispatch: one wave owns a contiguous segment of kSegPairs flat pair ids
constexpr int kSegPairs = 1024;

inline int64_t dispatch_segments(const moe_cfg* c) {
  return (pairs(c) + kSegPairs - 1) / kSegPairs;
}

inline size_t dispatch_ws_bytes(const moe_cfg* c) {
  size_t b = (size_t)dispatch_segments(c) * c->E * sizeof(int32_t);
  return align_up(b < 256 ? 256 : b, 256);
}

// ---- expert FFN tiling shared by the tile-table builder and the GEMMs
constexpr int kBM = 128;        // rows of a GEMM tile (tokens)
constexpr int kBNH = 128;       // h columns of a gate/up tile (128 gate + 128 up weight rows)
constexpr int kBN2 = 256;       // output columns of a down tile

// One tile of the grouped GEMMs: segment (routed expert e < E, or E = shared),
// first row in the A operand, valid rows, and the column-tile index.
struct TileDesc {
  int32_t seg, row0, rows, nt;
};

struct FfnLayout {
  int64_t R, Rs;                 // routed row-tile bound, shared row tiles
  int64_t nt1, nt1s, nt2;        // column tiles: gate/up routed, gate/up shared, down
  int64_t max1, max2;            // tile-table capacities
  size_t off_hdr, off_t1, off_t2, off_hp, off_hps, off_hs, off_hss, off_xq, off_xqs, total;
  int hbytes;                    // bytes per stored h element

  explicit FfnLayout(const moe_cfg* c) {
    const int64_t P = pairs(c);
    R = P / kBM + c->E;
    Rs = c->S > 0 ? (c->T + kBM - 1) / kBM : 0;
    nt1 = c->I / kBNH;
    nt1s = (int64_t)c->S * c->I / kBNH;
    nt2 = (c->H + kBN2 - 1) / kBN2;
    max1 = R * nt1 + Rs * nt1s;
    max2 = (R + Rs) * nt2;
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
