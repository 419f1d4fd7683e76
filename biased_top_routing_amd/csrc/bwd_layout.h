// Workspace layouts of the backward calls (host and device agree on them).
#pragma once

#include "common.h"
#include "ffn_layout.h"

namespace moe {

// Backward GEMM tiles: 256 x 256 outputs, K slices of 64.
constexpr int kBwdBM = 256, kBwdBN = 256;

// Weight-gradient launches (one tile of an expert's dW per workgroup, K = the
// expert's rows): the n_sh shared-expert tiles (K = T, the longest) come
// first, one per workgroup id, so that they spread over all XCDs and start
// early; the n_rt routed tiles follow in runs of PW consecutive tiles dealt to
// the 8 XCDs in turn, so that the XCDs work on one expert's tiles together
// and its operand rows, missed by every XCD's L2 within a short time, come
// from the memory-side cache (against one contiguous range per XCD: dW_gate_up
// 2-3% faster with runs of 32, dW_down 3% with runs of 8).  Returns the
// workgroup's tile: [0, n_sh) shared, n_sh + L routed tile L, -1 surplus.
constexpr int kStripeDwGu = 32, kStripeDwD = 8;
__host__ __device__ inline int dw_tile_at(int b, int n_sh, int n_rt, int PW) {
  const int n_sh8 = (n_sh + 7) & ~7;   // padded to whole XCD rounds: b - n_sh8 keeps b's XCD
  if (b < n_sh8) return b < n_sh ? b : -1;
  const int r = b - n_sh8;
  const int L = xcd_run_index(r >> 3, r & 7, PW);
  return L < n_rt ? n_sh + L : -1;
}
// Workgroups of such a launch: each XCD takes ceil(n_rt / 8) + PW routed
// positions, at least the PW * ceil(n_rt / 8PW) that its runs need.
inline int64_t dw_grid(int64_t n_sh, int64_t n_rt, int PW) {
  return (int64_t)align_up((size_t)n_sh, 8) + (int64_t)align_up((size_t)n_rt, 8) + 8 * PW;
}

// moe_expert_ffn_backward: tile tables of the three row-segmented GEMMs (gate/up
// recomputation, dh, dx), the recomputed gate and up outputs g, u, the gradient
// of the gate/up outputs dgu (gate part, then up part, per expert), and h
// recomputed for the down weights' gradient.  Routed rows [T*k, .], shared
// rows [T, S * .]; all bf16.
struct FfnBwdLayout {
  int64_t P;
  int64_t max_re, max_dh, max_dx;                  // tile-table capacities
  int nt_re, nts_re, nt_dh, nts_dh, nt_dx;         // column tiles
  size_t off_hdr, off_tre, off_tdh, off_tdx;
  size_t off_g, off_u, off_gs, off_us, off_dgu, off_dgus, off_h, off_hs, total;

  explicit FfnBwdLayout(const moe_cfg* c) {
    P = pairs(c);
    const int64_t SI = (int64_t)c->S * c->I;
    nt_re = (c->I + kBNH - 1) / kBNH;
    nts_re = (int)((SI + kBNH - 1) / kBNH);
    nt_dh = (c->I + kBwdBN - 1) / kBwdBN;
    nts_dh = (int)((SI + kBwdBN - 1) / kBwdBN);
    nt_dx = (c->H + kBwdBN - 1) / kBwdBN;
    const int64_t rs_re = c->S > 0 ? (c->T + kBM1 - 1) / kBM1 : 0;
    const int64_t rs_bw = c->S > 0 ? (c->T + kBwdBM - 1) / kBwdBM : 0;
    max_re = (P / kBM1 + c->E) * nt_re + rs_re * nts_re;
    max_dh = (P / kBwdBM + c->E) * nt_dh + rs_bw * nts_dh;
    max_dx = (P / kBwdBM + c->E + rs_bw) * nt_dx;
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
    off_hdr = take(64);
    off_tre = take((size_t)max_re * sizeof(TileDesc));
    off_tdh = take((size_t)max_dh * sizeof(TileDesc));
    off_tdx = take((size_t)max_dx * sizeof(TileDesc));
    off_g = take((size_t)P * c->I * 2);
    off_u = take((size_t)P * c->I * 2);
    off_gs = take((size_t)c->T * SI * 2);
    off_us = take((size_t)c->T * SI * 2);
    off_dgu = take((size_t)P * 2 * c->I * 2);
    off_dgus = take((size_t)c->T * 2 * SI * 2);
    off_h = take((size_t)P * c->I * 2);
    off_hs = take((size_t)c->T * SI * 2);
    total = o;
  }
};

// moe_route_backward: per-chunk expert statistics of every sequence (selection
// counts and sums of the normalised affinities), the per-(sequence, expert)
// coefficient of the balance loss, dlogit in bf16 for the GEMMs, and the
// split-K partial sums of the router weights' gradient.
constexpr int kSeqChunk = 64;      // tokens per statistics chunk
constexpr int kRouterKSplit = 1024;  // token rows per split of the router-weight gradient

struct RouteBwdLayout {
  int nseq, seq_len, nchunk, nsplit;
  size_t off_cnt, off_psum, off_coef, off_dlogit, off_part, total;

  RouteBwdLayout(const moe_cfg* c, int seq) {
    seq_len = seq > 0 ? seq : (c->T > 0 ? c->T : 1);
    nseq = c->T / seq_len;
    nchunk = (seq_len + kSeqChunk - 1) / kSeqChunk;
    nsplit = (c->T + kRouterKSplit - 1) / kRouterKSplit;
    // sizes from bounds that hold for every sequence length (nseq * nchunk <=
    // T + T / 64 + 1, nseq <= T), so the workspace size does not depend on it
    const size_t chunks_max = (size_t)c->T + c->T / kSeqChunk + 1, seqs_max = (size_t)(c->T > 0 ? c->T : 1);
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
    off_cnt = take(chunks_max * c->E * 4);
    off_psum = take(chunks_max * c->E * 4);
    off_coef = take(seqs_max * c->E * 4);
    off_dlogit = take((size_t)c->T * c->E * 2);
    off_part = take((size_t)nsplit * c->E * c->H * 4);
    total = o;
  }
};

}  // namespace moe
