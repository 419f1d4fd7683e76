// Host build of the grouped GEMM launches' workgroup -> tile mappings
// (grouped_tile_at with grouped_grid, dw_tile_at with dw_grid): for every
// table size, shared-tile count and run length listed, every tile of the table
// is taken by exactly one workgroup of the launch grid, no workgroup takes a
// position outside the table, and a routed tile dealt in runs of P sits on the
// XCD (workgroup id mod 8) that its run is dealt to.  Prints "ok <cases>" or
// the first failing case.
#include <cstdio>
#include <vector>

#include "bwd_layout.h"
#include "ffn_layout.h"

using namespace moe;

static int fail(const char* what, int a, int b, int c, int d) {
  std::printf("FAIL %s %d %d %d %d\n", what, a, b, c, d);
  return 1;
}

// forward grouped launch: n_rt routed tiles then n_s shared, capacity max_tiles
static int check_grouped(int n_rt, int n_s, int P, int64_t max_tiles) {
  const int n_real = n_rt + n_s;
  const int64_t grid = grouped_grid(max_tiles, P);
  if (max_tiles == 0) return grid == 0 ? 0 : fail("grid of an empty table", n_rt, n_s, P, (int)grid);
  std::vector<int> seen(n_real, -1);
  for (int b = 0; b < grid; ++b) {
    const int L = grouped_tile_at(b, n_real, n_rt, P);
    if (L < -1 || L >= n_real) return fail("position outside the table", n_rt, n_s, P, b);
    if (L < 0) continue;
    if (seen[L] >= 0) return fail("tile taken twice", n_rt, n_s, P, L);
    seen[L] = b;
    if (P > 0 && L < n_rt && (L / P) % 8 != (b & 7)) return fail("routed run on another XCD", n_rt, n_s, P, L);
    if (L >= n_rt && (b & 7) != (L - n_rt) / ((n_s + 7) / 8)) return fail("shared share on another XCD", n_rt, n_s, P, L);
  }
  for (int L = 0; L < n_real; ++L)
    if (seen[L] < 0) return fail("tile never taken", n_rt, n_s, P, L);
  return 0;
}

// weight-gradient launch: n_sh shared tiles then n_rt routed ones
static int check_dw(int n_sh, int n_rt, int PW) {
  const int64_t grid = dw_grid(n_sh, n_rt, PW);
  std::vector<int> seen(n_sh + n_rt, -1);
  for (int b = 0; b < grid; ++b) {
    const int q = dw_tile_at(b, n_sh, n_rt, PW);
    if (q < -1 || q >= n_sh + n_rt) return fail("dW tile outside", n_sh, n_rt, PW, b);
    if (q < 0) continue;
    if (seen[q] >= 0) return fail("dW tile taken twice", n_sh, n_rt, PW, q);
    seen[q] = b;
    if (q < n_sh && q != b) return fail("dW shared tile off its workgroup", n_sh, n_rt, PW, q);
    if (q >= n_sh && ((q - n_sh) / PW) % 8 != (b & 7)) return fail("dW run on another XCD", n_sh, n_rt, PW, q);
  }
  for (int q = 0; q < n_sh + n_rt; ++q)
    if (seen[q] < 0) return fail("dW tile never taken", n_sh, n_rt, PW, q);
  return 0;
}

int main() {
  const int runs[] = {0, 1, 2, 3, 5, 8, 16, 32};
  const int shared[] = {0, 1, 7, 8, 9, 63, 100, 832, 1648};
  std::vector<int> routed;
  for (int n = 0; n <= 300; ++n) routed.push_back(n);
  for (int n : {511, 512, 513, 1000, 4097, 8191, 9000, 20003}) routed.push_back(n);
  long cases = 0;
  for (int P : runs)
    for (int n_s : shared)
      for (int n_rt : routed)
        for (int slack : {0, 1, 13}) {
          if (check_grouped(n_rt, n_s, P, (int64_t)n_rt + n_s + slack)) return 1;
          ++cases;
        }
  const int dw_runs[] = {1, 2, 8, kStripeDwD, kStripeDwGu, 64};
  const int dw_shared[] = {0, 1, 7, 8, 17, 112, 448};
  for (int PW : dw_runs)
    for (int n_sh : dw_shared)
      for (int n_rt : routed) {
        if (check_dw(n_sh, n_rt, PW)) return 1;
        ++cases;
      }
  std::printf("ok %ld\n", cases);
  return 0;
}
