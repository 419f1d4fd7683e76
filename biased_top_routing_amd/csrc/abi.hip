// Host side of the C ABI: configuration checks, workspace sizing, status text.
// Everything here runs before any device call, so it also works without a GPU.
#include <algorithm>

#include "common.h"
#include "bwd_layout.h"
#include "ffn_layout.h"

namespace moe {

bool gemm_dtype_ok(const moe_cfg* c) {
  if (c->act == MOE_F32 && c->wgt == MOE_F32) return true;
  if (c->act == MOE_BF16 && (c->wgt == MOE_BF16 || c->wgt == MOE_FP8_E4M3)) return true;
  return false;
}

moe_status validate_cfg(const moe_cfg* c) {
  if (!c) return MOE_ERR_NULL;
  if (!gemm_dtype_ok(c)) return MOE_ERR_UNSUPPORTED;
  if (c->bias_eq_mode != 0 && c->bias_eq_mode != 1) return MOE_ERR_UNSUPPORTED;
  if (c->T < 0 || c->H <= 0 || c->E <= 0 || c->G <= 0 || c->M <= 0 || c->k <= 0 || c->S < 0 ||
      c->I <= 0)
    return MOE_ERR_SHAPE;
  if (c->E > 512 || c->G > 64 || c->E % c->G != 0 || c->M > c->G) return MOE_ERR_SHAPE;
  const int gsz = c->E / c->G;
  if (c->k > 32 || c->k > c->M * gsz) return MOE_ERR_SHAPE;
  if (c->group_topr < 1 || c->group_topr > gsz || c->group_topr > 8) return MOE_ERR_SHAPE;
  if ((int64_t)c->T * c->k >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if ((int64_t)c->T * c->k * c->H >= ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  if (!(c->route_scale == c->route_scale)) return MOE_ERR_SHAPE;   // NaN
  // 32-bit byte offsets inside a GEMM tile (up to 257 rows of the widest operand)
  if (c->H > (1 << 20) || c->I > (1 << 20) || (int64_t)c->S * c->I > (1 << 20)) return MOE_ERR_SHAPE;
  // one buffer descriptor covers a segment's weights (all shared experts together)
  if ((int64_t)(c->S > 1 ? c->S : 1) * 2 * c->I * c->H * 2 >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  if ((int64_t)c->E * c->H * 2 >= ((int64_t)1 << 31)) return MOE_ERR_SHAPE;
  // the grouped GEMMs' tile tables and launch grids count tiles in 32 bits (tiles
  // of at least 32 rows x 64 columns, plus a ragged one per segment)
  const int64_t rows = (int64_t)c->T * (c->k + c->S);
  const int64_t widest = std::max((int64_t)c->H, (int64_t)(c->S > 1 ? c->S : 1) * c->I);
  if ((rows / 32 + c->E + 2) * (widest / 64 + 2) >= ((int64_t)1 << 30)) return MOE_ERR_SHAPE;
  if (c->act == MOE_F32) {
    if (c->H % 4 || c->I % 4) return MOE_ERR_SHAPE;
  } else if (c->wgt == MOE_BF16) {
    if (c->H % 64 || c->I % 128) return MOE_ERR_SHAPE;
  } else {  // fp8 experts: K of every GEMM at most kFp8MaxKC chunks of 128
    if (c->H % 128 || c->I % 128) return MOE_ERR_SHAPE;
    if (c->H > 128 * kFp8MaxKC || (int64_t)(c->S > 1 ? c->S : 1) * c->I > 128 * kFp8MaxKC)
      return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_workspace_bytes(const moe_cfg* cfg, int which) {
  if (validate_cfg(cfg) != MOE_OK) return 0;
  if (which == MOE_WS_ROUTE) return route_ws_bytes(cfg);
  if (which == MOE_WS_DISPATCH) return dispatch_ws_bytes(cfg);
  if (which == MOE_WS_FFN) return FfnLayout(cfg).total;
  if (which == MOE_WS_FFN_BWD) return FfnBwdLayout(cfg).total;
  if (which == MOE_WS_ROUTE_BWD) return RouteBwdLayout(cfg, 0).total;
  return 0;
}

extern "C" moe_status moe_ffn_workspace_part(const moe_cfg* cfg, int part, size_t* offset, size_t* bytes) {
  const moe_status st = validate_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!offset || !bytes) return MOE_ERR_NULL;
  const FfnLayout L(cfg);
  switch (part) {
    case MOE_WSP_H: *offset = L.off_hp; *bytes = L.off_hps - L.off_hp; break;
    case MOE_WSP_H_SCALE: *offset = L.off_hps; *bytes = L.off_hs - L.off_hps; break;
    case MOE_WSP_H_SHARED: *offset = L.off_hs; *bytes = L.off_hss - L.off_hs; break;
    case MOE_WSP_H_SHARED_SCALE: *offset = L.off_hss; *bytes = L.off_xq - L.off_hss; break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "sizes inconsistent or outside the supported range";
    case MOE_ERR_UNSUPPORTED: return "dtype combination or option not supported";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_SCRATCH: return "sizes exceed the fixed scratch of a no-allocation entry point";
  }
  return "unknown status";
}

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }
