// moe_host.cpp -- host-only entry points of the C ABI (no HIP calls): workspace sizing,
// tiling description, status strings, ABI version.  Builds with g++ as well as hipcc.
#include "moe.h"
#include "moe_plan.h"

extern "C" {

moe_status moe_workspace_size(const moe_problem *p, size_t *bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  const moe_status st = moe::validate_problem(p);
  if (st != MOE_OK) return st;
  *bytes = moe::make_layout(p).total;
  return MOE_OK;
}

moe_status moe_plan_describe(const moe_problem *p, moe_plan_info *info) {
  if (!info) return MOE_ERR_INVALID_ARGUMENT;
  const moe_status st = moe::validate_problem(p);
  if (st != MOE_OK) return st;
  const moe::Layout L = moe::make_layout(p);
  *info = moe_plan_info{};
  info->m_tile_rows = L.tiles.bm;
  info->gateup_cols = L.tiles.gu_cols;
  info->down_cols = L.tiles.dn_cols;
  info->router_k_split = L.tiles.rt_split;
  info->max_m_tiles = L.mt_routed_max;
  info->group_m = L.tiles.group_m;
  info->fp8_activations = L.tiles.aq;
  return MOE_OK;
}

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEVICE_FAULT: return "MOE_ERR_DEVICE_FAULT";
  }
  return "MOE_ERR_UNKNOWN";
}

int moe_abi_version(void) { return MOE_ABI_VERSION; }

}  // extern "C"
