// The C ABI of libattn: argument checks, launch geometry, error mapping.
// The operation and its contract are documented in include/attn.h.
#include <hip/hip_runtime_api.h>
#include <math.h>

#include <atomic>

#include "attn.h"
#include "launch.hpp"
#include "tile_plan.hpp"
#include "validate.hpp"

extern "C" {

attn_status_t attn_fwd_check(int64_t B, int64_t H, int64_t N, int64_t d, float scale, int32_t mask_mode,
                             const void* params) {
  return attn::check_problem(B, H, N, d, scale, mask_mode, params);
}

}  // extern "C"

namespace {

// CU count of the current device, cached per device.
attn_status_t device_cus(int32_t* cus) {
  constexpr int kDevices = 64;
  static std::atomic<int32_t> cache[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev >= 0 && dev < kDevices) {
    const int32_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return ATTN_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return ATTN_ERR_HIP;
  *cus = n;
  if (dev >= 0 && dev < kDevices) cache[dev].store(n, std::memory_order_relaxed);
  return ATTN_OK;
}

attn::SplitPlan plan_for(int64_t B, int64_t H, int64_t N, int32_t mask_mode, int32_t cus) {
  const int64_t n_tiles = B * H * attn::cdiv(N, attn::kBlockM);
  return attn::split_plan(mask_mode, n_tiles, (int32_t)attn::cdiv(N, attn::tile_keys()), cus);
}

attn_status_t run_fwd(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N, int64_t d,
                      float scale, int32_t mask_mode, const void* params, const attn::SplitPlan* split,
                      void* workspace, void* stream) {
  attn::KernelArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.N = (int32_t)N;
  a.BH = (int32_t)(B * H);
  a.n_qtiles = (int32_t)attn::cdiv(N, attn::kBlockM);
  a.n_kvtiles = (int32_t)attn::cdiv(N, attn::tile_keys());
  // exp(x) = 2^(x log2 e): the kernel works in base 2 with the scale folded in
  a.c = (float)(fabs((double)scale) * 1.4426950408889634);
  a.q_sign = scale < 0.f ? 0x80008000u : 0u;
  if (mask_mode == ATTN_MASK_NA2D) {
    a.na = attn::na_geom(*static_cast<const attn_na2d_params_t*>(params));
    a.na_inv_w = 1.0f / (float)a.na.grid_w;
    a.na_phases = (a.na.grid_w % 32 == 0 && a.na.grid_w <= 128) ? a.na.grid_w / 32 : 0;
  }
  int32_t n_wg = a.BH * a.n_qtiles, rem = 0;
  if (split != nullptr && split->rem > 0) {
    a.ws_parts = static_cast<float*>(workspace);
    a.split_full = split->full;
    a.split_parts = split->parts;
    n_wg = split->groups();
    rem = split->rem;
  }
  const hipError_t e = attn::launch_fwd(a, (int32_t)d, mask_mode, n_wg, rem, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                       int64_t d, float scale, int32_t mask_mode, const void* params, void* stream) {
  attn_status_t st = attn::check_problem(B, H, N, d, scale, mask_mode, params);
  if (st != ATTN_OK) return st;
  st = attn::check_pointers(q, k, v, o, B, H, N, d);
  if (st != ATTN_OK) return st;
  return run_fwd(q, k, v, o, B, H, N, d, scale, mask_mode, params, nullptr, nullptr, stream);
}

attn_status_t attn_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int32_t mask_mode,
                                      const void* params, uint64_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  attn_status_t st = attn::check_problem(B, H, N, d, 1.0f, mask_mode, params);
  if (st != ATTN_OK) return st;
  int32_t cus = 0;
  st = device_cus(&cus);
  if (st != ATTN_OK) return st;
  *bytes = (uint64_t)attn::split_workspace_bytes(plan_for(B, H, N, mask_mode, cus), d);
  return ATTN_OK;
}

attn_status_t attn_fwd_ws(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                          int64_t d, float scale, int32_t mask_mode, const void* params, void* workspace,
                          uint64_t workspace_bytes, void* stream) {
  attn_status_t st = attn::check_problem(B, H, N, d, scale, mask_mode, params);
  if (st != ATTN_OK) return st;
  st = attn::check_pointers(q, k, v, o, B, H, N, d);
  if (st != ATTN_OK) return st;
  int32_t cus = 0;
  st = device_cus(&cus);
  if (st != ATTN_OK) return st;
  const attn::SplitPlan plan = plan_for(B, H, N, mask_mode, cus);
  const int64_t need = attn::split_workspace_bytes(plan, d);
  if (need > 0) {
    st = attn::check_workspace(workspace, workspace_bytes, need, q, k, v, o, B, H, N, d);
    if (st != ATTN_OK) return st;
  }
  return run_fwd(q, k, v, o, B, H, N, d, scale, mask_mode, params, &plan, workspace, stream);
}

const char* attn_status_string(int32_t status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size, non-finite scale, "
                                      "unknown mask mode, misplaced params, or output overlapping an input)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported problem (head size must be 32 or 64; sizes must fit 32-bit "
                                      "launch geometry)";
    case ATTN_ERR_PARAMS: return "inconsistent 2D neighbourhood parameters (grid_h*grid_w must equal N; "
                                 "kernels odd and within the grid; wrap 0 or 1; dilation 1)";
    case ATTN_ERR_ALIGNMENT: return "q, k, v and o must be 16-byte aligned";
    case ATTN_ERR_HIP: return "HIP runtime error (no device, or a failed query or launch)";
    case ATTN_ERR_WORKSPACE: return "workspace missing, too small, not 256-byte aligned, or overlapping q, k, v or o";
    default: return "unknown status";
  }
}

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
