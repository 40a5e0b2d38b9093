// Argument checks of attn_fwd, as pure C++ (no HIP calls), so a host-only
// build can exercise them under sanitizers.
#pragma once

#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "tile_plan.hpp"

namespace attn {

// Query-tile rows per work-group; the launch geometry and the limits below use it.
constexpr int32_t kBlockM = 128;

// Checks that need no pointer: sizes, scale, mask mode and parameters.
inline attn_status_t check_problem(int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                   int32_t mask_mode, const void* params) {
  if (B <= 0 || H <= 0 || N <= 0) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (mask_mode != ATTN_MASK_NONE && mask_mode != ATTN_MASK_CAUSAL && mask_mode != ATTN_MASK_NA2D)
    return ATTN_ERR_INVALID_ARG;
  if (mask_mode != ATTN_MASK_NA2D && params != nullptr) return ATTN_ERR_INVALID_ARG;
  if (mask_mode == ATTN_MASK_NA2D && params == nullptr) return ATTN_ERR_INVALID_ARG;
  if (d != 32 && d != 64) return ATTN_ERR_UNSUPPORTED;
  // 32-bit launch geometry and token indices: N and the work-group count stay below 2^31
  if (N > INT32_MAX - 2 * kBlockM) return ATTN_ERR_UNSUPPORTED;
  if (B > INT32_MAX / H) return ATTN_ERR_UNSUPPORTED;
  const int64_t bh = B * H;
  const int64_t n_wg = bh * cdiv(N, kBlockM);
  if (n_wg > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  if (bh > INT64_MAX / N / d) return ATTN_ERR_UNSUPPORTED;
  // one head's rows are addressed through a 32-bit buffer record count
  if (N * d * 2 > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  if (mask_mode == ATTN_MASK_NA2D) {
    const attn_na2d_params_t* p = static_cast<const attn_na2d_params_t*>(params);
    if (p->grid_h < 1 || p->grid_w < 1) return ATTN_ERR_PARAMS;
    if ((int64_t)p->grid_h * p->grid_w != N) return ATTN_ERR_PARAMS;
    if (p->kernel_h < 1 || p->kernel_h % 2 == 0 || p->kernel_h > p->grid_h) return ATTN_ERR_PARAMS;
    if (p->kernel_w < 1 || p->kernel_w % 2 == 0 || p->kernel_w > p->grid_w) return ATTN_ERR_PARAMS;
    if ((p->wrap_h != 0 && p->wrap_h != 1) || (p->wrap_w != 0 && p->wrap_w != 1)) return ATTN_ERR_PARAMS;
    if (p->dil_h != 1 || p->dil_w != 1) return ATTN_ERR_PARAMS;
  }
  return ATTN_OK;
}

inline bool overlaps(uintptr_t a, uintptr_t b, uintptr_t bytes) { return a < b + bytes && b < a + bytes; }

// Pointer checks: non-null, 16-byte aligned, output disjoint from the inputs.
inline attn_status_t check_pointers(const void* q, const void* k, const void* v, const void* o,
                                    int64_t B, int64_t H, int64_t N, int64_t d) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  const uintptr_t uq = (uintptr_t)q, uk = (uintptr_t)k, uv = (uintptr_t)v, uo = (uintptr_t)o;
  if ((uq | uk | uv | uo) & 15u) return ATTN_ERR_ALIGNMENT;
  const uintptr_t bytes = (uintptr_t)(B * H * N * d) * 2u;
  if (overlaps(uo, uq, bytes) || overlaps(uo, uk, bytes) || overlaps(uo, uv, bytes)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Workspace checks of attn_fwd_ws: present, large enough, 256-byte aligned,
// disjoint from the tensors.
inline attn_status_t check_workspace(const void* ws, uint64_t ws_bytes, int64_t need, const void* q, const void* k,
                                     const void* v, const void* o, int64_t B, int64_t H, int64_t N, int64_t d) {
  if (ws == nullptr || ws_bytes < (uint64_t)need) return ATTN_ERR_WORKSPACE;
  const uintptr_t uw = (uintptr_t)ws;
  if (uw & 255u) return ATTN_ERR_WORKSPACE;
  const uintptr_t bytes = (uintptr_t)(B * H * N * d) * 2u;
  for (const void* t : {q, k, v, o}) {
    const uintptr_t ut = (uintptr_t)t;
    if (uw < ut + bytes && ut < uw + (uintptr_t)need) return ATTN_ERR_WORKSPACE;
  }
  return ATTN_OK;
}

inline NaGeom na_geom(const attn_na2d_params_t& p) {
  return NaGeom{p.grid_h, p.grid_w, p.kernel_h, p.kernel_w, p.kernel_h / 2, p.kernel_w / 2, p.wrap_h, p.wrap_w};
}

}  // namespace attn
