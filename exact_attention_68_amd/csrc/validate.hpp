// Argument checks of the C ABI, as pure C++ (no HIP calls), so a host-only
// build can exercise them under sanitizers.
#pragma once

#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "tile_plan.hpp"

namespace attn {

// Query-tile rows per work-group; the launch geometry and the limits below use it.
constexpr int32_t kBlockM = 128;

// One attention problem as the entry points receive it. attn_fwd and attn_fwd_ws
// are the case Nq = Nkv = N with no lse output.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // optional
  int64_t B, H, Nq, Nkv, d;
  float scale;
  int32_t mask;
  const void* params;
};

// One neighbourhood axis: odd kernel, dilation >= 1, and a window that fits the
// axis (wrapped: (kernel - 1) * dil < len, so every key counts once; clamped:
// kernel * dil <= len, so every sub-grid of congruent cells holds a whole window).
inline bool na_axis_valid(int64_t len, int64_t kernel, int64_t wrap, int64_t dil) {
  if (len < 1 || kernel < 1 || kernel % 2 == 0 || dil < 1) return false;
  if (wrap != 0 && wrap != 1) return false;
  return wrap ? (kernel - 1) * dil < len : kernel * dil <= len;
}

// The geometry of a neighbourhood mask in kernel form (a 2D grid is one plane).
inline NaGeom na_geom(int32_t mask, const void* params) {
  if (mask == ATTN_MASK_NA3D) {
    const attn_na3d_params_t& p = *static_cast<const attn_na3d_params_t*>(params);
    return NaGeom{p.grid_h, p.grid_w, p.kernel_h, p.kernel_w, p.kernel_h / 2, p.kernel_w / 2, p.wrap_h, p.wrap_w,
                  p.dil_h, p.dil_w, p.grid_d, p.kernel_d, p.kernel_d / 2, p.wrap_d, p.dil_d};
  }
  const attn_na2d_params_t& p = *static_cast<const attn_na2d_params_t*>(params);
  return NaGeom{p.grid_h, p.grid_w, p.kernel_h, p.kernel_w, p.kernel_h / 2, p.kernel_w / 2, p.wrap_h, p.wrap_w,
                p.dil_h, p.dil_w, 1, 1, 0, 0, 1};
}

inline bool is_na_mode(int32_t mask) { return mask == ATTN_MASK_NA2D || mask == ATTN_MASK_NA3D; }

// Checks that need no pointer: sizes, scale, mask mode and parameters.
inline attn_status_t check_problem(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale,
                                   int32_t mask_mode, const void* params) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (mask_mode != ATTN_MASK_NONE && mask_mode != ATTN_MASK_CAUSAL && !is_na_mode(mask_mode))
    return ATTN_ERR_INVALID_ARG;
  if (!is_na_mode(mask_mode) && params != nullptr) return ATTN_ERR_INVALID_ARG;
  if (is_na_mode(mask_mode) && params == nullptr) return ATTN_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // 32-bit launch geometry and token indices: Nq, Nkv and the work-group count stay below 2^31
  for (int64_t n : {Nq, Nkv})
    if (n > INT32_MAX - 2 * kBlockM) return ATTN_ERR_UNSUPPORTED;
  if (B > INT32_MAX / H) return ATTN_ERR_UNSUPPORTED;
  const int64_t bh = B * H;
  const int64_t n_wg = bh * cdiv(Nq, kBlockM);
  if (n_wg > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  for (int64_t n : {Nq, Nkv})
    if (bh > INT64_MAX / n / d) return ATTN_ERR_UNSUPPORTED;
  // one head's rows are addressed through a 32-bit buffer record count
  if (Nkv * d * 2 > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  if (is_na_mode(mask_mode)) {
    int64_t dims[3], kern[3], wrap[3], dil[3];
    if (mask_mode == ATTN_MASK_NA3D) {
      const attn_na3d_params_t* p = static_cast<const attn_na3d_params_t*>(params);
      const int64_t a[4][3] = {{p->grid_d, p->grid_h, p->grid_w}, {p->kernel_d, p->kernel_h, p->kernel_w},
                               {p->wrap_d, p->wrap_h, p->wrap_w}, {p->dil_d, p->dil_h, p->dil_w}};
      for (int i = 0; i < 3; ++i) dims[i] = a[0][i], kern[i] = a[1][i], wrap[i] = a[2][i], dil[i] = a[3][i];
    } else {
      const attn_na2d_params_t* p = static_cast<const attn_na2d_params_t*>(params);
      const int64_t a[4][3] = {{1, p->grid_h, p->grid_w}, {1, p->kernel_h, p->kernel_w},
                               {0, p->wrap_h, p->wrap_w}, {1, p->dil_h, p->dil_w}};
      for (int i = 0; i < 3; ++i) dims[i] = a[0][i], kern[i] = a[1][i], wrap[i] = a[2][i], dil[i] = a[3][i];
    }
    for (int i = 0; i < 3; ++i)
      if (dims[i] < 1 || dims[i] > INT32_MAX) return ATTN_ERR_PARAMS;
    if (dims[0] * dims[1] * dims[2] != Nq || Nq != Nkv) return ATTN_ERR_PARAMS;
    for (int i = 0; i < 3; ++i)
      if (!na_axis_valid(dims[i], kern[i], wrap[i], dil[i])) return ATTN_ERR_PARAMS;
  }
  return ATTN_OK;
}

inline attn_status_t check_problem(const Problem& p) {
  return check_problem(p.B, p.H, p.Nq, p.Nkv, p.d, p.scale, p.mask, p.params);
}

inline bool overlaps(uintptr_t a, uintptr_t a_bytes, uintptr_t b, uintptr_t b_bytes) {
  return a < b + b_bytes && b < a + a_bytes;
}

// Pointer checks: non-null tensors, 16-byte aligned (lse: 4-byte), outputs disjoint
// from the inputs and from each other.
inline attn_status_t check_pointers(const Problem& p) {
  if (!p.q || !p.k || !p.v || !p.o) return ATTN_ERR_INVALID_ARG;
  const uintptr_t uq = (uintptr_t)p.q, uk = (uintptr_t)p.k, uv = (uintptr_t)p.v, uo = (uintptr_t)p.o;
  const uintptr_t ul = (uintptr_t)p.lse;
  if ((uq | uk | uv | uo) & 15u) return ATTN_ERR_ALIGNMENT;
  if (ul & 3u) return ATTN_ERR_ALIGNMENT;
  const uintptr_t q_bytes = (uintptr_t)(p.B * p.H * p.Nq * p.d) * 2u;
  const uintptr_t kv_bytes = (uintptr_t)(p.B * p.H * p.Nkv * p.d) * 2u;
  if (overlaps(uo, q_bytes, uq, q_bytes) || overlaps(uo, q_bytes, uk, kv_bytes) || overlaps(uo, q_bytes, uv, kv_bytes))
    return ATTN_ERR_INVALID_ARG;
  if (ul) {
    const uintptr_t l_bytes = (uintptr_t)(p.B * p.H * p.Nq) * 4u;
    if (overlaps(ul, l_bytes, uq, q_bytes) || overlaps(ul, l_bytes, uk, kv_bytes) ||
        overlaps(ul, l_bytes, uv, kv_bytes) || overlaps(ul, l_bytes, uo, q_bytes))
      return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

// Workspace checks: present, large enough, 256-byte aligned, disjoint from the
// tensors (lse included).
inline attn_status_t check_workspace(const void* ws, uint64_t ws_bytes, int64_t need, const Problem& p) {
  if (ws == nullptr || ws_bytes < (uint64_t)need) return ATTN_ERR_WORKSPACE;
  const uintptr_t uw = (uintptr_t)ws;
  if (uw & 255u) return ATTN_ERR_WORKSPACE;
  const uintptr_t q_bytes = (uintptr_t)(p.B * p.H * p.Nq * p.d) * 2u;
  const uintptr_t kv_bytes = (uintptr_t)(p.B * p.H * p.Nkv * p.d) * 2u;
  const uintptr_t l_bytes = (uintptr_t)(p.B * p.H * p.Nq) * 4u;
  const struct {
    const void* ptr;
    uintptr_t bytes;
  } t[5] = {{p.q, q_bytes}, {p.k, kv_bytes}, {p.v, kv_bytes}, {p.o, q_bytes}, {p.lse, l_bytes}};
  for (const auto& x : t)
    if (x.ptr && overlaps(uw, (uintptr_t)need, (uintptr_t)x.ptr, x.bytes)) return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

// Backward: the backward kernels take every problem the forward takes (d = 32, 64
// or 128, every mask, Nq != Nkv). The dK/dV kernel also streams one head's Q and
// dO rows through a 32-bit buffer record count, so Nq * d * 2 bytes must fit too.
inline attn_status_t check_bwd_problem(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale,
                                       int32_t mask_mode, const void* params) {
  const attn_status_t st = check_problem(B, H, Nq, Nkv, d, scale, mask_mode, params);
  if (st != ATTN_OK) return st;
  if (Nq * d * 2 > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Backward pointers: every tensor present and aligned (lse 4 bytes, the rest 16),
// outputs disjoint from the inputs and from each other, the workspace (if any
// bytes are needed) large enough, 256-byte aligned and disjoint from all tensors.
struct BwdPointers {
  const void *q, *k, *v, *o, *dout, *lse;
  void *dq, *dk, *dv;
};

inline attn_status_t check_bwd_pointers(const BwdPointers& p, int64_t B, int64_t H, int64_t Nq, int64_t Nkv,
                                        int64_t d, const void* ws, uint64_t ws_bytes) {
  const void* all[9] = {p.q, p.k, p.v, p.o, p.dout, p.lse, p.dq, p.dk, p.dv};
  for (const void* x : all)
    if (x == nullptr) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < 9; ++i)
    if ((uintptr_t)all[i] & (i == 5 ? 3u : 15u)) return ATTN_ERR_ALIGNMENT;
  const uintptr_t qb = (uintptr_t)(B * H * Nq * d) * 2u, kb = (uintptr_t)(B * H * Nkv * d) * 2u;
  const uintptr_t lb = (uintptr_t)(B * H * Nq) * 4u;
  const uintptr_t bytes[9] = {qb, kb, kb, qb, qb, lb, qb, kb, kb};
  for (int out = 6; out < 9; ++out)
    for (int i = 0; i < 9; ++i)
      if (i != out && overlaps((uintptr_t)all[out], bytes[out], (uintptr_t)all[i], bytes[i])) return ATTN_ERR_INVALID_ARG;
  const uint64_t need = (uint64_t)lb;
  if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws & 255u)) return ATTN_ERR_WORKSPACE;
  for (int i = 0; i < 9; ++i)
    if (overlaps((uintptr_t)ws, (uintptr_t)need, (uintptr_t)all[i], bytes[i])) return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

}  // namespace attn
