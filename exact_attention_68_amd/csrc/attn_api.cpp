// The C ABI of libattn: argument checks, launch geometry, error mapping.
// The operation and its contract are documented in include/attn.h.
#include <hip/hip_runtime_api.h>
#include <math.h>

#include <atomic>

#include "attn.h"
#include "launch.hpp"
#include "tile_plan.hpp"
#include "validate.hpp"

static_assert(ATTN_STATIC_SCRATCH_BYTES == attn::kStaticScratchBytes, "header and library agree on the scratch size");

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

attn::SplitPlan plan_for(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, int32_t mask_mode, int32_t cus) {
  const int64_t n_tiles = B * H * attn::cdiv(Nq, attn::kBlockM);
  return attn::split_plan(mask_mode, n_tiles, (int32_t)attn::cdiv(Nkv, attn::tile_keys(d)), cus);
}

// Key rows per LDS stage of the forward row kernel for this window, 0 if it fits neither
// the narrow nor the wide stages.
int32_t rows_stage(int64_t d, const attn::NaGeom& g) {
  const int32_t narrow = attn::rows_lds_rows(d), wide = attn::rows_wide_lds(d);
  if (narrow > 0 && attn::na_rows_eligible(g, narrow)) return narrow;
  if (wide > 0 && attn::na_rows_eligible(g, wide)) return wide;
  return 0;
}

// Kernel mask kind for a checked problem: the patch kernel for 2D windows whose
// patch bands fit it (na_patch_eligible, d = 32 or 64); the row kernel for other
// windows on grids at most 32 wide whose bands fit its stages (rows_stage, d = 32 or 64); the
// block-masked neighbourhood kernel for other undilated 2D windows on grids of
// width 32, 64, 96 or 128; the grid-mask kernel for other grids of width 4..124
// with rows and planes <= 128; the element predicate for the rest.
int32_t kernel_mask(const attn::Problem& p, const attn::NaGeom& g) {
  if (p.mask == ATTN_MASK_NONE) return attn::MASK_NONE;
  if (p.mask == ATTN_MASK_CAUSAL) return attn::MASK_CAUSAL;
  const int32_t patch_rows = attn::patch_lds_rows(p.d);
  if (patch_rows > 0 && attn::na_patch_eligible(g, patch_rows)) {
    const int64_t patches =
        p.B * p.H * attn::na_patch_row_groups(g) * attn::na_patch_col_groups(g, attn::na_patch_cols_strided(g));
    if (patches <= INT32_MAX) return attn::MASK_NA_PATCH;
  }
  if (rows_stage(p.d, g) > 0) {
    const int64_t groups = p.B * p.H * (int64_t)g.grid_d * attn::na_row_groups(g);
    if (groups <= INT32_MAX) return attn::MASK_NA_ROWS;
  }
  const bool blocks = g.grid_d == 1 && g.dil_h == 1 && g.dil_w == 1 && g.grid_w % 32 == 0 && g.grid_w <= 128;
  if (blocks) return attn::MASK_NA_BLOCKS;
  return attn::na_grid_eligible(g) ? attn::MASK_NA_GRID : attn::MASK_NA;
}

attn_status_t run_fwd(const attn::Problem& p, const attn::SplitPlan* split, void* workspace, void* stream) {
  attn::KernelArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.k = static_cast<const uint16_t*>(p.k);
  a.v = static_cast<const uint16_t*>(p.v);
  a.o = static_cast<uint16_t*>(p.o);
  a.lse = p.lse;
  a.Nq = (int32_t)p.Nq;
  a.Nkv = (int32_t)p.Nkv;
  a.BH = (int32_t)(p.B * p.H);
  a.n_qtiles = (int32_t)attn::cdiv(p.Nq, attn::kBlockM);
  a.n_kvtiles = (int32_t)attn::cdiv(p.Nkv, attn::tile_keys(p.d));
  // causal forward: every head in one superblock, longest first over the whole grid. Head
  // groups sized to the XCDs' slots (the backward's order) measured 7 % slower on the causal
  // B4 H16 N2048 d64 problem: fewer L2 misses, but the long and short items no longer pair
  // up as evenly on the CUs.
  a.causal_group = (int32_t)attn::cdiv(a.BH, 8);
  // exp(x) = 2^(x log2 e): the kernel works in base 2 with the scale folded in
  a.c = (float)(fabs((double)p.scale) * 1.4426950408889634);
  a.q_sign = p.scale < 0.f ? 0x80008000u : 0u;
  int32_t mask = attn::MASK_NONE;
  if (attn::is_na_mode(p.mask)) {
    a.na = attn::na_geom(p.mask, p.params);
    a.na_inv_w = 1.0f / (float)a.na.grid_w;
    a.na_inv_h = 1.0f / (float)a.na.grid_h;
  }
  mask = kernel_mask(p, a.na);
  a.na_phases = mask == attn::MASK_NA_BLOCKS ? a.na.grid_w / 32 : 0;
  int32_t n_wg = a.BH * a.n_qtiles, rem = 0;
  if (mask == attn::MASK_NA_PATCH) {
    a.patch_cols_strided = attn::na_patch_cols_strided(a.na) ? 1 : 0;
    a.patch_nx = attn::na_patch_col_groups(a.na, a.patch_cols_strided != 0);
    a.patch_ny = attn::na_patch_row_groups(a.na);
    n_wg = a.BH * a.patch_nx * a.patch_ny;
  }
  if (mask == attn::MASK_NA_ROWS) {
    a.patch_nx = 1;
    a.patch_ny = attn::na_row_groups(a.na);
    a.rows_stage = rows_stage(p.d, a.na);
    n_wg = a.BH * a.na.grid_d * a.patch_ny;
  }
  if (split != nullptr && split->rem > 0) {
    a.ws_parts = static_cast<float*>(workspace);
    a.split_count = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(workspace) +
                                                (int64_t)split->slots() * attn::part_slot_bytes(p.d));
    a.split_full = split->full;
    a.split_parts = split->parts;
    n_wg = split->groups();
    rem = split->rem;
  }
  const hipError_t e = attn::launch_fwd(a, (int32_t)p.d, mask, n_wg, rem, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// The shared body of attn_fwd_ws and attn_fwd_ex.
attn_status_t run_with_workspace(const attn::Problem& p, void* workspace, uint64_t workspace_bytes, void* stream) {
  attn_status_t st = attn::check_problem(p);
  if (st != ATTN_OK) return st;
  st = attn::check_pointers(p);
  if (st != ATTN_OK) return st;
  int32_t cus = 0;
  st = device_cus(&cus);
  if (st != ATTN_OK) return st;
  const attn::SplitPlan plan = plan_for(p.B, p.H, p.Nq, p.Nkv, p.d, p.mask, cus);
  const int64_t need = attn::split_workspace_bytes(plan, p.d);
  if (need > 0) {
    st = attn::check_workspace(workspace, workspace_bytes, need, p);
    if (st != ATTN_OK) return st;
  }
  return run_fwd(p, &plan, workspace, stream);
}

attn_status_t workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, int32_t mask_mode,
                             const void* params, uint64_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  attn_status_t st = attn::check_problem(B, H, Nq, Nkv, d, 1.0f, mask_mode, params);
  if (st != ATTN_OK) return st;
  int32_t cus = 0;
  st = device_cus(&cus);
  if (st != ATTN_OK) return st;
  *bytes = (uint64_t)attn::split_workspace_bytes(plan_for(B, H, Nq, Nkv, d, mask_mode, cus), d);
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_check(int64_t B, int64_t H, int64_t N, int64_t d, float scale, int32_t mask_mode,
                             const void* params) {
  return attn::check_problem(B, H, N, N, d, scale, mask_mode, params);
}

attn_status_t attn_fwd_ex_check(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale,
                                int32_t mask_mode, const void* params) {
  return attn::check_problem(B, H, Nq, Nkv, d, scale, mask_mode, params);
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                       int64_t d, float scale, int32_t mask_mode, const void* params, void* stream) {
  const attn::Problem p{q, k, v, o, nullptr, B, H, N, N, d, scale, mask_mode, params};
  attn_status_t st = attn::check_problem(p);
  if (st != ATTN_OK) return st;
  st = attn::check_pointers(p);
  if (st != ATTN_OK) return st;
  return run_fwd(p, nullptr, nullptr, stream);
}

attn_status_t attn_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int32_t mask_mode,
                                      const void* params, uint64_t* bytes) {
  return workspace_size(B, H, N, N, d, mask_mode, params, bytes);
}

attn_status_t attn_fwd_ex_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                                         int32_t mask_mode, const void* params, uint64_t* bytes) {
  return workspace_size(B, H, Nq, Nkv, d, mask_mode, params, bytes);
}

attn_status_t attn_fwd_ws(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H, int64_t N,
                          int64_t d, float scale, int32_t mask_mode, const void* params, void* workspace,
                          uint64_t workspace_bytes, void* stream) {
  const attn::Problem p{q, k, v, o, nullptr, B, H, N, N, d, scale, mask_mode, params};
  return run_with_workspace(p, workspace, workspace_bytes, stream);
}

attn_status_t attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                          int64_t Nq, int64_t Nkv, int64_t d, float scale, int32_t mask_mode, const void* params,
                          void* workspace, uint64_t workspace_bytes, void* stream) {
  const attn::Problem p{q, k, v, o, lse, B, H, Nq, Nkv, d, scale, mask_mode, params};
  return run_with_workspace(p, workspace, workspace_bytes, stream);
}

attn_status_t attn_fwd_ex_static(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                 int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale, int32_t mask_mode,
                                 const void* params, void* stream) {
  const attn::Problem p{q, k, v, o, lse, B, H, Nq, Nkv, d, scale, mask_mode, params};
  attn_status_t st = attn::check_problem(p);
  if (st != ATTN_OK) return st;
  st = attn::check_pointers(p);
  if (st != ATTN_OK) return st;
  int32_t cus = 0;
  st = device_cus(&cus);
  if (st != ATTN_OK) return st;
  const attn::SplitPlan plan = plan_for(p.B, p.H, p.Nq, p.Nkv, p.d, p.mask, cus);
  const int64_t need = attn::split_workspace_bytes(plan, p.d);
  if (need > attn::kStaticScratchBytes) return ATTN_ERR_SCRATCH;
  void* scratch = nullptr;
  if (need > 0 && attn::static_scratch(&scratch) != hipSuccess) return ATTN_ERR_HIP;
  return run_fwd(p, &plan, scratch, stream);
}

attn_status_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d, int32_t mask_mode,
                                      const void* params, uint64_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  const attn_status_t st = attn::check_bwd_problem(B, H, Nq, Nkv, d, 1.0f, mask_mode, params);
  if (st != ATTN_OK) return st;
  *bytes = (uint64_t)(B * H * Nq) * 4u;
  return ATTN_OK;
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                       void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nkv, int64_t d,
                       float scale, int32_t mask_mode, const void* params, void* workspace, uint64_t workspace_bytes,
                       void* stream) {
  attn_status_t st = attn::check_bwd_problem(B, H, Nq, Nkv, d, scale, mask_mode, params);
  if (st != ATTN_OK) return st;
  st = attn::check_bwd_pointers(attn::BwdPointers{q, k, v, o, dout, lse, dq, dk, dv}, B, H, Nq, Nkv, d, workspace,
                                workspace_bytes);
  if (st != ATTN_OK) return st;
  attn::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.delta = static_cast<float*>(workspace);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.Nq = (int32_t)Nq;
  a.Nkv = (int32_t)Nkv;
  a.BH = (int32_t)(B * H);
  a.n_qtiles = (int32_t)attn::cdiv(Nq, attn::kBlockM);
  a.n_ktiles = (int32_t)attn::cdiv(Nkv, attn::kBlockM);
  a.c = (float)(fabs((double)scale) * 1.4426950408889634);
  a.scale = scale;
  a.q_sign = scale < 0.f ? 0x80008000u : 0u;
  if ((int64_t)a.BH * a.n_ktiles > INT32_MAX) return ATTN_ERR_UNSUPPORTED;
  int32_t cus = 0;
  st = device_cus(&cus);
  if (st != ATTN_OK) return st;
  a.group_q = attn::causal_group(a.n_qtiles, cus, attn::bwd_wgs_per_cu(d));
  a.group_k = attn::causal_group(a.n_ktiles, cus, attn::bwd_wgs_per_cu(d));
  int32_t mask = mask_mode == ATTN_MASK_CAUSAL ? attn::MASK_CAUSAL : attn::MASK_NONE;
  if (attn::is_na_mode(mask_mode)) {
    a.na = attn::na_geom(mask_mode, params);
    a.na_inv_w = 1.0f / (float)a.na.grid_w;
    a.na_inv_h = 1.0f / (float)a.na.grid_h;
    a.na_grid = attn::na_grid_eligible(a.na) ? 1 : 0;
    mask = attn::MASK_NA;
    const int32_t dq_lds = attn::bwd_dq_rows_lds(d), dkv_lds = attn::bwd_dkv_rows_lds(d);
    a.row_groups = attn::na_row_groups(a.na);
    const bool groups_fit = (int64_t)a.BH * a.na.grid_d * a.row_groups <= INT32_MAX;
    const int32_t wide = attn::rows_wide_lds(d);
    if (groups_fit) {  // the narrow stages where they fit, else the wide ones
      a.dq_rows = dq_lds > 0 && attn::na_rows_eligible(a.na, dq_lds) ? dq_lds
                  : wide > 0 && attn::na_rows_eligible(a.na, wide) ? wide : 0;
      a.dkv_rows = dkv_lds > 0 && attn::na_rows_reverse_eligible(a.na, dkv_lds) ? dkv_lds
                   : wide > 0 && attn::na_rows_reverse_eligible(a.na, wide) ? wide : 0;
    }
    // wider single-plane grids: the patch kernels (the row kernels keep the narrow ones)
    const int32_t patch_lds = attn::bwd_patch_lds(d);
    a.patch_cols_strided = attn::na_patch_cols_strided(a.na) ? 1 : 0;
    a.patch_nx = attn::na_patch_col_groups(a.na, a.patch_cols_strided != 0);
    a.patch_ny = attn::na_patch_row_groups(a.na);
    const bool patches_fit = (int64_t)a.BH * a.patch_nx * a.patch_ny <= INT32_MAX;
    a.dq_patch = !a.dq_rows && patches_fit && attn::na_patch_bwd_eligible(a.na, patch_lds, false) ? 1 : 0;
    a.dkv_patch = !a.dkv_rows && patches_fit && attn::na_patch_bwd_eligible(a.na, patch_lds, true) ? 1 : 0;
  }
  const hipError_t e = attn::launch_bwd(a, (int32_t)d, mask, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char* attn_status_string(int32_t status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size, non-finite scale, "
                                      "unknown mask mode, misplaced params, or an output overlapping an input "
                                      "or the other output)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported problem (head size must be 32, 64 or 128; sizes must fit "
                                      "32-bit launch geometry, and one head's K and V rows (the backward: also "
                                      "Q and dO rows) at most 2^31 - 1 bytes)";
    case ATTN_ERR_PARAMS: return "inconsistent neighbourhood parameters (grid size must equal Nq and Nkv; "
                                 "kernels odd; wrap 0 or 1; dilation >= 1; (kernel-1)*dilation < size when "
                                 "wrapped, kernel*dilation <= size when clamped)";
    case ATTN_ERR_ALIGNMENT: return "q, k, v and o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_HIP: return "HIP runtime error (no device, or a failed query or launch)";
    case ATTN_ERR_WORKSPACE: return "workspace missing, too small, not 256-byte aligned, or overlapping a tensor";
    case ATTN_ERR_SCRATCH: return "attn_fwd_ex_static: the problem's split needs more than the library's static "
                                  "device scratch (ATTN_STATIC_SCRATCH_BYTES); use attn_fwd_ex with a workspace";
    default: return "unknown status";
  }
}

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
