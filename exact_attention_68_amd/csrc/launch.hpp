// Internal interface between the C ABI (attn_api.cpp) and the kernels (attn_fwd.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "tile_plan.hpp"
#include "validate.hpp"

namespace attn {

// Arguments of one launch, passed by value to the kernel.
struct KernelArgs {
  const uint16_t* q;  // bfloat16 bit patterns, [B, H, Nq, d]
  const uint16_t* k;  // [B, H, Nkv, d]
  const uint16_t* v;
  uint16_t* o;        // [B, H, Nq, d]
  float* lse;         // [B, H, Nq] or null
  int32_t Nq, Nkv;    // queries and keys per head
  int32_t BH;         // B * H
  int32_t n_qtiles;   // ceil(Nq / 128)
  int32_t n_kvtiles;  // ceil(Nkv / key tile)
  float c;            // |scale| * log2(e)
  uint32_t q_sign;    // 0x80008000 when scale < 0 (flips Q's sign bits), else 0
  NaGeom na;          // neighbourhood geometry (neighbourhood masks only)
  float na_inv_w;     // 1 / grid_w, rounded to float
  float na_inv_h;     // 1 / grid_h, rounded to float
  int32_t na_phases;  // grid_w / 32 for the block-masked kernel, else 0
  // remainder split (SplitPlan; ws_parts null = one work-group per query tile)
  float* ws_parts;       // rem * parts slots of part_slot_bytes(d)
  uint32_t* split_count; // rem arrival counters (after the slots), zeroed before the launch
  int32_t split_full;   // whole-tile work-groups
  int32_t split_parts;  // parts per split tile
  int32_t causal_group; // causal: heads per XCD dispatched together (causal_item)
  int32_t patch_nx, patch_ny;  // MASK_NA_PATCH: patches per grid row and per grid column;
                               // MASK_NA_ROWS: patch_ny row groups per plane (na_row_groups)
  int32_t rows_stage;  // MASK_NA_ROWS: key rows per LDS stage (rows_lds_rows or rows_wide_lds)
  int32_t patch_cols_strided;  // MASK_NA_PATCH: na_patch_cols_strided
};

// Bytes of one part slot (partial output, maximum and sums of 4 wavefronts x 64 lanes).
constexpr int64_t part_slot_bytes(int64_t d) { return (4 * (d / 32) * 4 * 64 * 4 + 2 * 4 * 64) * 4; }
// Bytes of the arrival counters of `rem` split tiles (one 32-bit word each, whole 256-byte lines).
constexpr int64_t split_count_bytes(int64_t rem) { return (rem * 4 + 255) / 256 * 256; }
constexpr int64_t split_workspace_bytes(const SplitPlan& p, int64_t d) {
  return p.rem > 0 ? (int64_t)p.slots() * part_slot_bytes(d) + split_count_bytes(p.rem) : 0;
}

// Bytes of the device scratch of attn_fwd_ex_static: the split workspace of the largest
// plan on a device of up to 256 CUs (at most one part slot per CU, d = 128 slots, and
// fewer than 256 split tiles).
constexpr int64_t kStaticScratchBytes = 256 * part_slot_bytes(128) + split_count_bytes(256);

// Device address of this device's static scratch (file-scope __device__ array,
// looked up once per device with hipGetSymbolAddress and cached).
hipError_t static_scratch(void** ptr);

// Key rows (32 keys each) the patch kernel of 2D neighbourhood windows keeps in LDS for
// head size d (0: no patch kernel at that size).
constexpr int32_t patch_lds_rows(int64_t d) { return d == 32 ? 24 : d == 64 ? 17 : 0; }

// Key rows per LDS stage of the row kernel of narrow grids for head size d (0: none). At
// d = 64 the two 8-row stages take 128 KB: one work-group, one wavefront per SIMD, per CU
// (1.11x the tile kernel on the 20x20x20 volume with a 5x5x5 window, 1.72x at dilation 2).
constexpr int32_t rows_lds_rows(int64_t d) { return d == 32 ? 10 : d == 64 ? 8 : 0; }

// The wide stages of the three row kernels (forward, backward dQ and dK/dV) at d = 32: 12
// rows, for bands past the narrow stages (clamped windows whose reverse bands near a
// border pass 8 rows; dilated rows on a wrapped axis the dilation does not divide, whose
// groups stay consecutive). Their two stages take 96-102 KB of LDS: one work-group per CU.
constexpr int32_t rows_wide_lds(int64_t d) { return d == 32 ? 12 : 0; }

// Work-groups of the backward kernels resident per CU: two at d <= 64 and one at d = 128
// (their register and LDS budgets). The causal dispatch order sizes its head groups with it.
constexpr int32_t bwd_wgs_per_cu(int64_t d) { return d == 128 ? 1 : 2; }

// Keys per key/value tile of the kernel for head size d: 128 for d = 32 and 64,
// 64 for d = 128 (the same 16 KB of LDS per K or V tile).
constexpr int32_t tile_keys(int64_t d) { return d == 128 ? 64 : 128; }

// Arguments of the backward kernels (attn_bwd.hip), passed by value.
struct BwdArgs {
  const uint16_t* q;     // bfloat16 [B, H, Nq, d]
  const uint16_t* k;     // [B, H, Nkv, d]
  const uint16_t* v;
  const uint16_t* o;     // forward output [B, H, Nq, d]
  const uint16_t* dout;  // output gradient [B, H, Nq, d]
  const float* lse;      // forward logsumexp (natural log) [B, H, Nq]
  float* delta;          // workspace: rowsum(dO * O) [B, H, Nq]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int32_t Nq, Nkv, BH;
  int32_t n_qtiles;  // ceil(Nq / 128)
  int32_t n_ktiles;  // ceil(Nkv / 128)
  float c;           // |scale| * log2(e)
  float scale;       // signed
  uint32_t q_sign;   // 0x80008000 when scale < 0, else 0
  NaGeom na;         // neighbourhood geometry (neighbourhood masks only)
  float na_inv_w;    // 1 / grid_w, rounded to float
  float na_inv_h;    // 1 / grid_h, rounded to float
  int32_t na_grid;   // 1: per-axis window masks (na_grid_eligible), else the element test
  int32_t group_q;   // causal: heads per XCD dispatched together by the dQ kernel (causal_group)
  int32_t group_k;   // and by the dK/dV kernel
  // neighbourhood windows on grids at most 32 wide: the row kernels, with this many rows per
  // LDS stage (bwd_dq_rows_lds / bwd_dkv_rows_lds, else rows_wide_lds), or the tile kernels (0)
  int32_t dq_rows;   // dQ by query rows (na_rows_eligible)
  int32_t dkv_rows;  // dK/dV by key rows (na_rows_reverse_eligible)
  int32_t row_groups;  // row groups per plane, na_row_groups (either row kernel)
  // neighbourhood windows of one plane whose bands fit 32 columns: the patch kernels
  int32_t dq_patch;    // dQ by 8 x 16 query patches (na_patch_bwd_eligible, forward bands)
  int32_t dkv_patch;   // dK/dV by 8 x 16 key patches (reverse bands)
  int32_t patch_nx, patch_ny;  // patches per grid row and per grid column
  int32_t patch_cols_strided;  // na_patch_cols_strided
};

// Key rows per LDS stage of the dQ row kernel and query rows per stage of the dK/dV
// row kernel for head size d (0: no row kernel at that size).
constexpr int32_t bwd_dq_rows_lds(int64_t d) { return d == 32 ? 10 : d == 64 ? 8 : 0; }
constexpr int32_t bwd_dkv_rows_lds(int64_t d) { return d == 32 || d == 64 ? 8 : 0; }

// Rows (of 32 tokens) of the LDS rectangles of the backward patch kernels for head size d.
constexpr int32_t bwd_patch_lds(int64_t d) { return d == 32 ? 24 : d == 64 ? 17 : 0; }

// Launches the two backward kernels on `stream`: dQ (which also forms D = rowsum(dO * O)
// in the workspace), then dK and dV.
hipError_t launch_bwd(const BwdArgs& a, int32_t d, int32_t mask, hipStream_t stream);

// Launches the kernel for head size d (32, 64 or 128) and kernel mask `mask`
// (MASK_*). With a.ws_parts set (unmasked problems only), a one-work-group
// kernel zeroes the rem arrival counters, then n_wg = full + rem * parts
// work-groups run the whole tiles and the parts (each tile's last part merges
// it), both on `stream`.
hipError_t launch_fwd(const KernelArgs& a, int32_t d, int32_t mask, int32_t n_wg, int32_t rem, hipStream_t stream);

}  // namespace attn
