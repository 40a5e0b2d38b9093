// Backward pass of the fused exact attention for gfx950: the gradients of
// O = softmax(scale * Q K^T + mask) V with respect to Q, K and V, for an output
// gradient dO, without writing the score matrix (NATTEN issue 142: the fused
// forward saves the logsumexp for the backward, whose kernels visit query
// tiles per key tile; the gradients are those of its autograd function).
//
// With P = exp(scale * S - LSE) recomputed tile by tile from the saved row
// logsumexp, and D_i = sum_d dO_id O_id (the row sum of P * dP):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Two kernels on the caller's stream:
//   attn_bwd_dq_kernel    one work-group per 128-query tile (4 wavefronts x 32
//                         queries); first D of its queries (fp32, also left in
//                         the workspace for the next kernel), then key/value
//                         tiles streamed through LDS:
//                         S^T = K Q^T, dP^T = V dO^T (the forward's S^T layout,
//                         one query per lane column), dS^T, then dQ^T += K^T dS^T
//                         (the forward's O^T += V^T P^T layout, K read through
//                         the transposing LDS read);
//   attn_bwd_dkv_kernel   one work-group per 128-key tile (one key per lane
//                         column), query/dO tiles streamed: S = Q K^T,
//                         dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS.
// Both multiply bf16 operands on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation; P and dS are rounded to bf16 as MFMA operands. Masks: none,
// causal (top-left), and the 2D/3D neighbourhood windows through an element
// test; the dK/dV kernel visits a band of query tiles that holds every query
// whose window reaches its keys, so the gradients of keys reached across a
// wrapped border are summed in place.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn.h"
#include "kernel_common.hpp"
#include "launch.hpp"
#include "tile_plan.hpp"

namespace attn {

namespace {

template <int D>
struct BwdCfg {
  static constexpr int ROWS = 128;  // rows of a streamed tile; a work-group holds 4 x 32 resident rows
  // Two buffers of two streamed tiles: 64 KB of LDS at d <= 64 (two work-groups per CU),
  // 128 KB at d = 128 (one work-group per CU, whose wavefronts then get the whole
  // register file: the d = 128 accumulators do not fit in half of it).
  static constexpr int WAVES_PER_EU = D == 128 ? 1 : 2;
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int TILE = ROWS * D;
  static constexpr int LOADS = ROWS * ROW_CHUNKS / THREADS;  // 16-byte loads per thread per tile
  static constexpr int SB = ROWS / 32;                       // 32-row blocks per streamed tile
  static constexpr int KB = D / 16;
  static constexpr int DT = D / 32;
  static_assert(ROWS * ROW_CHUNKS % THREADS == 0, "tile chunks must split evenly");
};

// Global -> LDS copy of a tile of ROWS rows of one head (the forward's layout and swizzle).
template <int D>
struct RowTileLoader {
  using C = BwdCfg<D>;
  uint32_t voff[C::LOADS];
  int wave;

  __device__ __forceinline__ RowTileLoader(int wave_, int lane) : wave(wave_) {
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int p = (j * C::WAVES + wave_) * 64 + lane;
      const int row = p / C::ROW_CHUNKS;
      const int chunk = (p % C::ROW_CHUNKS) ^ chunk_swizzle<D>(row);
      voff[j] = (uint32_t)(row * D + chunk * 8) * 2u;
    }
  }

  __device__ __forceinline__ void load(i32x4_t src, int32_t tile, const uint16_t* lds_tile) const {
    // byte offset of the tile in the head, below 2^31 (one head's rows fit a 32-bit record count)
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)tile * (uint32_t)(C::ROWS * D * 2));
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds_tile) + wave * 1024);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) dma_lds16(src, base + j * C::WAVES * 1024, voff[j], soff);
  }
};

// Fragment of a resident row (the lane's query or key) as the B operand of a
// 32x32x16 MFMA: d = 16kb + 8*half + 0..7; zero past the last row.
template <int D>
__device__ __forceinline__ void row_fragment(const uint16_t* rows, int32_t row, int32_t n_rows, uint32_t sign, int half,
                                             bf16x8_t (&f)[D / 16]) {
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    u32x4_t x = u32x4_t{0, 0, 0, 0};
    if (row < n_rows) {
      x = *reinterpret_cast<const u32x4_t*>(rows + (size_t)row * D + kb * 16 + half * 8);
      x ^= sign;
    }
    f[kb] = __builtin_bit_cast(bf16x8_t, x);
  }
}

// One 32-row block of a streamed tile times the resident fragments: acc = T[rows] R^T,
// lane holds rows 32sb + 8(r/4) + 4*half + r%4 of its resident column.
template <int D>
__device__ __forceinline__ f32x16_t block_product(const uint16_t* tile, int sb, int col, int half, int swz,
                                                  const bf16x8_t (&f)[D / 16]) {
  f32x16_t acc = f32x16_t{};
  const int row = sb * 32 + col;
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(tile + row * D + (((2 * kb + half) ^ swz) << 3));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), f[kb], acc, 0, 0, 0);
  }
  return acc;
}

// acc^T += tile[block rows]^T W^T for the 32 rows of block sb, with W (bf16, two
// 16-row halves) in the accumulator order of block_product: the forward's P V step.
template <int D>
__device__ __forceinline__ void block_transpose_product(const uint16_t* tile, int sb, const int (&v_row)[2],
                                                        const int (&v_off)[2][D / 32], const bf16x8_t (&w)[2],
                                                        f32x16_t (&acc)[D / 32]) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int row0 = sb * 32 + kb2 * 16;
      u32x2_t x[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        x[h] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                               (lds_s16x4*)((lds_u16*)tile + (row0 + v_row[h]) * D + v_off[h][dt])));
      const bf16x8_t tf = __builtin_bit_cast(bf16x8_t, u32x4_t{x[0][0], x[0][1], x[1][0], x[1][1]});
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf, w[kb2], acc[dt], 0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void transpose_offsets(int lane, int half, int (&v_row)[2], int (&v_off)[2][D / 32]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v_row[h] = h * 8 + half * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int dcol = dt * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
      v_off[h][dt] = (((dcol >> 3) ^ chunk_swizzle<D>(v_row[h])) << 3) + (dcol & 7);
    }
  }
}

// Rounds an accumulator block to the bf16 MFMA operand (two halves of 8 elements).
__device__ __forceinline__ void to_bf16_operand(const f32x16_t& x, bf16x8_t (&w)[2]) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2_t pr = {(__bf16)x[kb2 * 8 + e], (__bf16)x[kb2 * 8 + e + 1]};
      w[kb2][e] = pr[0];
      w[kb2][e + 1] = pr[1];
    }
}

// Stores scale * acc^T (d x 32 columns, the lane's column = one row of the output) as bf16 rows.
template <int D>
__device__ __forceinline__ void store_rows_scaled(uint16_t* out, int32_t row, int32_t n_rows, int half,
                                                  const f32x16_t (&acc)[D / 32], float scale) {
  if (row >= n_rows) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4_t ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(acc[dt][g * 4 + e] * scale);
      *reinterpret_cast<u32x2_t*>(out + (size_t)row * D + dt * 32 + g * 8 + half * 4) = __builtin_bit_cast(u32x2_t, ob);
    }
}

constexpr float kLog2e = 1.4426950408889634f;

// Whether a tile's 32-row blocks run as a two-stage pipeline (next block's S and
// dP products before this block's softmax arithmetic): only where the extra two
// accumulators fit the registers without spilling.
template <int D>
constexpr bool kPipelineBlocks = D == 32;

// Neighbourhood windows: grid coordinates of the tokens of a tile, decoded from
// the tile's first token (one division per tile) plus an offset below 128.
struct TileOrigin {
  int32_t x0, y0, z0;
};

__device__ __forceinline__ TileOrigin tile_origin(int32_t t0, const NaGeom& g) {
  const int32_t row0 = t0 / g.grid_w, z0 = row0 / g.grid_h;
  return TileOrigin{t0 - row0 * g.grid_w, row0 - z0 * g.grid_h, z0};
}

// For n < 2^21 the quotient (n + 0.5) / L stays at least 0.5 / L from an integer, far
// more than the float error, so truncation is exact (n = x0 + off < grid_w + 128 here).
__device__ __forceinline__ void token_coords(const TileOrigin& o, int32_t off, const NaGeom& g, float inv_w,
                                             float inv_h, int32_t& z, int32_t& y, int32_t& x) {
  const int32_t dy = (int32_t)(((float)(o.x0 + off) + 0.5f) * inv_w);
  x = o.x0 + off - dy * g.grid_w;
  const int32_t yy = o.y0 + dy;
  const int32_t dz = (int32_t)(((float)yy + 0.5f) * inv_h);
  y = yy - dz * g.grid_h;
  z = o.z0 + dz;
}

// Whether key (zk, yk, xk) lies in the window of query (zq, yq, xq), every axis.
__device__ __forceinline__ bool na_visible(const NaGeom& g, int32_t zq, int32_t yq, int32_t xq, int32_t zk, int32_t yk,
                                           int32_t xk) {
  if ((g.dil_d | g.dil_h | g.dil_w) == 1)
    return na_axis_ok(zq, zk, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d) &
           na_axis_ok(yq, yk, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h) &
           na_axis_ok(xq, xk, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w);
  return na_dil_ok(na_dil_anchor(zq, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d), zk, g.grid_d, g.kernel_d,
                   g.rad_d, g.wrap_d, g.dil_d) &
         na_dil_ok(na_dil_anchor(yq, g.grid_h, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h), yk, g.grid_h, g.kernel_h,
                   g.rad_h, g.wrap_h, g.dil_h) &
         na_dil_ok(na_dil_anchor(xq, g.grid_w, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w), xk, g.grid_w, g.kernel_w,
                   g.rad_w, g.wrap_w, g.dil_w);
}

}  // namespace

// This lane's share of D = sum_d dO_d O_d for its row: the fragments hold
// d = 16kb + 8*half + 0..7 (bf16, widened exactly); the two half-waves hold the
// two halves of d, combined by the caller.
template <int D>
__device__ __forceinline__ float row_delta_part(const bf16x8_t (&o)[D / 16], const bf16x8_t (&g)[D / 16]) {
  float acc = 0.f;
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    const u32x4_t x = __builtin_bit_cast(u32x4_t, o[kb]);
    const u32x4_t y = __builtin_bit_cast(u32x4_t, g[kb]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += __uint_as_float(x[w] << 16) * __uint_as_float(y[w] << 16);
      acc += __uint_as_float(x[w] & 0xffff0000u) * __uint_as_float(y[w] & 0xffff0000u);
    }
  }
  return acc;
}

// dQ for one 128-query tile: key/value tiles through a two-buffer LDS ring.
template <int D, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_EU)))
void attn_bwd_dq_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][C::TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int32_t Nq = a.Nq, Nkv = a.Nkv;
  const WorkItem w = work_item(MASK, blockIdx.x, gridDim.x, a.n_qtiles, a.BH, a.group_q);
  const int32_t q0 = w.qtile * C::ROWS, my_q = q0 + wave * 32 + col;
  const size_t qhead = (size_t)w.bh * Nq, khead = (size_t)w.bh * Nkv;

  bf16x8_t qf[C::KB], gf[C::KB];
  row_fragment<D>(a.q + qhead * D, my_q, Nq, a.q_sign, half, qf);
  row_fragment<D>(a.dout + qhead * D, my_q, Nq, 0u, half, gf);
  const float l2 = my_q < Nq ? a.lse[qhead + my_q] * kLog2e : 0.f;
  // D of the lane's query from its O and dO rows; the dK/dV kernel, which runs
  // after this one on the same stream, reads it from the workspace
  float dlt;
  {
    bf16x8_t of[C::KB];
    row_fragment<D>(a.o + qhead * D, my_q, Nq, 0u, half, of);
    dlt = swap_halves_sum(row_delta_part<D>(of, gf));
    if (my_q < Nq && half == 0) a.delta[qhead + my_q] = dlt;
  }

  int v_row[2], v_off[2][C::DT];
  transpose_offsets<D>(lane, half, v_row, v_off);
  const int swz = chunk_swizzle<D>(col);
  const RowTileLoader<D> ld(__builtin_amdgcn_readfirstlane(wave), lane);
  const uint32_t head_bytes = (uint32_t)Nkv * (uint32_t)(D * 2);
  const i32x4_t k_rsrc = head_rsrc(a.k + khead * D, head_bytes);
  const i32x4_t v_rsrc = head_rsrc(a.v + khead * D, head_bytes);

  const KvRun run = kv_run(MASK, Nq, Nkv, C::ROWS, C::ROWS, q0, a.na);
  int32_t zq = 0, yq = 0, xq = 0;  // the lane's query in the grid (neighbourhood masks)
  GridMasks gm{};                  // its window per axis, on grids of width 4..124 (a.na_grid)
  if constexpr (MASK == MASK_NA) {
    const int32_t plane = a.na.grid_h * a.na.grid_w;
    zq = my_q / plane;
    yq = (my_q - zq * plane) / a.na.grid_w;
    xq = my_q - zq * plane - yq * a.na.grid_w;
    if (a.na_grid) gm = na_grid_masks(zq, yq, xq, a.na);
  }
  const int32_t n = run.count;
  f32x16_t dq[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dq[dt] = f32x16_t{};

  ld.load(k_rsrc, kv_tile_at(run, 0, a.n_ktiles), k_lds[0]);
  ld.load(v_rsrc, kv_tile_at(run, 0, a.n_ktiles), v_lds[0]);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t t = kv_tile_at(run, i, a.n_ktiles);
    const int buf = i & 1;
    TileOrigin org{0, 0, 0};
    uint32_t bm[C::SB] = {};  // window bits of the tile's keys (a.na_grid)
    if constexpr (MASK == MASK_NA) {
      org = tile_origin(t * C::ROWS, a.na);
      if (a.na_grid) {
        uint32_t w4[C::SB];
        na_tile_window(gm, (t * C::ROWS) / a.na.grid_w, org.x0, a.na, w4);
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) bm[sb] = lane_block_bits(w4[sb], half);
      }
    }
    if (!kSerialTiles && i + 1 < n) {  // the other buffer was last read before the previous barrier
      const int32_t tn = kv_tile_at(run, i + 1, a.n_ktiles);
      ld.load(k_rsrc, tn, k_lds[buf ^ 1]);
      ld.load(v_rsrc, tn, v_lds[buf ^ 1]);
      wait_tile_loads<2 * C::LOADS>();
    } else {
      wait_tile_loads<0>();
    }
    __syncthreads();
    // A hidden score enters the exponent as -inf (P = 0, dS = 0 for any scale, 0 included).
    // Rows past Nq need no test: their Q and dO fragments are zero, so dS = 1 * (0 - 0).
    // Keys past Nkv do (K = 0 there, but P * (0 - D) could overflow), as do causal
    // diagonal tiles and every window tile; other tiles take the body without any test,
    // chosen per tile (uniform): a per-element select of the product itself compiles
    // into a branch around each exponential.
    auto tile_body = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      // At d = 32 a two-stage pipeline over the 32-key blocks: the next block's S
      // and dP products are issued before this block's exponentials, so the matrix
      // core has independent work while the VALU runs. At d = 64 and 128 the extra
      // accumulators do not fit the register budget (they spill), so blocks run in order.
      constexpr bool PIPE = kPipelineBlocks<D>;
      f32x16_t s_nx{}, dp_nx{};
      if constexpr (PIPE) {
        s_nx = block_product<D>(k_lds[buf], 0, col, half, swz, qf);
        dp_nx = block_product<D>(v_lds[buf], 0, col, half, swz, gf);
      }
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb) {
        f32x16_t s, dp;
        if constexpr (PIPE) {
          s = s_nx;
          dp = dp_nx;
          if (sb + 1 < C::SB) {
            s_nx = block_product<D>(k_lds[buf], sb + 1, col, half, swz, qf);
            dp_nx = block_product<D>(v_lds[buf], sb + 1, col, half, swz, gf);
          }
        } else {
          s = block_product<D>(k_lds[buf], sb, col, half, swz, qf);
          dp = block_product<D>(v_lds[buf], sb, col, half, swz, gf);
        }
        f32x16_t ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float add = -l2;
          if constexpr (MASKED) {
            const int32_t off = sb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const int32_t key = t * C::ROWS + off;
            bool ok = key < Nkv;
            if (MASK == MASK_CAUSAL) ok = ok & (key <= my_q);
            if constexpr (MASK == MASK_NA) {
              if (a.na_grid) {
                ok = ok & (((bm[sb] >> r) & 1u) != 0u);
              } else {
                int32_t zk, yk, xk;
                token_coords(org, off, a.na, a.na_inv_w, a.na_inv_h, zk, yk, xk);
                ok = ok & na_visible(a.na, zq, yq, xq, zk, yk, xk);
              }
            }
            add = ok ? add : -INFINITY;
          }
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, add));
          ds[r] = p * (dp[r] - dlt);
        }
        bf16x8_t dsb[2];
        to_bf16_operand(ds, dsb);
        block_transpose_product<D>(k_lds[buf], sb, v_row, v_off, dsb, dq);
      }
    };
    bool masked = MASK == MASK_NA || (t + 1) * C::ROWS > Nkv;
    if (MASK == MASK_CAUSAL) masked = masked || t * C::ROWS + C::ROWS - 1 > q0;
    if (masked)
      tile_body(std::true_type{});
    else
      tile_body(std::false_type{});
    if (kSerialTiles && i + 1 < n) {  // race check: the next tile's loads only after this tile's compute
      const int32_t tn = kv_tile_at(run, i + 1, a.n_ktiles);
      ld.load(k_rsrc, tn, k_lds[buf ^ 1]);
      ld.load(v_rsrc, tn, v_lds[buf ^ 1]);
    }
    __syncthreads();  // every wavefront is done with this buffer before it is refilled
  }
  store_rows_scaled<D>(a.dq + qhead * D, my_q, Nq, half, dq, a.scale);
}

// dK and dV for one 128-key tile: query/dO tiles and their logsumexp and D values
// through a two-buffer LDS ring.
template <int D, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_EU)))
void attn_bwd_dkv_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds[2][C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t g_lds[2][C::TILE];
  __shared__ __attribute__((aligned(16))) float l2_lds[2][C::ROWS];
  __shared__ __attribute__((aligned(16))) float dl_lds[2][C::ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int32_t Nq = a.Nq, Nkv = a.Nkv;
  // causal: key tile 0 sees every query tile, the last one the fewest, so they go longest
  // first in head groups (causal_item, as the forward's causal order); otherwise the key tiles
  // of a head are kept on one XCD (xcd_contiguous), whose L2 then serves its Q and dO tiles
  int32_t bh, ktile;
  if constexpr (MASK == MASK_CAUSAL) {
    const RankedItem r = causal_item(blockIdx.x, a.n_ktiles, a.BH, a.group_k);
    bh = r.bh;
    ktile = r.rank;
  } else {
    const int32_t wg = xcd_contiguous(blockIdx.x, gridDim.x);
    bh = wg / a.n_ktiles;
    ktile = wg - bh * a.n_ktiles;
  }
  const int32_t k0 = ktile * C::ROWS, my_k = k0 + wave * 32 + col;
  const size_t qhead = (size_t)bh * Nq, khead = (size_t)bh * Nkv;

  // scale < 0: K's sign bits flipped, so c S = scale * (Q K^T) with c = |scale| log2 e
  bf16x8_t kf[C::KB], vf[C::KB];
  row_fragment<D>(a.k + khead * D, my_k, Nkv, a.q_sign, half, kf);
  row_fragment<D>(a.v + khead * D, my_k, Nkv, 0u, half, vf);

  int v_row[2], v_off[2][C::DT];
  transpose_offsets<D>(lane, half, v_row, v_off);
  const int swz = chunk_swizzle<D>(col);
  const RowTileLoader<D> ld(__builtin_amdgcn_readfirstlane(wave), lane);
  const uint32_t head_bytes = (uint32_t)Nq * (uint32_t)(D * 2);
  const i32x4_t q_rsrc = head_rsrc(a.q + qhead * D, head_bytes);
  const i32x4_t g_rsrc = head_rsrc(a.dout + qhead * D, head_bytes);

  // query tiles that see some key of this tile: all; (causal, key j <= query i) those from the
  // tile holding query k0 on; for neighbourhood windows a band of them
  KvRun qrun{0, a.n_qtiles};
  if (MASK == MASK_CAUSAL) qrun = KvRun{k0 / C::ROWS, k0 / C::ROWS < a.n_qtiles ? a.n_qtiles - k0 / C::ROWS : 0};
  int32_t zk = 0, yk = 0, xk = 0;  // the lane's key in the grid (neighbourhood masks)
  GridMasks rm{};                  // per axis, the queries whose window holds it (a.na_grid)
  if constexpr (MASK == MASK_NA) {
    qrun = na_query_run(a.na, Nkv, C::ROWS, k0);
    const int32_t plane = a.na.grid_h * a.na.grid_w;
    zk = my_k / plane;
    yk = (my_k - zk * plane) / a.na.grid_w;
    xk = my_k - zk * plane - yk * a.na.grid_w;
    if (a.na_grid) rm = na_grid_reverse_masks(zk, yk, xk, a.na);
  }
  const int32_t n = qrun.count;

  f32x16_t dk[C::DT], dv[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) dk[dt] = dv[dt] = f32x16_t{};

  // logsumexp (base 2) and D of query tile qt, one value per thread of the first 128
  auto stats = [&](int32_t qt, float& l2v, float& dlv) {
    const int32_t qi = qt * C::ROWS + tid;
    const bool in = tid < C::ROWS && qi < Nq;
    l2v = in ? a.lse[qhead + qi] * kLog2e : INFINITY;  // rows past Nq: P = 0
    dlv = in ? a.delta[qhead + qi] : 0.f;
  };
  float l2n = 0.f, dln = 0.f;
  if (n > 0) {
    const int32_t q_first = kv_tile_at(qrun, 0, a.n_qtiles);
    ld.load(q_rsrc, q_first, q_lds[0]);
    ld.load(g_rsrc, q_first, g_lds[0]);
    stats(q_first, l2n, dln);
    wait_tile_loads<0>();
    if (tid < C::ROWS) {
      l2_lds[0][tid] = l2n;
      dl_lds[0][tid] = dln;
    }
    __syncthreads();
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t qt = kv_tile_at(qrun, i, a.n_qtiles);
    const int buf = i & 1;
    TileOrigin org{0, 0, 0};
    uint32_t bm[C::SB] = {};  // bits of the tile's queries whose window holds the lane's key (a.na_grid)
    if constexpr (MASK == MASK_NA) {
      org = tile_origin(qt * C::ROWS, a.na);
      if (a.na_grid) {
        uint32_t w4[C::SB];
        na_tile_window(rm, (qt * C::ROWS) / a.na.grid_w, org.x0, a.na, w4);
#pragma unroll
        for (int sb = 0; sb < C::SB; ++sb) bm[sb] = lane_block_bits(w4[sb], half);
      }
    }
    auto next_loads = [&]() {
      if (i + 1 < n) {  // next tile into the other buffers (last read before the previous barrier)
        const int32_t qn = kv_tile_at(qrun, i + 1, a.n_qtiles);
        ld.load(q_rsrc, qn, q_lds[buf ^ 1]);
        ld.load(g_rsrc, qn, g_lds[buf ^ 1]);
        stats(qn, l2n, dln);
      }
    };
    if constexpr (!kSerialTiles) next_loads();
    const int32_t kd = my_k - qt * C::ROWS;  // causal: the lane's key sees the tile's queries from kd on
    // As in the dQ kernel, a hidden score enters the exponent as -inf. Queries past Nq
    // need no test (their logsumexp is stored as +inf, so P = 0), nor do keys past Nkv
    // (their columns of dK and dV are never stored); causal tiles that hold a query
    // before a key and every window tile take the masked body, chosen per tile.
    auto tile_body = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      // Two-stage pipeline over the 32-query blocks at d = 32, as in the dQ kernel.
      constexpr bool PIPE = kPipelineBlocks<D>;
      f32x16_t s_nx{}, dp_nx{};
      if constexpr (PIPE) {
        s_nx = block_product<D>(q_lds[buf], 0, col, half, swz, kf);
        dp_nx = block_product<D>(g_lds[buf], 0, col, half, swz, vf);
      }
#pragma unroll
      for (int sb = 0; sb < C::SB; ++sb) {
        f32x16_t s, dp;
        if constexpr (PIPE) {
          s = s_nx;
          dp = dp_nx;
          if (sb + 1 < C::SB) {
            s_nx = block_product<D>(q_lds[buf], sb + 1, col, half, swz, kf);
            dp_nx = block_product<D>(g_lds[buf], sb + 1, col, half, swz, vf);
          }
        } else {
          s = block_product<D>(q_lds[buf], sb, col, half, swz, kf);
          dp = block_product<D>(g_lds[buf], sb, col, half, swz, vf);
        }
        f32x16_t p, ds;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qr = sb * 32 + 8 * g4 + 4 * half;  // first of the 4 queries of this group
          const float4 l4 = *reinterpret_cast<const float4*>(&l2_lds[buf][qr]);
          const float4 d4 = *reinterpret_cast<const float4*>(&dl_lds[buf][qr]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * g4 + j;
            float add = -lv[j];
            if constexpr (MASKED) {
              bool ok = true;
              if (MASK == MASK_CAUSAL) ok = kd <= qr + j;
              if constexpr (MASK == MASK_NA) {
                if (a.na_grid) {
                  ok = ((bm[sb] >> r) & 1u) != 0u;
                } else {
                  int32_t zq, yq, xq;
                  token_coords(org, qr + j, a.na, a.na_inv_w, a.na_inv_h, zq, yq, xq);
                  ok = na_visible(a.na, zq, yq, xq, zk, yk, xk);
                }
              }
              add = ok ? add : -INFINITY;
            }
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.c, add));
            p[r] = pv;
            ds[r] = pv * (dp[r] - dv4[j]);
          }
        }
        bf16x8_t pb[2], dsb[2];
        to_bf16_operand(p, pb);
        to_bf16_operand(ds, dsb);
        block_transpose_product<D>(g_lds[buf], sb, v_row, v_off, pb, dv);
        block_transpose_product<D>(q_lds[buf], sb, v_row, v_off, dsb, dk);
      }
    };
    bool masked = MASK != MASK_NONE;
    if (masked)
      tile_body(std::true_type{});
    else
      tile_body(std::false_type{});
    if constexpr (kSerialTiles) next_loads();  // race check: loads only after this tile's compute
    wait_tile_loads<0>();
    if (i + 1 < n && tid < C::ROWS) {
      l2_lds[buf ^ 1][tid] = l2n;
      dl_lds[buf ^ 1][tid] = dln;
    }
    __syncthreads();  // next tile published; this buffer free for refill
  }
  store_rows_scaled<D>(a.dk + khead * D, my_k, Nkv, half, dk, a.scale);
  store_rows_scaled<D>(a.dv + khead * D, my_k, Nkv, half, dv, 1.0f);
}

// ---------------------------------------------------------------------------
// Neighbourhood windows on grids at most 32 wide (na_rows_eligible,
// na_rows_reverse_eligible): the forward row kernel's layout. A work-group holds
// a group of 4 rows of one plane (RowGroup: consecutive, or of one residue mod the
// dilation), a wavefront one row and a lane one column (lanes past the
// width idle); the band rows of each plane that the work-group's windows reach
// stream through two LDS stages (32 tokens per row, columns past the width read
// as zero); each wavefront visits only its own visible rows, in order, and the
// window test inside a row is the lane's per-element addend of the exponent (-inf
// for a hidden pair). A visible row is one 32-row block of the tile kernels'
// products. Stage ring: wait for this stage, barrier (which also frees the other
// stage), issue the next stage, compute.

// ROWS rows of 32 tokens of D elements, copied in whole rounds of 256 lanes.
template <int D, int ROWS_>
struct RowStage {
  static constexpr int ROWS = ROWS_;
  static constexpr int RC = D / 8;  // 16-byte chunks per token
  static constexpr int CHUNKS = ROWS * 32 * RC;
  static_assert(ROWS > 0 && CHUNKS % 256 == 0, "a stage is copied in whole rounds of 256 lanes");
  static constexpr int LOADS = CHUNKS / 256;  // per lane, stage and tensor
  static constexpr int ELEMS = CHUNKS * 8;
};

// Copies rows [by.start, by.start + by.count) (mod H) of plane z of two tensors of
// one head into a stage each: LDS chunk p holds chunk (p % RC) ^ swizzle of token
// p / RC = 32 r + x (band row r, column x), the tile layout; columns past W and
// rows past the band read as zero (an offset past the head).
template <int D, int ROWS>
__device__ __forceinline__ void load_row_stage(i32x4_t ra, i32x4_t rb, const uint16_t* la, const uint16_t* lb,
                                               int32_t z, const RowGroup& rg, int32_t H, int32_t W,
                                               uint32_t head_bytes, int wave, int tid) {
  using R = RowStage<D, ROWS>;
  const uint32_t a_base = __builtin_amdgcn_readfirstlane(lds_addr(la) + wave * 1024);
  const uint32_t b_base = __builtin_amdgcn_readfirstlane(lds_addr(lb) + wave * 1024);
#pragma unroll
  for (int j = 0; j < R::LOADS; ++j) {
    const int32_t p = j * 256 + tid;
    const int32_t tok = p / R::RC, r = tok / 32, x = tok % 32;
    const int32_t chunk = (p % R::RC) ^ chunk_swizzle<D>(tok);
    uint32_t voff = head_bytes;
    if (r < rg.band.count && x < W) {
      const int32_t y = row_group_row(rg, r);
      voff = (uint32_t)((z * H + y) * W + x) * (uint32_t)(D * 2) + (uint32_t)chunk * 16u;
    }
    dma_lds16(ra, a_base + (uint32_t)j * 4096u, voff, 0u);
    dma_lds16(rb, b_base + (uint32_t)j * 4096u, voff, 0u);
  }
}

// The band cell of plane index j of a walk that starts at the work-group's own
// plane and runs through the band circularly.
__device__ __forceinline__ int32_t band_plane(const Band& bz, int32_t i_own, int32_t j, int32_t len) {
  int32_t i = i_own + j;
  i -= i >= bz.count ? bz.count : 0;
  const int32_t c = bz.start + i;
  return c >= len ? c - len : c;
}

// dQ by query rows: per visible key row (32 keys) S^T = K Q^T, dP^T = V dO^T,
// P = 2^(c s - lse2) (hidden keys 0), dS = P (dP - D), dQ^T += K^T dS^T; also
// forms D of its queries for the dK/dV kernel, as the tile kernel does.
template <int D, int ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 32 && ROWS <= 10 ? 2 : 1)))
void attn_bwd_dq_rows_kernel(BwdArgs a) {
  using R = RowStage<D, ROWS>;
  constexpr int KB = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][R::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][R::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const NaGeom& g = a.na;
  const int32_t H = g.grid_h, W = g.grid_w, N = a.Nq;

  // (head, plane, group of 4 rows), the items of one head kept on one XCD
  const int32_t groups = a.row_groups, per_head = g.grid_d * groups;
  const int32_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int32_t bh = item / per_head, rest = item - bh * per_head;
  const int32_t z = rest / groups;
  const RowGroup rg = na_row_group(g, rest - z * groups, false);
  const int32_t y = rg.rho + rg.stride * (rg.u0 + wave);  // this wavefront's grid row
  const bool row_in = rg.u0 + wave < rg.len;
  const bool q_ok = row_in && col < W;
  const int32_t my_q = (z * H + y) * W + col;
  const int32_t q_row = q_ok ? my_q : N;  // past the last row: zero fragments, no store
  const size_t head = (size_t)bh * (size_t)N;
  const uint32_t head_bytes = (uint32_t)N * (uint32_t)(D * 2);

  const Band bz = na_band(z, z, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d);
  const Band by = rg.band;  // by.count <= R::ROWS
  int32_t i_own = z - bz.start;  // the own plane is in its windows: its stage goes first
  i_own += i_own < 0 ? g.grid_d : 0;
  const i32x4_t k_rsrc = head_rsrc(a.k + head * D, head_bytes);
  const i32x4_t v_rsrc = head_rsrc(a.v + head * D, head_bytes);
  load_row_stage<D, R::ROWS>(k_rsrc, v_rsrc, k_lds[0], v_lds[0], z, rg, H, W, head_bytes, wave, tid);

  // scale < 0: Q's sign bits flipped, so c S = scale * (Q K^T) with c = |scale| log2 e
  bf16x8_t qf[KB], gf[KB];
  row_fragment<D>(a.q + head * D, q_row, N, a.q_sign, half, qf);
  row_fragment<D>(a.dout + head * D, q_row, N, 0u, half, gf);

  // window per axis; the lane's columns as the exponent's addend: -lse2 for a key
  // in the window, -inf for the rest (and for a lane outside the grid)
  const GridMasks gm = na_grid_masks(z, imin(y, H - 1), imin(col, W - 1), g);
  const float l2 = q_ok ? a.lse[head + my_q] * kLog2e : 0.f;
  const uint32_t cm16 = q_ok ? lane_block_bits((uint32_t)gm.x0, half) : 0u;
  float add[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) add[e] = ((cm16 >> e) & 1u) ? -l2 : -INFINITY;
  uint32_t rows_vis = 0;  // bit r: band row r in this wavefront's row window
  for (int32_t r = 0; r < by.count; ++r) {
    rows_vis |= (uint32_t)bit128(gm.y0, gm.y1, row_group_row(rg, r)) << r;
  }
  rows_vis = row_in ? __builtin_amdgcn_readfirstlane(rows_vis) : 0u;
  auto next_plane = [&](int32_t j) {  // first visit from j whose plane is in the window (uniform)
    while (j < bz.count &&
           __builtin_amdgcn_readfirstlane((int)bit128(gm.z0, gm.z1, band_plane(bz, i_own, j, g.grid_d))) == 0)
      ++j;
    return j;
  };

  float dlt;
  {
    bf16x8_t of[KB];
    row_fragment<D>(a.o + head * D, q_row, N, 0u, half, of);
    dlt = swap_halves_sum(row_delta_part<D>(of, gf));
    if (q_ok && half == 0) a.delta[head + my_q] = dlt;
  }

  int v_row[2], v_off[2][DT];
  transpose_offsets<D>(lane, half, v_row, v_off);
  const int swz = chunk_swizzle<D>(col);
  f32x16_t dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16_t{};

  for (int32_t i = 0, stage = 0; i < bz.count; stage ^= 1) {
    const int32_t i_next = next_plane(i + 1);
    const bool more = i_next < bz.count;
    wait_tile_loads<0>();  // this stage has landed
    __syncthreads();       // published; the other stage was last read before this barrier
    if (!kSerialTiles && more)
      load_row_stage<D, R::ROWS>(k_rsrc, v_rsrc, k_lds[stage ^ 1], v_lds[stage ^ 1],
                                 band_plane(bz, i_own, i_next, g.grid_d), rg, H, W, head_bytes, wave, tid);
    // the wavefront's visible rows of the stage, in order: the next row's products are
    // issued before this row's exponentials
    const uint16_t* ks = k_lds[stage];
    const uint16_t* vs = v_lds[stage];
    uint32_t rem = rows_vis;
    if (rem != 0u) {
      int32_t r = __builtin_ctz(rem);
      f32x16_t s_nx = block_product<D>(ks + r * 32 * D, 0, col, half, swz, qf);
      f32x16_t dp_nx = block_product<D>(vs + r * 32 * D, 0, col, half, swz, gf);
      while (true) {
        const f32x16_t s = s_nx, dp = dp_nx;
        const int32_t rc = r;
        rem &= rem - 1u;
        const bool nxt = rem != 0u;
        if (nxt) {
          r = __builtin_ctz(rem);
          s_nx = block_product<D>(ks + r * 32 * D, 0, col, half, swz, qf);
          dp_nx = block_product<D>(vs + r * 32 * D, 0, col, half, swz, gf);
        }
        f32x16_t ds;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.c, add[e]));
          ds[e] = p * (dp[e] - dlt);
        }
        bf16x8_t dsb[2];
        to_bf16_operand(ds, dsb);
        block_transpose_product<D>(ks + rc * 32 * D, 0, v_row, v_off, dsb, dq);
        if (!nxt) break;
      }
    }
    if (kSerialTiles && more)  // race check: the next stage's loads only after this stage's compute
      load_row_stage<D, R::ROWS>(k_rsrc, v_rsrc, k_lds[stage ^ 1], v_lds[stage ^ 1],
                                 band_plane(bz, i_own, i_next, g.grid_d), rg, H, W, head_bytes, wave, tid);
    i = i_next;
  }
  store_rows_scaled<D>(a.dq + head * D, q_row, N, half, dq, a.scale);
}

// dK and dV by key rows: a work-group holds 4 key rows of one plane and streams
// the query rows whose windows reach them (na_band_reverse per axis, the key's
// reverse window masks deciding); per visible query row (32 queries) S = Q K^T,
// dP = dO V^T, P = 2^(c s - lse2) (hidden pairs 0), dS = P (dP - D), dV^T +=
// dO^T P, dK^T += Q^T dS. Each stage also holds its queries' lse2 and D.
template <int D, int ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 32 && ROWS <= 8 ? 2 : 1)))
void attn_bwd_dkv_rows_kernel(BwdArgs a) {
  using R = RowStage<D, ROWS>;
  constexpr int KB = D / 16, DT = D / 32, TOK = R::ROWS * 32;
  constexpr int ST = (TOK + 255) / 256;  // statistics per thread and stage (tokens tid + 256 s)
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds[2][R::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t g_lds[2][R::ELEMS];
  __shared__ __attribute__((aligned(16))) float l2_lds[2][TOK];
  __shared__ __attribute__((aligned(16))) float dl_lds[2][TOK];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const NaGeom& g = a.na;
  const int32_t H = g.grid_h, W = g.grid_w, N = a.Nkv;

  const int32_t groups = a.row_groups, per_head = g.grid_d * groups;
  const int32_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int32_t bh = item / per_head, rest = item - bh * per_head;
  const int32_t z = rest / groups;
  const RowGroup rg = na_row_group(g, rest - z * groups, true);
  const int32_t y = rg.rho + rg.stride * (rg.u0 + wave);  // this wavefront's key row
  const bool row_in = rg.u0 + wave < rg.len;
  const bool k_ok = row_in && col < W;
  const int32_t my_k = (z * H + y) * W + col;
  const int32_t k_row = k_ok ? my_k : N;
  const size_t head = (size_t)bh * (size_t)N;
  const uint32_t head_bytes = (uint32_t)N * (uint32_t)(D * 2);

  const Band bz = na_band_reverse(z, z, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d);
  const Band by = rg.band;  // by.count <= R::ROWS
  int32_t i_own = z - bz.start;  // a key's own plane sees it: its stage goes first
  i_own += i_own < 0 ? g.grid_d : 0;
  const i32x4_t q_rsrc = head_rsrc(a.q + head * D, head_bytes);
  const i32x4_t g_rsrc = head_rsrc(a.dout + head * D, head_bytes);
  // lse2 and D of the stage's tokens (thread tid: tokens t = tid + 256 s = 32 r + x), +inf
  // and 0 past the band and the width (P = 0 there)
  auto stats = [&](int32_t zq, float (&l2v)[ST], float (&dlv)[ST]) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int32_t t = tid + 256 * st, r = t / 32, x = t % 32;
      l2v[st] = INFINITY;
      dlv[st] = 0.f;
      if (t < TOK && r < by.count && x < W) {
        const int32_t yq = row_group_row(rg, r);
        const int32_t qi = (zq * H + yq) * W + x;
        l2v[st] = a.lse[head + qi] * kLog2e;
        dlv[st] = a.delta[head + qi];
      }
    }
  };
  auto put_stats = [&](int stage, const float (&l2v)[ST], const float (&dlv)[ST]) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int32_t t = tid + 256 * st;
      if (t < TOK) {
        l2_lds[stage][t] = l2v[st];
        dl_lds[stage][t] = dlv[st];
      }
    }
  };
  load_row_stage<D, R::ROWS>(q_rsrc, g_rsrc, q_lds[0], g_lds[0], z, rg, H, W, head_bytes, wave, tid);
  float l2n[ST], dln[ST];
  stats(z, l2n, dln);

  // scale < 0: K's sign bits flipped, so c S = scale * (Q K^T) with c = |scale| log2 e
  bf16x8_t kf[KB], vf[KB];
  row_fragment<D>(a.k + head * D, k_row, N, a.q_sign, half, kf);
  row_fragment<D>(a.v + head * D, k_row, N, 0u, half, vf);

  // per axis, the queries whose window holds the lane's key; its query columns as a
  // per-element bias (0 or -inf; -inf for every query of a lane outside the grid)
  const GridMasks rm = na_grid_reverse_masks(z, imin(y, H - 1), imin(col, W - 1), g);
  const uint32_t cm16 = k_ok ? lane_block_bits((uint32_t)rm.x0, half) : 0u;
  float bias[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) bias[e] = ((cm16 >> e) & 1u) ? 0.f : -INFINITY;
  uint32_t rows_vis = 0;  // bit r: band query row r reaches this wavefront's key row
  for (int32_t r = 0; r < by.count; ++r) {
    rows_vis |= (uint32_t)bit128(rm.y0, rm.y1, row_group_row(rg, r)) << r;
  }
  rows_vis = row_in ? __builtin_amdgcn_readfirstlane(rows_vis) : 0u;
  auto next_plane = [&](int32_t j) {
    while (j < bz.count &&
           __builtin_amdgcn_readfirstlane((int)bit128(rm.z0, rm.z1, band_plane(bz, i_own, j, g.grid_d))) == 0)
      ++j;
    return j;
  };

  int v_row[2], v_off[2][DT];
  transpose_offsets<D>(lane, half, v_row, v_off);
  const int swz = chunk_swizzle<D>(col);
  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16_t{};

  put_stats(0, l2n, dln);  // the first stage's statistics (published by the loop's first barrier)
  for (int32_t i = 0, stage = 0; i < bz.count; stage ^= 1) {
    const int32_t i_next = next_plane(i + 1);
    const bool more = i_next < bz.count;
    const int32_t z_next = more ? band_plane(bz, i_own, i_next, g.grid_d) : 0;
    wait_tile_loads<0>();
    __syncthreads();
    if (!kSerialTiles && more) {
      load_row_stage<D, R::ROWS>(q_rsrc, g_rsrc, q_lds[stage ^ 1], g_lds[stage ^ 1], z_next, rg, H, W, head_bytes,
                                 wave, tid);
      stats(z_next, l2n, dln);
    }
    const uint16_t* qs = q_lds[stage];
    const uint16_t* gs = g_lds[stage];
    uint32_t rem = rows_vis;
    if (rem != 0u) {
      int32_t r = __builtin_ctz(rem);
      f32x16_t s_nx = block_product<D>(qs + r * 32 * D, 0, col, half, swz, kf);
      f32x16_t dp_nx = block_product<D>(gs + r * 32 * D, 0, col, half, swz, vf);
      while (true) {
        const f32x16_t s = s_nx, dp = dp_nx;
        const int32_t rc = r;
        rem &= rem - 1u;
        const bool nxt = rem != 0u;
        if (nxt) {
          r = __builtin_ctz(rem);
          s_nx = block_product<D>(qs + r * 32 * D, 0, col, half, swz, kf);
          dp_nx = block_product<D>(gs + r * 32 * D, 0, col, half, swz, vf);
        }
        f32x16_t p, ds;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qr = rc * 32 + 8 * g4 + 4 * half;  // first of the 4 queries of this group
          const float4 l4 = *reinterpret_cast<const float4*>(&l2_lds[stage][qr]);
          const float4 d4 = *reinterpret_cast<const float4*>(&dl_lds[stage][qr]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * g4 + j;
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.c, bias[e] - lv[j]));
            p[e] = pv;
            ds[e] = pv * (dp[e] - dv4[j]);
          }
        }
        bf16x8_t pb[2], dsb[2];
        to_bf16_operand(p, pb);
        to_bf16_operand(ds, dsb);
        block_transpose_product<D>(gs + rc * 32 * D, 0, v_row, v_off, pb, dv);
        block_transpose_product<D>(qs + rc * 32 * D, 0, v_row, v_off, dsb, dk);
        if (!nxt) break;
      }
    }
    if (kSerialTiles && more) {  // race check: the next stage's loads only after this stage's compute
      load_row_stage<D, R::ROWS>(q_rsrc, g_rsrc, q_lds[stage ^ 1], g_lds[stage ^ 1], z_next, rg, H, W, head_bytes,
                                 wave, tid);
      stats(z_next, l2n, dln);
    }
    if (more) put_stats(stage ^ 1, l2n, dln);  // the other stage's were last read before this step's barrier
    i = i_next;
  }
  store_rows_scaled<D>(a.dk + head * D, k_row, N, half, dk, a.scale);
  store_rows_scaled<D>(a.dv + head * D, k_row, N, half, dv, 1.0f);
}

// ---------------------------------------------------------------------------
// Neighbourhood windows of one plane by 8 x 16 patches (na_patch_bwd_eligible),
// the forward patch kernel's layout: the dQ kernel holds a patch of queries and
// copies the key rectangle its windows reach (K and V) into LDS once; the dK/dV
// kernel holds a patch of keys and copies the rectangle of queries whose windows
// reach them (Q, dO and their lse2 and D). Wavefront w holds the patch's rows 2w
// and 2w + 1 (lane column col: row col / 16, column col % 16) and walks the band
// rows of those two rows in the rectangle; each query wavefront has a second
// wavefront on its SIMD that takes every other row (two parts, summed at the end
// through LDS). Window bits per lane: its columns over the rectangle's column
// cells (an exponent addend per element) and its rows over the rectangle's rows.

template <int D>
struct BwdPatchCfg {
  static constexpr int ROWS = bwd_patch_lds(D);  // rows of 32 tokens per rectangle
  // d = 32: two wavefronts per SIMD (the parts); d = 64: the rectangles take 136-140 KB,
  // so one work-group of one wavefront per SIMD, which then gets the whole register file
  static constexpr int PARTS = D == 32 ? 2 : 1;
  static constexpr int WAVES_PER_EU = PARTS;
  static constexpr int THREADS = 256 * PARTS;
  static constexpr int RC = D / 8;
  static constexpr int CHUNKS = ROWS * kPatchKeyCols * RC;
  static_assert(ROWS > 0 && CHUNKS % THREADS == 0, "the copy runs in whole rounds of the work-group's lanes");
  static constexpr int ELEMS = CHUNKS * 8;
};

// Copies the rectangle (rows x cols band cells, each mod its axis) of two tensors of
// one head into LDS: chunk p holds chunk (p % RC) ^ swizzle of token p / RC = 32 r +
// x (row cell r, column cell x); columns past the column band read as zero.
template <int D>
__device__ __forceinline__ void load_patch_rect(i32x4_t ra, i32x4_t rb, const uint16_t* la, const uint16_t* lb,
                                                const PatchBands& pb, const PatchGroup& pr, int32_t H, int32_t W,
                                                uint32_t head_bytes, int wave8, int tid) {
  using P = BwdPatchCfg<D>;
  const uint32_t a_base = __builtin_amdgcn_readfirstlane(lds_addr(la) + wave8 * 1024);
  const uint32_t b_base = __builtin_amdgcn_readfirstlane(lds_addr(lb) + wave8 * 1024);
  const int32_t n_loads = (int32_t)cdiv((int64_t)pb.rows.count * kPatchKeyCols * P::RC, P::THREADS);
  for (int32_t j = 0; j < n_loads; ++j) {
    const int32_t p = j * P::THREADS + tid;
    const int32_t tok = p / P::RC, r = tok / kPatchKeyCols, x = tok % kPatchKeyCols;
    const int32_t chunk = (p % P::RC) ^ chunk_swizzle<D>(tok);
    uint32_t voff = head_bytes;
    if (r < pb.rows.count && x < pb.cols.count) {
      int32_t ty = pb.rows.start + r, tx = pb.cols.start + x;
      ty -= ty >= H ? H : 0;  // both start inside the axis and span at most its length
      tx -= tx >= W ? W : 0;
      voff = (uint32_t)patch_token(pr, ty, tx) * (uint32_t)(D * 2) + (uint32_t)chunk * 16u;
    }
    dma_lds16(ra, a_base + (uint32_t)j * (P::THREADS * 16u), voff, 0u);
    dma_lds16(rb, b_base + (uint32_t)j * (P::THREADS * 16u), voff, 0u);
  }
}

// The lane's column bits of a 32-token block, in accumulator element order.
__device__ __forceinline__ uint32_t block_elem_bits(uint32_t cm, int half) {
  uint32_t m = 0;
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) m |= ((cm >> (8 * g4 + 4 * half)) & 0xFu) << (4 * g4);
  return m;
}

// dQ by query patches; also forms D of its queries for the dK/dV kernel.
template <int D>
__global__ __launch_bounds__(BwdPatchCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(BwdPatchCfg<D>::WAVES_PER_EU)))
void attn_bwd_dq_patch_kernel(BwdArgs a) {
  using P = BwdPatchCfg<D>;
  constexpr int KB = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[P::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[P::ELEMS];
  __shared__ float merge_lds[P::PARTS > 1 ? 4 * DT * 16 * 64 : 1];  // the second part's dQ
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wave8 & 3, part = wave8 >> 2;
  const int32_t per_head = a.patch_ny * a.patch_nx;
  const int32_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int32_t bh = item / per_head, pidx = item - bh * per_head;
  const int32_t py = pidx / a.patch_nx;
  // rows and columns in the coordinates of the patch's sub-grids (na_patch_group)
  const PatchGroup pr = na_patch_group(a.na, py, pidx - py * a.patch_nx, a.patch_cols_strided != 0);
  const NaGeom& g = pr.geom;
  const int32_t H = g.grid_h, W = g.grid_w, N = a.Nq;
  const int32_t y0 = pr.u0, x0 = pr.v0;
  const PatchBands pb = na_patch_bands(y0, x0, g);
  const size_t head = (size_t)bh * (size_t)N;
  const uint32_t head_bytes = (uint32_t)N * (uint32_t)(D * 2);
  load_patch_rect<D>(head_rsrc(a.k + head * D, head_bytes), head_rsrc(a.v + head * D, head_bytes), k_lds, v_lds, pb,
                     pr, H, W, head_bytes, wave8, tid);

  const int32_t qy = y0 + 2 * wave + (col >> 4), qx = x0 + (col & 15);
  const bool q_ok = qy < H && qx < W;
  const int32_t my_q = patch_token(pr, qy, qx);
  const int32_t q_row = q_ok ? my_q : N;
  bf16x8_t qf[KB], gf[KB];
  row_fragment<D>(a.q + head * D, q_row, N, a.q_sign, half, qf);
  row_fragment<D>(a.dout + head * D, q_row, N, 0u, half, gf);
  const float l2 = q_ok ? a.lse[head + my_q] * kLog2e : 0.f;
  float dlt;
  {
    bf16x8_t of[KB];
    row_fragment<D>(a.o + head * D, q_row, N, 0u, half, of);
    dlt = swap_halves_sum(row_delta_part<D>(of, gf));
    if (part == 0 && q_ok && half == 0) a.delta[head + my_q] = dlt;
  }
  // window bits: key column cells of the rectangle, key rows of the rectangle
  const int32_t cy = imin(qy, H - 1), cx = imin(qx, W - 1);
  const uint32_t cm = block_elem_bits(band_window_bits(cx, pb.cols, W, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w, false),
                                      half);
  const uint32_t rows_w = band_window_bits(cy, pb.rows, H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h, false);
  float add[16];  // -lse2 for a key column in the window, -inf otherwise (and for a lane outside the grid)
#pragma unroll
  for (int e = 0; e < 16; ++e) add[e] = q_ok && ((cm >> e) & 1u) ? -l2 : -INFINITY;
  // this wavefront's rows: the band of its two query rows, a run of the rectangle's band
  const bool rows_in = y0 + 2 * wave < H;
  const int32_t wy0 = imin(y0 + 2 * wave, H - 1);
  const Band wb = na_band(wy0, imin(wy0 + 1, H - 1), H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h);
  int32_t off = wb.start - pb.rows.start;
  off += off < 0 ? H : 0;
  const int32_t end = rows_in ? off + wb.count : 0;

  int v_row[2], v_off[2][DT];
  transpose_offsets<D>(lane, half, v_row, v_off);
  const int swz = chunk_swizzle<D>(col);
  f32x16_t dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16_t{};

  wait_tile_loads<0>();
  __syncthreads();  // the rectangle is read-only from here on
  // rows off + part, off + part + 2, ... that some lane of the wavefront sees
  auto next_row = [&](int32_t r) {
    while (r < end && __builtin_amdgcn_ballot_w64(((rows_w >> r) & 1u) != 0u) == 0) r += P::PARTS;
    return r;
  };
  int32_t r = next_row(off + part);
  if (r < end) {
    f32x16_t s_nx = block_product<D>(k_lds + r * 32 * D, 0, col, half, swz, qf);
    f32x16_t dp_nx = block_product<D>(v_lds + r * 32 * D, 0, col, half, swz, gf);
    while (true) {
      const f32x16_t s = s_nx, dp = dp_nx;
      const int32_t rc = r;
      r = next_row(r + P::PARTS);
      const bool nxt = r < end;
      if (nxt) {
        s_nx = block_product<D>(k_lds + r * 32 * D, 0, col, half, swz, qf);
        dp_nx = block_product<D>(v_lds + r * 32 * D, 0, col, half, swz, gf);
      }
      const bool live = ((rows_w >> rc) & 1u) != 0u;
      f32x16_t ds;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.c, live ? add[e] : -INFINITY));
        ds[e] = p * (dp[e] - dlt);
      }
      bf16x8_t dsb[2];
      to_bf16_operand(ds, dsb);
      block_transpose_product<D>(k_lds + rc * 32 * D, 0, v_row, v_off, dsb, dq);
      if (!nxt) break;
    }
  }
  if constexpr (P::PARTS > 1) {  // the second part's sums join the first's (lane order), which stores
    float* slot = merge_lds + wave * DT * 16 * 64 + lane;
    if (part == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) slot[(dt * 16 + e) * 64] = dq[dt][e];
    }
    __syncthreads();
    if (part == 1) return;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[dt][e] += slot[(dt * 16 + e) * 64];
  }
  store_rows_scaled<D>(a.dq + head * D, q_row, N, half, dq, a.scale);
}

// dK and dV by key patches over the rectangle of queries whose windows reach them.
template <int D>
__global__ __launch_bounds__(BwdPatchCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(BwdPatchCfg<D>::WAVES_PER_EU)))
void attn_bwd_dkv_patch_kernel(BwdArgs a) {
  using P = BwdPatchCfg<D>;
  constexpr int KB = D / 16, DT = D / 32, TOK = P::ROWS * kPatchKeyCols;
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds[P::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t g_lds[P::ELEMS];
  __shared__ __attribute__((aligned(16))) float l2_lds[TOK];
  __shared__ __attribute__((aligned(16))) float dl_lds[TOK];
  __shared__ float merge_lds[P::PARTS > 1 ? 4 * 2 * DT * 16 * 64 : 1];  // the second part's dK and dV
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wave8 & 3, part = wave8 >> 2;
  const int32_t per_head = a.patch_ny * a.patch_nx;
  const int32_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int32_t bh = item / per_head, pidx = item - bh * per_head;
  const int32_t py = pidx / a.patch_nx;
  // rows and columns in the coordinates of the patch's sub-grids (na_patch_group)
  const PatchGroup pr = na_patch_group(a.na, py, pidx - py * a.patch_nx, a.patch_cols_strided != 0);
  const NaGeom& g = pr.geom;
  const int32_t H = g.grid_h, W = g.grid_w, N = a.Nkv;
  const int32_t y0 = pr.u0, x0 = pr.v0;
  const PatchBands pb = na_patch_reverse_bands(y0, x0, g);
  const size_t head = (size_t)bh * (size_t)N;
  const uint32_t head_bytes = (uint32_t)N * (uint32_t)(D * 2);
  load_patch_rect<D>(head_rsrc(a.q + head * D, head_bytes), head_rsrc(a.dout + head * D, head_bytes), q_lds, g_lds,
                     pb, pr, H, W, head_bytes, wave8, tid);
  // lse2 and D of the rectangle's queries (+inf and 0 past its bands: P = 0 there)
  for (int32_t t = tid; t < TOK; t += P::THREADS) {
    const int32_t r = t / kPatchKeyCols, x = t % kPatchKeyCols;
    float l2v = INFINITY, dlv = 0.f;
    if (r < pb.rows.count && x < pb.cols.count) {
      int32_t ty = pb.rows.start + r, tx = pb.cols.start + x;
      ty -= ty >= H ? H : 0;
      tx -= tx >= W ? W : 0;
      const int32_t qi = patch_token(pr, ty, tx);
      l2v = a.lse[head + qi] * kLog2e;
      dlv = a.delta[head + qi];
    }
    l2_lds[t] = l2v;
    dl_lds[t] = dlv;
  }

  const int32_t ky = y0 + 2 * wave + (col >> 4), kx = x0 + (col & 15);
  const bool k_ok = ky < H && kx < W;
  const int32_t my_k = patch_token(pr, ky, kx);
  const int32_t k_row = k_ok ? my_k : N;
  // scale < 0: K's sign bits flipped, so c S = scale * (Q K^T) with c = |scale| log2 e
  bf16x8_t kf[KB], vf[KB];
  row_fragment<D>(a.k + head * D, k_row, N, a.q_sign, half, kf);
  row_fragment<D>(a.v + head * D, k_row, N, 0u, half, vf);
  // window bits: the rectangle's query columns and rows whose windows hold the lane's key
  const int32_t cy = imin(ky, H - 1), cx = imin(kx, W - 1);
  const uint32_t cm = block_elem_bits(band_window_bits(cx, pb.cols, W, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w, true),
                                      half);
  const uint32_t rows_w = band_window_bits(cy, pb.rows, H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h, true);
  float bias[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) bias[e] = k_ok && ((cm >> e) & 1u) ? 0.f : -INFINITY;
  const bool rows_in = y0 + 2 * wave < H;
  const int32_t wy0 = imin(y0 + 2 * wave, H - 1);
  const Band wb = na_band_reverse(wy0, imin(wy0 + 1, H - 1), H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h);
  int32_t off = wb.start - pb.rows.start;
  off += off < 0 ? H : 0;
  const int32_t end = rows_in ? off + wb.count : 0;

  int v_row[2], v_off[2][DT];
  transpose_offsets<D>(lane, half, v_row, v_off);
  const int swz = chunk_swizzle<D>(col);
  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16_t{};

  wait_tile_loads<0>();
  __syncthreads();  // the rectangle and its statistics are read-only from here on
  auto next_row = [&](int32_t r) {
    while (r < end && __builtin_amdgcn_ballot_w64(((rows_w >> r) & 1u) != 0u) == 0) r += P::PARTS;
    return r;
  };
  int32_t r = next_row(off + part);
  if (r < end) {
    f32x16_t s_nx = block_product<D>(q_lds + r * 32 * D, 0, col, half, swz, kf);
    f32x16_t dp_nx = block_product<D>(g_lds + r * 32 * D, 0, col, half, swz, vf);
    while (true) {
      const f32x16_t s = s_nx, dp = dp_nx;
      const int32_t rc = r;
      r = next_row(r + P::PARTS);
      const bool nxt = r < end;
      if (nxt) {
        s_nx = block_product<D>(q_lds + r * 32 * D, 0, col, half, swz, kf);
        dp_nx = block_product<D>(g_lds + r * 32 * D, 0, col, half, swz, vf);
      }
      const bool live = ((rows_w >> rc) & 1u) != 0u;
      f32x16_t p, ds;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qr = rc * 32 + 8 * g4 + 4 * half;  // first of the 4 queries of this group
        const float4 l4 = *reinterpret_cast<const float4*>(&l2_lds[qr]);
        const float4 d4 = *reinterpret_cast<const float4*>(&dl_lds[qr]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * g4 + j;
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.c, live ? bias[e] - lv[j] : -INFINITY));
          p[e] = pv;
          ds[e] = pv * (dp[e] - dv4[j]);
        }
      }
      bf16x8_t pb2[2], dsb[2];
      to_bf16_operand(p, pb2);
      to_bf16_operand(ds, dsb);
      block_transpose_product<D>(g_lds + rc * 32 * D, 0, v_row, v_off, pb2, dv);
      block_transpose_product<D>(q_lds + rc * 32 * D, 0, v_row, v_off, dsb, dk);
      if (!nxt) break;
    }
  }
  if constexpr (P::PARTS > 1) {
    float* slot = merge_lds + wave * 2 * DT * 16 * 64 + lane;
    if (part == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          slot[(dt * 16 + e) * 64] = dk[dt][e];
          slot[((DT + dt) * 16 + e) * 64] = dv[dt][e];
        }
    }
    __syncthreads();
    if (part == 1) return;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dk[dt][e] += slot[(dt * 16 + e) * 64];
        dv[dt][e] += slot[((DT + dt) * 16 + e) * 64];
      }
  }
  store_rows_scaled<D>(a.dk + head * D, k_row, N, half, dk, a.scale);
  store_rows_scaled<D>(a.dv + head * D, k_row, N, half, dv, 1.0f);
}

static_assert(BwdCfg<32>::WAVES_PER_EU == bwd_wgs_per_cu(32) && BwdCfg<64>::WAVES_PER_EU == bwd_wgs_per_cu(64) &&
                  BwdCfg<128>::WAVES_PER_EU == bwd_wgs_per_cu(128),
              "one wavefront per SIMD per work-group: waves per SIMD = work-groups per CU");

template <int D, int MASK>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  bool dq_rows = false, dkv_rows = false, dq_patch = false, dkv_patch = false;
  if constexpr (MASK == MASK_NA && (D == 32 || D == 64)) {
    dq_rows = a.dq_rows != 0;
    dkv_rows = a.dkv_rows != 0;
  }
  if constexpr (MASK == MASK_NA && (D == 32 || D == 64)) {
    dq_patch = !dq_rows && a.dq_patch != 0;
    dkv_patch = !dkv_rows && a.dkv_patch != 0;
  }
  const dim3 rows_grid(dq_rows || dkv_rows ? a.BH * a.na.grid_d * a.row_groups : 1);
  const dim3 patch_grid(dq_patch || dkv_patch ? a.BH * a.patch_nx * a.patch_ny : 1);
  if constexpr (MASK == MASK_NA && (D == 32 || D == 64)) {
    if (dq_rows && a.dq_rows == bwd_dq_rows_lds(D))
      hipLaunchKernelGGL((attn_bwd_dq_rows_kernel<D, bwd_dq_rows_lds(D)>), rows_grid, dim3(256), 0, stream, a);
    if constexpr (rows_wide_lds(D) > 0) {
      if (dq_rows && a.dq_rows == rows_wide_lds(D))
        hipLaunchKernelGGL((attn_bwd_dq_rows_kernel<D, rows_wide_lds(D)>), rows_grid, dim3(256), 0, stream, a);
    }
  }
  if constexpr (MASK == MASK_NA && (D == 32 || D == 64)) {
    if (dq_patch)
      hipLaunchKernelGGL((attn_bwd_dq_patch_kernel<D>), patch_grid, dim3(BwdPatchCfg<D>::THREADS), 0, stream, a);
  }
  if (!dq_rows && !dq_patch)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, MASK>), dim3(a.BH * a.n_qtiles), dim3(BwdCfg<D>::THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (MASK == MASK_NA && (D == 32 || D == 64)) {
    if (dkv_rows && a.dkv_rows == bwd_dkv_rows_lds(D))
      hipLaunchKernelGGL((attn_bwd_dkv_rows_kernel<D, bwd_dkv_rows_lds(D)>), rows_grid, dim3(256), 0, stream, a);
    if constexpr (rows_wide_lds(D) > 0) {
      if (dkv_rows && a.dkv_rows == rows_wide_lds(D))
        hipLaunchKernelGGL((attn_bwd_dkv_rows_kernel<D, rows_wide_lds(D)>), rows_grid, dim3(256), 0, stream, a);
    }
  }
  if constexpr (MASK == MASK_NA && (D == 32 || D == 64)) {
    if (dkv_patch)
      hipLaunchKernelGGL((attn_bwd_dkv_patch_kernel<D>), patch_grid, dim3(BwdPatchCfg<D>::THREADS), 0, stream, a);
  }
  if (!dkv_rows && !dkv_patch)
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, MASK>), dim3(a.BH * a.n_ktiles), dim3(BwdCfg<D>::THREADS), 0, stream,
                       a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_mask(const BwdArgs& a, int32_t mask, hipStream_t stream) {
  switch (mask) {
    case MASK_NONE: return launch_bwd_d<D, MASK_NONE>(a, stream);
    case MASK_CAUSAL: return launch_bwd_d<D, MASK_CAUSAL>(a, stream);
    case MASK_NA: return launch_bwd_d<D, MASK_NA>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdArgs& a, int32_t d, int32_t mask, hipStream_t stream) {
  if (d == 64) return launch_bwd_mask<64>(a, mask, stream);
  if (d == 32) return launch_bwd_mask<32>(a, mask, stream);
  if (d == 128) return launch_bwd_mask<128>(a, mask, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
