// Fused exact-attention forward for gfx950 (MI355X, CDNA4).
//
// O = softmax(scale * Q K^T + mask) V per (batch, head), computed one query
// tile at a time without writing the N x N score matrix anywhere: the
// scores of each key tile are reduced on the fly with a running row maximum
// and row sum, and the division by the row sum happens once, after the
// product with V (AWS Neuron NKI tutorial "Fused Self Attention", sections
// "Fusion to Save SBUF Space" and "Softmax implementation"; PhotoRoom's
// xformers post, the running-softmax paragraph).
//
// Work decomposition: one work-group = 4 wavefronts = one tile of 128
// queries of one head; each wavefront owns 32 queries. Key/value tiles of
// 128 tokens (64 at d = 128) stream through LDS rings (2 tiles deep at d = 64
// and 128, 4 at d = 32) shared by the 4 wavefronts; later tiles' global loads are in flight while
// the current tile is computed. An unmasked launch may instead run a round of
// whole tiles plus key-range parts of the remaining tiles, each tile's parts
// merged by the last of them to finish (remainder split, tile_plan.hpp).
//
// Per key tile and wavefront:
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, K from LDS (A operand), Q held
//                   in registers for the whole loop (B operand). Each lane then
//                   holds 16 keys of one query column per 32-key block, so
//                   row reductions are in-lane plus one exchange between the
//                   two half-waves (v_permlane32_swap).
//   reference max   P is taken against a reference maximum m (base 2, with
//                   c = |scale| * log2(e)); m only moves, with O and l rescaled
//                   by 2^(m_old - m_new), when a tile's row sum shows that some
//                   probability would pass 2^20 (see kSafeSum).
//   P = 2^(c S - m) fp32, rounded to bfloat16 for the second product;
//                   l = l + rowsum of the rounded P, kept per lane.
//   O^T = V^T P^T   v_mfma_f32_32x32x16_bf16 with P straight from registers
//                   (B operand) and V read from LDS with ds_read_b64_tr_b16,
//                   which hands each lane 4 consecutive keys of one d column.
//                   The key order inside a 16-key MFMA block follows the
//                   accumulator layout of S^T; the V reads use the same order.
// Finally O / l (delayed division), rounded to bfloat16 (nearest even).
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "attn.h"
#include "kernel_common.hpp"
#include "launch.hpp"
#include "tile_plan.hpp"


namespace attn {

template <int D>
struct Cfg {
  static constexpr int BM = 128;     // queries per work-group (4 wavefronts x 32)
  static constexpr int BN = D == 128 ? 64 : 128;  // keys per tile (16 KB of K or V at d = 64 and 128)
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROW_CHUNKS = D / 8;                     // 16-byte chunks per K or V row
  static constexpr int TILE = BN * D;                          // 16-bit elements per K or V tile
  static constexpr int LOADS = BN * ROW_CHUNKS / THREADS;      // 16-byte loads per thread per tile
  static_assert(BN * ROW_CHUNKS % THREADS == 0, "tile chunks must split evenly");
  // Buffers of each of the K and V rings: 64 KB of LDS in both cases, so two
  // work-groups fit per CU. A tile's loads are issued STAGES - 1 steps before the
  // step that reads it (d = 32 steps are short, so their tiles start earlier).
  static constexpr int STAGES = D == 32 ? 4 : 2;
  static_assert((STAGES & (STAGES - 1)) == 0, "ring indices use a mask");
  // 16-byte loads a wavefront may still have in flight at the end of a step: those
  // of the STAGES - 2 later steps (each step issues one K and one V tile).
  static constexpr int LOADS_AHEAD = (STAGES - 2) * 2 * LOADS;
};

static_assert(Cfg<128>::BM == kBlockM && Cfg<64>::BM == kBlockM && Cfg<32>::BM == kBlockM,
              "launch geometry and kernel tile must agree");
static_assert(Cfg<128>::BN == tile_keys(128) && Cfg<64>::BN == tile_keys(64) && Cfg<32>::BN == tile_keys(32),
              "host tile counts and kernel tiles must agree");

template <int D>
struct TileLoader {
  using C = Cfg<D>;
  uint32_t voff[C::LOADS];  // byte offset of this lane's chunk inside a tile
  int wave;                 // wave index (uniform)

  __device__ __forceinline__ TileLoader(int wave_, int lane) : wave(wave_) {
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int p = (j * C::WAVES + wave_) * 64 + lane;
      const int row = p / C::ROW_CHUNKS;
      const int chunk = (p % C::ROW_CHUNKS) ^ chunk_swizzle<D>(row);
      voff[j] = (uint32_t)(row * D + chunk * 8) * 2u;
    }
  }

  // One of the LOADS 16-byte loads of a tile (lets a step spread its loads out).
  __device__ __forceinline__ void load_part(i32x4_t src, int32_t tile, const uint16_t* lds_tile, int j) const {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)tile * (uint32_t)(C::BN * D * 2));
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds_tile) + wave * 1024);
    dma_lds16(src, base + j * C::WAVES * 1024, voff[j], soff);
  }

  __device__ __forceinline__ void load(i32x4_t src, int32_t tile, const uint16_t* lds_tile) const {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)tile * (uint32_t)(C::BN * D * 2));
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds_tile) + wave * 1024);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) dma_lds16(src, base + j * C::WAVES * 1024, voff[j], soff);
  }
};



// Probabilities are computed against a reference maximum m that is only moved
// when a lane's row sum for a tile exceeds 2^20 (which bounds every probability
// of the tile by 2^20), so the rescale of O is rare. Any reference gives the
// same O / l; moving it only keeps the sums far from overflow.
constexpr float kSafeSum = 1048576.0f;

// Natural-log logsumexp of a row from its reference maximum m (base 2, scale
// folded in) and the sum l of its probabilities 2^(c s - m): ln 2 * (m + log2 l);
// -inf when no key was visible (l = 0).
__device__ __forceinline__ float row_lse(float m, float l) {
  return l > 0.f ? 0.69314718055994531f * (m + log2f(l)) : -INFINITY;
}

// Partial result of one part of a shared query tile, in the lanes' own register
// order so that each write or read instruction moves one contiguous 1 KB row:
//   o[wave][dt][g][lane][4]  unnormalised output: the lane's oacc[dt][4g .. 4g + 3]
//   m[wave][lane]            reference maximum of the lane's query (base 2, scaled)
//   l[wave][lane]            sum of the probabilities of the lane's keys
template <int D>
struct PartSlot {
  static constexpr int DT = D / 32;
  static constexpr int M = 4 * DT * 4 * 64 * 4;
  static constexpr int L = M + 4 * 64;
  static constexpr int FLOATS = L + 4 * 64;
};
static_assert(PartSlot<128>::FLOATS * 4 == part_slot_bytes(128) && PartSlot<64>::FLOATS * 4 == part_slot_bytes(64) &&
                  PartSlot<32>::FLOATS * 4 == part_slot_bytes(32),
              "workspace slot size and kernel layout must agree");

// A part's slot is written and read with device-coherent accesses (the sc1
// cache policy: stores write through the XCD's L2, loads read past it), so the
// parts of a tile meet across XCDs without a writeback or invalidation of a
// whole L2 (the agent-scope fences, which measured 1.25x slower on SD2.1-512).
constexpr int kCoherent = 16;  // buffer cache-policy bit sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int D>
__device__ __forceinline__ void write_part(float* slot, int wave, int lane, const f32x16_t (&o)[D / 32], float m,
                                           float l) {
  const __amdgpu_buffer_rsrc_t rs = slot_rsrc(slot, PartSlot<D>::FLOATS * 4);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4_t x = {__float_as_uint(o[dt][4 * g]), __float_as_uint(o[dt][4 * g + 1]),
                         __float_as_uint(o[dt][4 * g + 2]), __float_as_uint(o[dt][4 * g + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(x, rs, (((wave * (D / 32) + dt) * 4 + g) * 64 + lane) * 16, 0, kCoherent);
    }
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), rs, (PartSlot<D>::M + wave * 64 + lane) * 4, 0, kCoherent);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rs, (PartSlot<D>::L + wave * 64 + lane) * 4, 0, kCoherent);
}

// Combines the parts of split tile r and stores the tile (run by the work-group
// of its last part to finish). Wavefront w takes the tile's rows 32 w .. 32 w +
// 31 with the lanes of write_part. Every part is rescaled to the largest of the
// parts' maxima and the parts are summed in part order, so the result does not
// depend on which part finished last; then the division by the row sum and the
// bfloat16 store of a whole tile. Parts are read one at a time (the registers
// hold one part's rows and the sums).
template <int D>
__device__ __forceinline__ void merge_parts(const KernelArgs& a, int32_t r, int wave, int lane) {
  constexpr int DT = D / 32;
  constexpr uint32_t SLOT = PartSlot<D>::FLOATS * 4;  // bytes
  const int col = lane & 31, half = lane >> 5;
  const int32_t parts = a.split_parts;
  const __amdgpu_buffer_rsrc_t rs = slot_rsrc(a.ws_parts + (size_t)r * parts * PartSlot<D>::FLOATS, parts * SLOT);
  const uint32_t row = (wave * 64 + lane) * 4;
  float m = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, PartSlot<D>::M * 4 + row, 0, kCoherent));
  for (int32_t p = 1; p < parts; ++p)
    m = fmaxf(m, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, p * SLOT + PartSlot<D>::M * 4 + row, 0,
                                                                      kCoherent)));
  float l = 0.f;
  float o[DT][16];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  for (int32_t p = 0; p < parts; ++p) {
    u32x4_t x[DT][4];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        x[dt][g] = __builtin_amdgcn_raw_buffer_load_b128(rs, p * SLOT + (((wave * DT + dt) * 4 + g) * 64 + lane) * 16,
                                                         0, kCoherent);
    const float mp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, p * SLOT + PartSlot<D>::M * 4 + row, 0,
                                                                          kCoherent));
    const float lp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, p * SLOT + PartSlot<D>::L * 4 + row, 0,
                                                                          kCoherent));
    const float w = __builtin_amdgcn_exp2f(mp - m);
    l += w * lp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][4 * g + e] += w * __uint_as_float(x[dt][g][e]);
  }
  const int32_t tile = a.split_full + r;
  const int32_t bh = tile / a.n_qtiles, qtile = tile - bh * a.n_qtiles;
  const int32_t my_q = qtile * Cfg<D>::BM + wave * 32 + col;
  const float l_tot = swap_halves_sum(l);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (my_q < a.Nq) {
    if (a.lse != nullptr && half == 0) a.lse[(size_t)bh * a.Nq + my_q] = row_lse(m, l_tot);
    uint16_t* __restrict__ oh = a.o + (size_t)bh * (size_t)a.Nq * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4_t ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(o[dt][g * 4 + e] * inv);
        *reinterpret_cast<u32x2_t*>(oh + (size_t)my_q * D + dt * 32 + g * 8 + half * 4) = __builtin_bit_cast(u32x2_t, ob);
      }
  }
}

// Zeroes the arrival counters of a split launch (queued just before it).
__global__ __launch_bounds__(256) void attn_split_clear_kernel(uint32_t* count, int32_t n) {
  for (int32_t i = threadIdx.x; i < n; i += 256) count[i] = 0u;
}

template <int D, int MASK, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(KernelArgs a) {
  using C = Cfg<D>;
  constexpr int KB = D / 16;      // 16-wide contraction blocks over d for S^T
  constexpr int DT = D / 32;      // 32-row output tiles over d for O^T
  constexpr int SB = C::BN / 32;  // 32-key blocks per key tile

  constexpr int S = C::STAGES;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[S][C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[S][C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column owned by this lane
  const int half = lane >> 5;  // which half-wave

  const int32_t Nq = a.Nq, Nkv = a.Nkv;
  const int32_t n_kv = a.n_kvtiles;
  const float c = a.c;
  const TileLoader<D> ld(__builtin_amdgcn_readfirstlane(wave), lane);
  const uint32_t head_bytes = (uint32_t)Nkv * (uint32_t)(D * 2);

  // LDS offsets that depend only on the lane
  const int k_swz = chunk_swizzle<D>(col);  // rows sb*32 + col share it
  int v_row[2], v_off[2][DT];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v_row[h] = h * 8 + half * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dcol = dt * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
      v_off[h][dt] = (((dcol >> 3) ^ chunk_swizzle<D>(v_row[h])) << 3) + (dcol & 7);
    }
  }

  // One query tile of head bh against the key tiles of `run`: leaves the
  // unnormalised output (O^T rows of the lane's query), the reference maximum
  // and the lane's row sum. No LDS DMA is in flight on return (the clamped refills
  // past the run are awaited at its end).
  auto segment = [&](const int32_t bh, const int32_t qtile, const KvRun run, f32x16_t (&oacc)[DT], float& m_run,
                     float& l_run) {
  const int32_t q0 = qtile * C::BM;
  const uint16_t* __restrict__ qh = a.q + (size_t)bh * (size_t)Nq * D;
  const uint16_t* __restrict__ kh = a.k + (size_t)bh * (size_t)Nkv * D;
  const uint16_t* __restrict__ vh = a.v + (size_t)bh * (size_t)Nkv * D;

  // ---- Q fragment: B operand of S^T = K Q^T; lane holds d = 16kb + 8*half + 0..7 of its query
  const int32_t my_q = q0 + wave * 32 + col;
  bf16x8_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    u32x4_t x = u32x4_t{0, 0, 0, 0};
    if (my_q < Nq) {
      x = *reinterpret_cast<const u32x4_t*>(qh + (size_t)my_q * D + kb * 16 + half * 8);
      x ^= a.q_sign;  // negative scale: flip Q's sign bits, use |scale|
    }
    qf[kb] = __builtin_bit_cast(bf16x8_t, x);
  }

  // the query's grid coordinates and, for dilated windows, its per-axis anchors (na_dil_anchor)
  int32_t zq = 0, yq = 0, xq = 0, az = 0, ay = 0, ax = 0;
  if (is_na(MASK)) {
    const int32_t plane = a.na.grid_h * a.na.grid_w;
    zq = my_q / plane;
    const int32_t rq = my_q - zq * plane;
    yq = rq / a.na.grid_w;
    xq = rq - yq * a.na.grid_w;
    az = na_dil_anchor(zq, a.na.grid_d, a.na.kernel_d, a.na.rad_d, a.na.wrap_d, a.na.dil_d);
    ay = na_dil_anchor(yq, a.na.grid_h, a.na.kernel_h, a.na.rad_h, a.na.wrap_h, a.na.dil_h);
    ax = na_dil_anchor(xq, a.na.grid_w, a.na.kernel_w, a.na.rad_w, a.na.wrap_w, a.na.dil_w);
  }
  // Neighbourhood grids whose width is a multiple of 32 (up to 128): every
  // 32-key MFMA block lies in one grid row, and the columns a lane's 16 keys of
  // a block fall on depend only on the block's phase (its start column / 32).
  // The column test is therefore done once per lane: bit 16*phase + r of col_bits
  // says whether accumulator element r of a block with that phase is in the
  // query's column window.
  constexpr bool NA_BLOCKS = MASK == MASK_NA_BLOCKS;
  uint32_t col_bits[2] = {0u, 0u};
  if (NA_BLOCKS) na_col_bits(xq, half, a.na.grid_w, a.na.kernel_w, a.na.rad_w, a.na.wrap_w, a.na_phases, col_bits);
  // Other grids of width 4..124 (3D, dilated): one window mask per axis and lane (GridMasks).
  constexpr bool NA_GRID = MASK == MASK_NA_GRID;
  constexpr bool NA_BITS = NA_BLOCKS || NA_GRID;
  GridMasks gm{};
  if constexpr (NA_GRID) gm = na_grid_masks(zq, yq, xq, a.na);


  const int32_t n = run.count;
  const i32x4_t k_rsrc = head_rsrc(kh, head_bytes);
  const i32x4_t v_rsrc = head_rsrc(vh, head_bytes);


  // S^T = K Q^T for the key tile in `ks`: lane holds keys 32sb + 8(r/4) + 4*half + r%4 of its query
  auto qk_tile = [&](const uint16_t* ks, f32x16_t (&s)[SB]) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) s[sb] = f32x16_t{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int row = sb * 32 + col;
        const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(ks + row * D + (((2 * kb + half) ^ k_swz) << 3));
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qf[kb], s[sb], 0, 0, 0);
      }
    }
  };

  // O^T += V^T P^T for the value tile in `vs`. Slot 8*half + e of 16-key block (sb, kb2)
  // holds key 32sb + 16kb2 + 8(e/4) + 4*half + e%4, matching the S^T accumulator layout.
  auto pv_tile = [&](const uint16_t* vs, const bf16x8_t (&p)[SB][2], f32x16_t (&o)[DT]) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int row0 = sb * 32 + kb2 * 16;  // multiple of 16: leaves the row swizzle unchanged
          u32x2_t x[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            x[h] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4*)((lds_u16*)vs + (row0 + v_row[h]) * D + v_off[h][dt])));
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{x[0][0], x[0][1], x[1][0], x[1][1]});
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[sb][kb2], o[dt], 0, 0, 0);
        }
      }
    }
  };

  // Element mask of key tile t (uniform decision whether to apply it at all). The
  // conditions are combined with bitwise & and applied with a select: no
  // per-lane control flow. (A short-circuit && followed by a conditional store
  // into the accumulator vector compiled, for the neighbourhood mask, into code
  // that dropped the second axis' condition.)
  auto apply_mask = [&](f32x16_t (&s)[SB], int32_t t) {
    // key = (row0, x0) + off in row-major order over all grid rows of all planes
    int32_t row0 = 0, x0 = 0, z0 = 0, y0 = 0;
    bool dilated = false;
    if (is_na(MASK)) {
      row0 = (t * C::BN) / a.na.grid_w;
      x0 = t * C::BN - row0 * a.na.grid_w;
      z0 = row0 / a.na.grid_h;
      y0 = row0 - z0 * a.na.grid_h;
      dilated = (a.na.dil_d | a.na.dil_h | a.na.dil_w) != 1;  // uniform
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t off = sb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const int32_t key = t * C::BN + off;
        bool ok = key < Nkv;
        if (MASK == MASK_CAUSAL) ok = ok & (key <= my_q);
        if (is_na(MASK)) {
          // For n < 2^21 the quotient (n + 0.5) / L stays at least 0.5 / L away
          // from an integer, far more than the float error, so truncation is
          // exact; here n = x0 + off < grid_w + BN and y0 + dy < grid_h + BN.
          const int32_t dy = (int32_t)(((float)(x0 + off) + 0.5f) * a.na_inv_w);
          const int32_t xk = x0 + off - dy * a.na.grid_w;
          const int32_t yy = y0 + dy;
          const int32_t dz = (int32_t)(((float)yy + 0.5f) * a.na_inv_h);
          const int32_t yk = yy - dz * a.na.grid_h, zk = z0 + dz;
          if (!dilated) {
            ok = ok & na_axis_ok(zq, zk, a.na.grid_d, a.na.kernel_d, a.na.rad_d, a.na.wrap_d) &
                 na_axis_ok(yq, yk, a.na.grid_h, a.na.kernel_h, a.na.rad_h, a.na.wrap_h) &
                 na_axis_ok(xq, xk, a.na.grid_w, a.na.kernel_w, a.na.rad_w, a.na.wrap_w);
          } else {
            ok = ok & na_dil_ok(az, zk, a.na.grid_d, a.na.kernel_d, a.na.rad_d, a.na.wrap_d, a.na.dil_d) &
                 na_dil_ok(ay, yk, a.na.grid_h, a.na.kernel_h, a.na.rad_h, a.na.wrap_h, a.na.dil_h) &
                 na_dil_ok(ax, xk, a.na.grid_w, a.na.kernel_w, a.na.rad_w, a.na.wrap_w, a.na.dil_w);
          }
        }
        s[sb][r] = ok ? s[sb][r] : -INFINITY;
      }
    }
  };

  // In-lane maximum of the tile; the lane pair (l, l + 32) is combined separately
  // (swap_halves_max), after the scheduling region of a step.
  auto lane_max = [&](const f32x16_t (&s)[SB]) {
    float mx = s[0][0];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
    return mx;
  };

  // P = 2^(c s - m) rounded to bfloat16; returns this lane's sum of the rounded values.
  auto exp_tile = [&](const f32x16_t (&s)[SB], float m, bool masked, bf16x8_t (&p)[SB][2]) {
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float s0 = s[sb][kb2 * 8 + e], s1 = s[sb][kb2 * 8 + e + 1];
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, -m));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, -m));
          if (masked) {
            p0 = s0 == -INFINITY ? 0.f : p0;
            p1 = s1 == -INFINITY ? 0.f : p1;
          }
          const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
          p[sb][kb2][e] = pp[0];
          p[sb][kb2][e + 1] = pp[1];
          psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
        }
      }
    }
    return psum;
  };

  // Per 32-key block of key tile t, the lane's 16-bit window mask (structured
  // neighbourhood grids): the block's grid row passes the row test and its
  // phase selects the column bits.
  auto block_masks = [&](int32_t t, uint32_t (&bm)[SB]) {
    const int32_t k0 = t * C::BN;                 // multiple of 32
    const int32_t row0 = k0 / a.na.grid_w;        // uniform: one division per tile
    int32_t row = row0, phase = (k0 - row0 * a.na.grid_w) >> 5;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      if (sb > 0 && ++phase == a.na_phases) {  // next 32-key block: next phase, or the next grid row
        phase = 0;
        ++row;
      }
      const bool rok = row < a.na.grid_h && na_axis_ok(yq, row, a.na.grid_h, a.na.kernel_h, a.na.rad_h, a.na.wrap_h);
      const uint32_t cb = (col_bits[phase >> 1] >> ((phase & 1) * 16)) & 0xffffu;
      bm[sb] = rok ? cb : 0u;
    }
  };
  // Per 32-key block of key tile t, the lane's 16-bit window mask on a grid of
  // width 4..124: the tile's window (na_tile_window), then the lane's own keys.
  auto grid_bits = [&](int32_t t, uint32_t (&bm)[SB]) {
    const int32_t k0 = t * C::BN;
    const int32_t row0 = k0 / a.na.grid_w;  // uniform: one division per tile
    uint32_t w[SB];
    na_tile_window(gm, row0, k0 - row0 * a.na.grid_w, a.na, w);
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) bm[sb] = lane_block_bits(w[sb], half);
  };
  // The 16-bit element masks of key tile t for a bit-masked step: the window bits
  // for the neighbourhood grids, else the keys up to the lane's last visible one
  // (its query for the causal mask, Nkv - 1 for a ragged last tile).
  auto tile_bits = [&](int32_t t, uint32_t (&bm)[SB]) {
    if constexpr (NA_BLOCKS) {
      block_masks(t, bm);
    } else if constexpr (NA_GRID) {
      grid_bits(t, bm);
    } else {
      int32_t last = Nkv - 1;
      if constexpr (MASK == MASK_CAUSAL) last = last < my_q ? last : my_q;
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) bm[sb] = limit_bits(last - (t * C::BN + sb * 32 + 4 * half));
    }
  };
  // Masked scores become -inf (rare slow path of a bitmask-masked step).
  auto apply_bits = [&](f32x16_t (&s)[SB], const uint32_t (&bm)[SB]) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sb][r] = ((bm[sb] >> r) & 1u) ? s[sb][r] : -INFINITY;
  };

#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  bf16x8_t p[SB][2];

  // Tile i of the run, clamped to the last one: loads past the end refill a
  // buffer nobody reads again, and keep the number of loads per step fixed.
  auto run_tile = [&](int32_t i) { return kv_tile_at(run, i < n ? i : n - 1, n_kv); };

  // ---- prologue: K of tile 0, then (K of tile i, V of tile i - 1) for i = 1 .. S - 1,
  // in the order the steps issue them; scores and probabilities of tile 0
  {
    const int32_t t0 = kv_tile_at(run, 0, n_kv);
    ld.load(k_rsrc, t0, k_lds[0]);
#pragma unroll
    for (int i = 1; i < S; ++i) {
      ld.load(k_rsrc, run_tile(i), k_lds[i]);
      ld.load(v_rsrc, run_tile(i - 1), v_lds[i - 1]);
    }
    wait_tile_loads<kSerialTiles ? 0 : C::LOADS_AHEAD + 2 * C::LOADS>();  // K of tile 0
    __syncthreads();
    f32x16_t s[SB];
    qk_tile(k_lds[0], s);
    const bool masked = tile_needs_mask(MASK, Nkv, C::BN, q0, t0);
    if constexpr (NA_BITS) {
      uint32_t bm0[SB];
      tile_bits(t0, bm0);
      apply_bits(s, bm0);
    } else {
      if (masked) apply_mask(s, t0);
    }
    const float mx = swap_halves_max(lane_max(s));
    m_run = mx == -INFINITY ? -FLT_MAX : mx * c;  // finite sentinel: never inf - inf
    l_run = exp_tile(s, m_run, masked, p);
    wait_tile_loads<kSerialTiles ? 0 : C::LOADS_AHEAD>();  // K of tile 1 and V of tile 0
    __syncthreads();  // ... published, and every wavefront has read K of tile 0 before its buffer is refilled
  }

  // Common tail of a step (the new probabilities are in pn). They were computed
  // against the reference maximum m_run of earlier tiles. Every probability is at most the
  // lane's row sum, so psum <= 2^kSafeLog2 proves that none exceeds 2^kSafeLog2
  // (far inside fp32/bf16 range: O and l stay finite for any Nkv). Otherwise (some
  // row's maximum moved up, rare after the first tile) the exact tile maximum
  // becomes the new reference, O and l are rescaled and the tile is redone.
  // Then the next tiles are awaited.
  auto finish_step = [&](float psum, f32x16_t (&s)[SB], bool masked, bf16x8_t (&pn)[SB][2],
                         const uint32_t (&bm)[SB], auto bits_tag) {
    if (__builtin_amdgcn_ballot_w64(!(psum <= kSafeSum))) {
      if constexpr (decltype(bits_tag)::value) {
        apply_bits(s, bm);
        masked = true;
      }
      const float mx = swap_halves_max(lane_max(s));
      const float cand = mx == -INFINITY ? -FLT_MAX : mx * c;
      const float m_new = fmaxf(m_run, cand);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      l_run *= alpha;
      psum = exp_tile(s, m_run, masked, pn);
    }
    l_run += psum;
    wait_tile_loads<kSerialTiles ? 0 : C::LOADS_AHEAD>();  // K of tile j + 2 and V of tile j + 1
    __syncthreads();
  };

  // Steady-state step for a key tile that needs no element mask. LDS holds K of
  // tile j+1 and V of tile j. A wavefront issues in order, so the matrix core and
  // the VALU only overlap if their instructions alternate; the order is fixed
  // slot by slot (sched_barrier fences):
  //   MFMA groups  S^T b0 | S^T b1 | PV b0 | S^T b2 | PV b1 | S^T b3 | PV b2 | PV b3
  //   (KB MFMAs per group), LDS reads two slots ahead of their MFMA, and the 32
  //   two-score pieces of softmax work (exp2, bf16 pack, row sum) spread over
  //   the slots after S^T b0, each after its own block's group.
  // Probabilities use the previous reference maximum, so no piece waits for the
  // whole tile's maximum.
  auto step_fast = [&](int32_t j, const bf16x8_t (&pc)[SB][2], bf16x8_t (&pn)[SB][2], auto bits_tag) {
    constexpr bool BITS = decltype(bits_tag)::value;  // structured neighbourhood mask
    const int32_t t1 = kv_tile_at(run, j + 1, n_kv);
    uint32_t bm[SB];
    if constexpr (BITS) tile_bits(t1, bm);
    // this step loads K of tile j + S into the buffer of K(j) and V of tile j + S - 1
    // into the buffer of V(j - 1): both were last read in step j - 1
    const int32_t tk = run_tile(j + S), tv = run_tile(j + S - 1);
    const uint16_t* ks = k_lds[(j + 1) & (S - 1)];
    const uint16_t* vs = v_lds[j & (S - 1)];
    const uint16_t* k_dst = k_lds[j & (S - 1)];
    const uint16_t* v_dst = v_lds[(j + S - 1) & (S - 1)];

    constexpr int GS = KB;                 // MFMAs per group (= 2 * DT)
    constexpr int TOT = 2 * SB * GS;       // MFMAs per step
    constexpr int NPAIR = SB * 8;          // two-score pieces per lane
    constexpr int VSLOTS = TOT - GS;       // slots after the first group
    constexpr int PF = 2;                  // read-ahead distance in slots
    // group g: kind 0 = S^T, 1 = PV; block of the group. Four blocks (128-key tiles):
    // S^T b0 | S^T b1 | PV b0 | S^T b2 | PV b1 | S^T b3 | PV b2 | PV b3; two blocks
    // (64-key tiles): S^T b0 | S^T b1 | PV b0 | PV b1.
    static_assert(SB == 4 || SB == 2, "group order for 2 or 4 blocks per tile");
    constexpr auto kind = [](int g) {
      if constexpr (SB == 2) return g >= 2 ? 1 : 0;
      return (g == 2 || g == 4 || g >= 6) ? 1 : 0;
    };
    constexpr auto blk = [](int g) {
      if constexpr (SB == 2) return g & 1;
      return g < 2 ? g : (g == 2 ? 0 : (g == 3 ? 2 : (g == 4 ? 1 : (g == 5 ? 3 : g - 4))));
    };

    f32x16_t s[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) s[sb] = f32x16_t{};
    u32x4_t kf[TOT];
    bf16x8_t vf[TOT];
    uint32_t pw[SB][2][4];  // new probabilities, two bf16 per word
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

    auto issue_read = [&](auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      constexpr int g = slot / GS, i = slot % GS, b = blk(g);
      if constexpr (kind(g) == 0) {
        const int row = b * 32 + col;
        kf[slot] = *reinterpret_cast<const u32x4_t*>(ks + row * D + (((2 * i + half) ^ k_swz) << 3));
      } else {
        constexpr int kb2 = i / DT, dt = i % DT;
        u32x2_t x[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          x[h] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (lds_s16x4*)((lds_u16*)vs + (b * 32 + kb2 * 16 + v_row[h]) * D +
                                                              v_off[h][dt])));
        // whole 32-bit words: element-wise 16-bit copies cost a v_perm per word
        vf[slot] = __builtin_bit_cast(bf16x8_t, u32x4_t{x[0][0], x[0][1], x[1][0], x[1][1]});
      }
    };

    // Softmax pieces (two scores each) run as three stages in consecutive slots,
    // so that no slot holds a chain of dependent VALU operations (each would wait
    // for the previous one's result): A = the exponents' arguments (fma), B = the
    // exponentials (and the window mask), C = the bf16 pack. Piece q starts
    // in slot GS + q * VSLOTS / NPAIR, after its block's S^T group; stages falling
    // past the last slot run after it. An empty asm pins each stage to its slot:
    // without a use there, IR passes sink the arithmetic below every MFMA.
    float xa[NPAIR][2];  // stage A results
    float pb[NPAIR][2];  // stage B results
    auto pieces_at = [&](auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      static_for<NPAIR>([&](auto q_c) {
        constexpr int q = decltype(q_c)::value;
        constexpr int a = GS + (q * VSLOTS) / NPAIR;
        constexpr int b2 = q / 8, pp = q % 8;
        if constexpr (a == slot) {
          float x0 = __builtin_fmaf(s[b2][2 * pp], c, -m_run);
          float x1 = __builtin_fmaf(s[b2][2 * pp + 1], c, -m_run);
          asm volatile("" : "+v"(x0), "+v"(x1));
          xa[q][0] = x0;
          xa[q][1] = x1;
        }
        if constexpr (a + 1 == slot) {
          float p0 = __builtin_amdgcn_exp2f(xa[q][0]);
          float p1 = __builtin_amdgcn_exp2f(xa[q][1]);
          if constexpr (BITS) {
            // signed one-bit extract: all ones where the key is in the window, else 0
            p0 = __uint_as_float(__float_as_uint(p0) & (uint32_t)__builtin_amdgcn_sbfe((int)bm[b2], 2 * pp, 1));
            p1 = __uint_as_float(__float_as_uint(p1) & (uint32_t)__builtin_amdgcn_sbfe((int)bm[b2], 2 * pp + 1, 1));
          }
          asm volatile("" : "+v"(p0), "+v"(p1));
          pb[q][0] = p0;
          pb[q][1] = p1;
        }
        if constexpr (a + 2 == slot) {
          const bf16x2_t pp2 = {(__bf16)pb[q][0], (__bf16)pb[q][1]};
          uint32_t pk = __builtin_bit_cast(uint32_t, pp2);
          asm volatile("" : "+v"(pk));
          pw[b2][pp / 4][pp % 4] = pk;
        }
      });
    };

    static_for<PF>([&](auto slot_c) { issue_read(slot_c); });
    static_for<TOT>([&](auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      if constexpr (slot + PF < TOT) issue_read(std::integral_constant<int, slot + PF>{});
      constexpr int g = slot / GS, i = slot % GS, b = blk(g);
      if constexpr (kind(g) == 0) {
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[slot]), qf[i], s[b], 0, 0, 0);
      } else {
        constexpr int kb2 = i / DT, dt = i % DT;
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[slot], pc[b][kb2], oacc[dt], 0, 0, 0);
      }
      // next tiles' loads, one every other slot in the first half of the step: issued
      // in one burst they back up the CU's path to LDS and stall the issuing wave
      if constexpr (!kSerialTiles && slot % 2 == 0 && slot / 2 < 2 * C::LOADS) {
        constexpr int li = slot / 2;
        if constexpr (li < C::LOADS) ld.load_part(k_rsrc, tk, k_dst, li);
        else ld.load_part(v_rsrc, tv, v_dst, li - C::LOADS);
      }
      pieces_at(slot_c);  // softmax stages assigned to this slot
      __builtin_amdgcn_sched_barrier(0);
    });
    pieces_at(std::integral_constant<int, TOT>{});
    __builtin_amdgcn_sched_barrier(0);
    pieces_at(std::integral_constant<int, TOT + 1>{});
    // Row sum of the rounded probabilities. v_dot2c_f32_bf16 does not run beside a
    // matrix instruction: the first one after an MFMA waits for the matrix core to
    // drain (about half an MFMA), later ones issue at the normal rate. One batch per
    // step, after the last MFMA, pays that wait once instead of once per slot.
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
    static_for<NPAIR>([&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      constexpr int b2 = q / 8, pp = q % 8;
      ps[q & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[b2][pp / 4][pp % 4]), ones,
                                                 ps[q & 3], false);
    });
    const float psum = (ps[0] + ps[2]) + (ps[1] + ps[3]);
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
        pn[sb][kb2] = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[sb][kb2][0], pw[sb][kb2][1], pw[sb][kb2][2], pw[sb][kb2][3]});
    if constexpr (kSerialTiles) {  // race check: this step's loads only after its compute
      ld.load(k_rsrc, tk, k_dst);
      ld.load(v_rsrc, tv, v_dst);
    }
    finish_step(psum, s, false, pn, bm, bits_tag);
  };

  // Step for a key tile of a neighbourhood grid that has no bit-mask form
  // (every tile needs the element predicate): plain order.
  auto step_masked = [&](int32_t j) {
    const int32_t t1 = kv_tile_at(run, j + 1, n_kv);
    auto loads = [&]() {
      ld.load(k_rsrc, run_tile(j + S), k_lds[j & (S - 1)]);
      ld.load(v_rsrc, run_tile(j + S - 1), v_lds[(j + S - 1) & (S - 1)]);
    };
    if constexpr (!kSerialTiles) loads();
    f32x16_t s[SB];
    qk_tile(k_lds[(j + 1) & (S - 1)], s);
    pv_tile(v_lds[j & (S - 1)], p, oacc);
    apply_mask(s, t1);
    bf16x8_t pn[SB][2];
    const float psum = exp_tile(s, m_run, true, pn);
    const uint32_t no_bits[SB] = {};
    if constexpr (kSerialTiles) loads();  // race check: loads only after the step's compute
    finish_step(psum, s, true, pn, no_bits, std::false_type{});
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      p[sb][0] = pn[sb][0];
      p[sb][1] = pn[sb][1];
    }
  };

  // Tiles that need no element mask come first for the none and causal masks (only
  // a ragged last tile or the diagonal tiles need one), so the loop splits once.
  // The fast loop is unrolled by two so the probabilities alternate between two
  // register sets instead of being copied every step.
  int32_t j = 0;
  auto fast_loop = [&](int32_t n_fast, auto bits_tag) {
    bf16x8_t p_alt[SB][2];
    for (; j + 1 < n_fast; j += 2) {
      step_fast(j, p, p_alt, bits_tag);
      step_fast(j + 1, p_alt, p, bits_tag);
    }
    if (j < n_fast) {
      step_fast(j, p, p_alt, bits_tag);
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        p[sb][0] = p_alt[sb][0];
        p[sb][1] = p_alt[sb][1];
      }
      ++j;
    }
  };
  if constexpr (NA_BITS) {
    fast_loop(n - 1, std::true_type{});
  } else if constexpr (MASK != MASK_NA) {
    int32_t n_fast = 0;  // steps whose next tile needs no element mask
    while (n_fast + 1 < n && !tile_needs_mask(MASK, Nkv, C::BN, q0, kv_tile_at(run, n_fast + 1, n_kv))) ++n_fast;
    fast_loop(n_fast, std::false_type{});
    fast_loop(n - 1, std::true_type{});  // the causal diagonal and a ragged last tile, on bit masks
  } else {
    for (; j + 1 < n; ++j) step_masked(j);
  }

  // ---- last tile's product with V
  pv_tile(v_lds[(n - 1) & (S - 1)], p, oacc);
  // refills issued past the end of the run (up to STAGES - 2 steps' worth at d = 32)
  // must land before the work-group's LDS is released
  wait_tile_loads<0>();
  };

  // Delayed division and store of query tile qtile of head bh: lane holds d = 32dt + 8(r/4) + 4*half + r%4.
  // With an lse output, lane `col` of the first half-wave also writes its row's
  // logsumexp: P = 2^(c s - m), so log(sum exp(scale s)) = ln 2 * (m + log2 l).
  auto store_rows = [&](const int32_t bh, const int32_t qtile, const f32x16_t (&oacc)[DT], const float m_run,
                        const float l_run) {
    const int32_t my_q = qtile * C::BM + wave * 32 + col;
    uint16_t* __restrict__ oh = a.o + (size_t)bh * (size_t)Nq * D;
    const float l_tot = swap_halves_sum(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (my_q < Nq) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4_t ob;
#pragma unroll
          for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(oacc[dt][g * 4 + e] * inv);
          *reinterpret_cast<u32x2_t*>(oh + (size_t)my_q * D + dt * 32 + g * 8 + half * 4) =
              __builtin_bit_cast(u32x2_t, ob);
        }
      }
      if (a.lse != nullptr && half == 0) a.lse[(size_t)bh * Nq + my_q] = row_lse(m_run, l_tot);
    }
  };

  f32x16_t oacc[DT];
  float m_run, l_run;
  if constexpr (!SPLIT) {
    const WorkItem w = work_item(MASK, blockIdx.x, gridDim.x, a.n_qtiles, a.BH, a.causal_group);
    segment(w.bh, w.qtile, kv_run(MASK, Nq, Nkv, C::BM, C::BN, w.qtile * C::BM, a.na), oacc, m_run, l_run);
    store_rows(w.bh, w.qtile, oacc, m_run, l_run);
  } else {
    // Remainder split (unmasked problems): whole tiles first, XCD-contiguous so
    // the tiles of one head share an L2; then the parts of the split tiles,
    // each of which leaves its partial result in its own workspace slot.
    // The parts are numbered part-major (all tiles' part 0, then part 1, ...) and
    // taken XCD-contiguously, so an XCD holds one key range of consecutive tiles,
    // mostly of one head: each key range of a head is fetched into one L2, not
    // into every L2 that holds some part of its tiles.
    const int32_t full = a.split_full, parts = a.split_parts;
    const bool whole = (int32_t)blockIdx.x < full;
    const int32_t rem = (gridDim.x - full) / parts;
    const int32_t j = whole ? 0 : xcd_contiguous(blockIdx.x - full, gridDim.x - full);  // parts only
    const int32_t r = whole ? 0 : j % rem;                // split tile
    const int32_t slot = whole ? 0 : r * parts + j / rem;  // its slot: part j / rem of tile r
    const int32_t tile = whole ? xcd_contiguous(blockIdx.x, full) : full + r;
    const int32_t bh = tile / a.n_qtiles, qtile = tile - bh * a.n_qtiles;
    segment(bh, qtile, whole ? KvRun{0, n_kv} : part_run(n_kv, parts, slot % parts), oacc, m_run, l_run);
    if (whole) {
      store_rows(bh, qtile, oacc, m_run, l_run);
      return;
    }
    write_part<D>(a.ws_parts + (size_t)slot * PartSlot<D>::FLOATS, wave, lane, oacc, m_run, l_run);
    // The tile's last part to finish merges it. Every wavefront waits until
    // its write-through slot stores have completed; then the work-group counts
    // one arrival on the tile's counter (an agent-scope atomic; the counters
    // are zeroed by the clear kernel queued before this one). The work-group
    // that brings the count to `parts` comes after every part's completed
    // stores, and reads the slots past its L2 (merge_parts).
    __shared__ uint32_t last_part;
    wait_tile_loads<0>();  // vmcnt(0): this wavefront's slot stores are done
    __syncthreads();
    if (tid == 0)
      last_part = __hip_atomic_fetch_add(a.split_count + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)parts - 1;
    __syncthreads();
    if (last_part) merge_parts<D>(a, r, wave, lane);
  }
}

// ---------------------------------------------------------------------------
// Neighbourhood windows by query patches (MASK_NA_PATCH, na_patch_eligible).
//
// One work-group per patch of 8 x 16 queries of one head. It copies the patch's
// key rectangle (a band of key rows times a band of at most 32 columns, see
// na_patch_bands) into LDS once, one 32-key block per key row, and waits for it
// once; query wavefront w then holds the 32 queries of patch rows 2w and 2w + 1
// (lane column col: row col / 16, column col % 16) and runs over the key rows of
// its own two rows' band, four blocks per step. The arithmetic per step is that of
// the tile kernel (scores on the matrix core, window bits, P = 2^(c s - m) against
// a reference maximum set by the part's first step and moved only past the 2^20
// row-sum guard, O += P V, delayed division). At d = 32 every query wavefront has
// a second wavefront on its SIMD that takes the odd steps of the same queries
// (two parts); the parts meet once at the end, where the second leaves its
// output, maximum and row sums in LDS and the first combines them exactly (the
// rescaling by 2^(m_i - m) of the running-softmax paragraph of PhotoRoom's
// xformers post) and stores.
// One step of a neighbourhood walk over key rows held in LDS (the patch kernel):
// the first nblk (1..4, uniform) of four 32-key blocks, block b at kb[b]
// and vb[b] (32 rows of D elements, swizzled as the tile rings). Element e of a
// block is key 8 (e / 4) + 4 half + e % 4. The window: a block whose key row is in
// the lane's window (live[b]) takes the lane's per-element bias over the row's
// columns (0 for a visible key, -inf for a hidden one); every key of another block
// is hidden. The window enters as the addend of the exponent's fma, so a hidden key
// gives 2^-inf = 0 with no test (also at scale 0: the addend is -inf, not the
// product). On the walk's first step (first)
// the reference maximum m_run is c times the largest visible score; P = 2^(c s -
// m_run) is rounded to bfloat16 and the lane's sum of the rounded values kept,
// redone against a new maximum past the 2^20 row-sum guard (the tile kernel's
// rule); O^T += V^T P^T. Blocks past nblk cost nothing.
template <int D>
__device__ __forceinline__ void window_step(const uint16_t* const (&kb)[4], const uint16_t* const (&vb)[4],
                                            const bool (&live)[4], const float (&bias)[16], int nblk, bool first,
                                            const bf16x8_t (&qf)[D / 16], float c, int col, int half, int k_swz,
                                            const int (&v_row)[2], const int (&v_off)[2][D / 32],
                                            f32x16_t (&oacc)[D / 32], float& m_run, float& l_run) {
  constexpr int KB = D / 16, DT = D / 32, SB = 4;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  // S^T = K Q^T: lane holds keys 8 (e / 4) + 4 half + e % 4 of each block, for its query
  f32x16_t s[SB];
#pragma unroll
  for (int sb = 0; sb < SB; ++sb) s[sb] = f32x16_t{};
#pragma unroll
  for (int kb_ = 0; kb_ < KB; ++kb_)
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      if (sb >= nblk) continue;
      const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(kb[sb] + col * D + (((2 * kb_ + half) ^ k_swz) << 3));
      s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qf[kb_], s[sb], 0, 0, 0);
    }
  // c * (largest visible score), -FLT_MAX when there is none (a finite sentinel)
  auto row_max = [&]() {
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (sb >= nblk) continue;
        mx = fmaxf(mx, live[sb] ? __builtin_fmaf(s[sb][e], c, bias[e]) : -INFINITY);
      }
    mx = swap_halves_max(mx);
    return mx == -INFINITY ? -FLT_MAX : mx;
  };
  if (first) m_run = row_max();
  bf16x8_t p[SB][2];
  auto probs = [&]() {
    float nb[16];  // the exponent's addend per element of a live block
#pragma unroll
    for (int e = 0; e < 16; ++e) nb[e] = bias[e] - m_run;
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          if (sb >= nblk) continue;
          const int e0 = kb2 * 8 + e, e1 = e0 + 1;
          const float a0 = live[sb] ? nb[e0] : -INFINITY;
          const float a1 = live[sb] ? nb[e1] : -INFINITY;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][e0], c, a0));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][e1], c, a1));
          const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
          p[sb][kb2][e] = pp[0];
          p[sb][kb2][e + 1] = pp[1];
          psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
        }
    return psum;
  };
  float psum = probs();
  if (__builtin_amdgcn_ballot_w64(!(psum <= kSafeSum))) {  // rare: a row's maximum moved far up
    const float m_new = fmaxf(m_run, row_max());
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    l_run *= alpha;
    psum = probs();
  }
  l_run += psum;
  // O^T += V^T P^T
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if (sb >= nblk) continue;
        u32x2_t x[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          x[h] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (lds_s16x4*)((lds_u16*)vb[sb] + (kb2 * 16 + v_row[h]) * D + v_off[h][dt])));
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{x[0][0], x[0][1], x[1][0], x[1][1]});
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[sb][kb2], oacc[dt], 0, 0, 0);
      }
}

// The same walk one key row (32-key block) at a time, for the row and patch
// kernels: the scores of the next visible row are issued on the matrix core
// before the current row's exponentials (row_scores), and row_update takes one
// row's softmax and P V. The row is in the lane's window (live) or hidden for
// it; inside it the lane's column bias decides. A lane's reference maximum is
// set by the first row that holds a visible key for it (m_run starts at the
// sentinel -FLT_MAX; a lane outside the grid starts at 0 and never sees one) and
// moved only past the 2^20 row-sum guard, per row.
template <int D>
__device__ __forceinline__ f32x16_t row_scores(const uint16_t* krow, const bf16x8_t (&qf)[D / 16], int col, int half,
                                               int k_swz) {
  f32x16_t s = f32x16_t{};
#pragma unroll
  for (int kb_ = 0; kb_ < D / 16; ++kb_) {
    const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(krow + col * D + (((2 * kb_ + half) ^ k_swz) << 3));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qf[kb_], s, 0, 0, 0);
  }
  return s;
}

template <int D>
__device__ __forceinline__ void row_update(const f32x16_t& s, const uint16_t* vrow, const float (&bias)[16],
                                           bool live, float c, const int (&v_row)[2], const int (&v_off)[2][D / 32],
                                           f32x16_t (&oacc)[D / 32], float& m_run, float& l_run) {
  constexpr int DT = D / 32;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  auto row_max = [&]() {  // c * (largest visible score of the row), -FLT_MAX when there is none
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, live ? __builtin_fmaf(s[e], c, bias[e]) : -INFINITY);
    mx = swap_halves_max(mx);
    return mx == -INFINITY ? -FLT_MAX : mx;
  };
  if (__builtin_amdgcn_ballot_w64(m_run == -FLT_MAX)) {  // some lane has seen no visible key yet
    const float mx = row_max();
    m_run = m_run == -FLT_MAX ? mx : m_run;
  }
  bf16x8_t p[2];
  auto probs = [&]() {
    float nb[16];  // the exponent's addend: bias - m for a row in the window, -inf otherwise
#pragma unroll
    for (int e = 0; e < 16; ++e) nb[e] = live ? bias[e] - m_run : -INFINITY;
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int e0 = kb2 * 8 + e, e1 = e0 + 1;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e0], c, nb[e0]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e1], c, nb[e1]));
        const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
        p[kb2][e] = pp[0];
        p[kb2][e + 1] = pp[1];
        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
      }
    return psum;
  };
  float psum = probs();
  if (__builtin_amdgcn_ballot_w64(!(psum <= kSafeSum))) {  // rare: a row's maximum moved far up
    const float m_new = fmaxf(m_run, row_max());
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    l_run *= alpha;
    psum = probs();
  }
  l_run += psum;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x2_t x[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        x[h] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                               (lds_s16x4*)((lds_u16*)vrow + (kb2 * 16 + v_row[h]) * D + v_off[h][dt])));
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{x[0][0], x[0][1], x[1][0], x[1][1]});
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[kb2], oacc[dt], 0, 0, 0);
    }
}

template <int D>
struct PatchCfg {
  // key rows (32 keys each) of the K and of the V rectangle in LDS: 96 KB in all at
  // d = 32 (114 KB with the two parts' merge area), 136 KB at d = 64
  static constexpr int ROWS = D == 32 ? 24 : 17;
  static constexpr int PARTS = D == 32 ? 2 : 1;  // wavefronts per query wavefront (step parity)
  static constexpr int THREADS = 256 * PARTS;
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int CHUNKS = ROWS * kPatchKeyCols * ROW_CHUNKS;  // 16-byte chunks per rectangle
  static_assert(CHUNKS % THREADS == 0, "the copy runs in whole rounds of the work-group's lanes");
  static constexpr int ELEMS = CHUNKS * 8;
  static constexpr int MERGE = PARTS > 1 ? 4 * (D / 32 * 16 + 2) * 64 : 1;  // floats: second part's O, m, l
};
static_assert(PatchCfg<32>::ROWS == patch_lds_rows(32) && PatchCfg<64>::ROWS == patch_lds_rows(64),
              "host eligibility and kernel LDS must agree");

template <int D>
__global__ __launch_bounds__(PatchCfg<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_na_patch_kernel(KernelArgs a) {
  using P = PatchCfg<D>;
  constexpr int KB = D / 16, DT = D / 32, SB = 4, RC = D / 8;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[P::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[P::ELEMS];
  __shared__ float merge_lds[P::MERGE];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wave8 & 3, part = wave8 >> 2;  // query wavefront, step parity
  const float c = a.c;

  // patches row-major within a head, heads kept on one XCD (xcd_contiguous)
  const int32_t per_head = a.patch_ny * a.patch_nx;
  const int32_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int32_t bh = item / per_head, pidx = item - bh * per_head;
  const int32_t py = pidx / a.patch_nx;
  // rows and columns in the coordinates of the patch's sub-grids (na_patch_group): H x W
  // cells, token patch_token(pr, row, column)
  const PatchGroup pr = na_patch_group(a.na, py, pidx - py * a.patch_nx, a.patch_cols_strided != 0);
  const NaGeom& g = pr.geom;
  const int32_t H = g.grid_h, W = g.grid_w, N = a.Nq;
  const int32_t y0 = pr.u0, x0 = pr.v0;
  const PatchBands pb = na_patch_bands(y0, x0, g);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * (uint32_t)(D * 2);

  // ---- the lane's query (loaded first, used after the rectangle has landed)
  const int32_t qy = y0 + 2 * wave + (col >> 4), qx = x0 + (col & 15);
  const bool q_ok = qy < H && qx < W;
  const int32_t my_q = patch_token(pr, qy, qx);
  // every lane loads (a query outside the grid reads query 0 and zeroes it after the wait)
  const int32_t q_row = q_ok ? my_q : 0;
  u32x4_t qraw[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qraw[kb] = *reinterpret_cast<const u32x4_t*>(a.q + head + (size_t)q_row * D + kb * 16 + half * 8);

  // ---- the key rectangle: LDS chunk p holds chunk (p % RC) ^ swizzle of key p / RC,
  // key = 32 r + x: row band cell r, column band cell x. Rows past the band (up to 3
  // are read by a wavefront's last step) and columns past the column band read as
  // zero (an offset past the head) and are masked.
  {
    const i32x4_t k_rsrc = head_rsrc(a.k + head, head_bytes);
    const i32x4_t v_rsrc = head_rsrc(a.v + head, head_bytes);
    const uint32_t k_base = __builtin_amdgcn_readfirstlane(lds_addr(k_lds) + wave8 * 1024);
    const uint32_t v_base = __builtin_amdgcn_readfirstlane(lds_addr(v_lds) + wave8 * 1024);
    const int32_t n_loads = (int32_t)cdiv((int64_t)(pb.rows.count + 3) * kPatchKeyCols * RC, P::THREADS);
    for (int32_t j = 0; j < n_loads; ++j) {
      const int32_t p = j * P::THREADS + tid;
      const int32_t key = p / RC, r = key / kPatchKeyCols, x = key % kPatchKeyCols;
      const int32_t chunk = (p % RC) ^ chunk_swizzle<D>(key);
      uint32_t voff = head_bytes;
      if (r < pb.rows.count && x < pb.cols.count) {
        int32_t ky = pb.rows.start + r, kx = pb.cols.start + x;
        ky -= ky >= H ? H : 0;  // both start inside the axis and span at most its length
        kx -= kx >= W ? W : 0;
        voff = (uint32_t)patch_token(pr, ky, kx) * (uint32_t)(D * 2) + (uint32_t)chunk * 16u;
      }
      dma_lds16(k_rsrc, k_base + (uint32_t)j * (P::THREADS * 16u), voff, 0u);
      dma_lds16(v_rsrc, v_base + (uint32_t)j * (P::THREADS * 16u), voff, 0u);
    }
    wait_tile_loads<0>();
    __syncthreads();  // the rectangle is read-only from here on
  }
  // a query wavefront below the grid (last patch row of a ragged grid) has no work; with two
  // parts it still meets the other part at the end
  const bool rows_in = y0 + 2 * wave < H;
  if (P::PARTS == 1 && !rows_in) return;

  bf16x8_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    u32x4_t x = qraw[kb];
    asm volatile("" : "+v"(x));  // keeps the wait for Q after the rectangle's copy has been issued
    x ^= a.q_sign;               // negative scale: flip Q's sign bits, use |scale|
    qf[kb] = __builtin_bit_cast(bf16x8_t, q_ok ? x : u32x4_t{0, 0, 0, 0});
  }

  // ---- this wavefront's key rows: the band of its two query rows, a run of the patch's band
  const int32_t wy0 = imin(y0 + 2 * wave, H - 1);
  const Band wb = na_band(wy0, imin(wy0 + 1, H - 1), H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h);
  int32_t off = wb.start - pb.rows.start;
  off += off < 0 ? H : 0;
  const int32_t n_steps = rows_in ? (wb.count + SB - 1) / SB : 0;

  // The window along an axis is `kernel` cells `dil` apart from its first cell (the
  // query's coordinate less rad * dil when wrapped, its anchor when clamped: na_dil_ok;
  // mod the axis length when wrapped); in band cells it starts lo cells into the band.
  // Window bits of the lane's column: bit x for column band cell x (a wrapped window on
  // an axis no longer than the band runs past the band's end and continues at cell 0);
  // of its row: bit r for band row r. Element e of a 32-key block of the lane holds
  // column cell 8 (e / 4) + 4 half + e % 4.
  auto win_first = [](int32_t c, int32_t len, int32_t kernel, int32_t rad, int32_t wrap, int32_t dil) {
    if (wrap) return c - rad * dil;
    return dil == 1 ? iclamp(c - rad, 0, len - kernel) : na_dil_anchor(c, len, kernel, rad, wrap, dil);
  };
  // kernel cells dil apart from bit lo (below bit 64): one run of bits when undilated
  auto cells = [](int32_t lo, int32_t kernel, int32_t dil) -> uint64_t {
    if (dil == 1) return ((uint64_t{1} << kernel) - 1u) << lo;
    uint64_t m = 0;
    for (int32_t t = 0; t < kernel; ++t) m |= uint64_t{1} << (lo + dil * t);
    return m;
  };
  int32_t lo_x = win_first(qx, W, g.kernel_w, g.rad_w, g.wrap_w, g.dil_w) - pb.cols.start;
  lo_x += lo_x < 0 ? W : 0;
  uint64_t cm64 = cells(lo_x, g.kernel_w, g.dil_w);
  cm64 |= cm64 >> pb.cols.count;  // the wrapped tail (cols.count = W here), else bits past 32 only
  const uint32_t cm = (uint32_t)cm64 & (uint32_t)((1ull << pb.cols.count) - 1ull);
  int32_t lo_y = win_first(qy, H, g.kernel_h, g.rad_h, g.wrap_h, g.dil_h) - pb.rows.start;  // the band holds the window
  lo_y += lo_y < 0 ? H : 0;
  const uint32_t rows_w = (uint32_t)cells(lo_y, g.kernel_h, g.dil_h);  // below the band's count (< 32)
  uint32_t cm16 = 0;
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) cm16 |= ((cm >> (8 * g4 + 4 * half)) & 0xFu) << (4 * g4);
  cm16 = q_ok ? cm16 : 0u;

  // LDS read offsets of the transposing V read (as in the tile kernel)
  const int k_swz = chunk_swizzle<D>(col);
  int v_row[2], v_off[2][DT];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v_row[h] = h * 8 + half * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dcol = dt * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
      v_off[h][dt] = (((dcol >> 3) ^ chunk_swizzle<D>(v_row[h])) << 3) + (dcol & 7);
    }
  }

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -FLT_MAX, l_run = 0.f;
  float bias[16];  // the lane's column window as an addend: 0 in the window, -inf outside
#pragma unroll
  for (int e = 0; e < 16; ++e) bias[e] = ((cm16 >> e) & 1u) ? 0.f : -INFINITY;

  // four key rows per step (window_step): with a wavefront's few rows per part, the four
  // blocks' independent products keep the matrix core busier than a row-by-row walk
  // (row_update), which ran 0.78-0.93x here
  for (int32_t st = part; st < n_steps; st += P::PARTS) {
    const int32_t r0 = off + SB * st;  // first band row of the step (r0 + 3 < pb.rows.count + 3)
    const uint16_t* kb[SB];
    const uint16_t* vb[SB];
    bool live[SB];  // the block's key row within this wavefront's band and the query's row window
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      kb[sb] = k_lds + (r0 + sb) * kPatchKeyCols * D;
      vb[sb] = v_lds + (r0 + sb) * kPatchKeyCols * D;
      live[sb] = ((rows_w >> (r0 + sb)) & 1u) != 0u;
    }
    window_step<D>(kb, vb, live, bias, SB, st == part, qf, c, col, half, k_swz, v_row, v_off, oacc, m_run, l_run);
  }

  if constexpr (P::PARTS > 1) {
    // the second part leaves O, m and l (per lane, in lane order); the first combines
    constexpr int F = DT * 16 + 2;
    float* slot = merge_lds + wave * F * 64 + lane;
    if (part == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) slot[(dt * 16 + e) * 64] = oacc[dt][e];
      slot[(F - 2) * 64] = m_run;
      slot[(F - 1) * 64] = l_run;
    }
    __syncthreads();
    if (part == 1 || !rows_in) return;
    const float m1 = slot[(F - 2) * 64], l1 = slot[(F - 1) * 64];
    const float m_new = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - m_new), a1 = __builtin_amdgcn_exp2f(m1 - m_new);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] = oacc[dt][e] * a0 + slot[(dt * 16 + e) * 64] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = m_new;
  }

  // ---- delayed division and store (lane `col` of the first half-wave also writes the logsumexp)
  const float l_tot = swap_halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* __restrict__ oh = a.o + head;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4_t ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(oacc[dt][g4 * 4 + e] * inv);
        *reinterpret_cast<u32x2_t*>(oh + (size_t)my_q * D + dt * 32 + g4 * 8 + half * 4) = __builtin_bit_cast(u32x2_t, ob);
      }
    if (a.lse != nullptr && half == 0) a.lse[(size_t)bh * N + my_q] = row_lse(m_run, l_tot);
  }
}

// ---------------------------------------------------------------------------
// Neighbourhood windows on grids at most 32 wide by grid rows (MASK_NA_ROWS,
// na_rows_eligible): wavefront w of a work-group holds row w of its row group (RowGroup) of plane z
// (lane column = grid column). The planes the windows reach stream through two LDS
// stages; a stage holds the work-group's band of key rows of one plane, each row
// as one 32-key block. A wavefront's window over a stage is uniform in its rows
// (the key row is in or out for every lane) and the lane's own column bits inside
// a block, so each wavefront runs over just its visible rows, one at a time with
// the next row's scores issued before this row's exponentials (row_scores,
// row_update), with the lane's column bits as the exponent's addend. (Four rows per
// step through window_step, with no overlap between steps, ran 0.75x.)
template <int D, int ROWS_>
struct RowsCfg {
  static constexpr int ROWS = ROWS_;  // key rows per stage: 20 KB of K or V at d = 32 and 10 rows
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int CHUNKS = ROWS * 32 * ROW_CHUNKS;  // 16-byte chunks of a stage of K (or V)
  static_assert(CHUNKS % 256 == 0, "a stage is copied in whole rounds of 256 lanes");
  static constexpr int LOADS = CHUNKS / 256;  // per lane, stage and tensor
  static constexpr int ELEMS = CHUNKS * 8;
};

// two work-groups per CU with the narrow stages at d = 32 (80 KB of LDS each), one with the wide
// ones and at d = 64 (128 KB)
template <int D, int ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 32 && ROWS <= 10 ? 2 : 1)))
void attn_fwd_na_rows_kernel(KernelArgs a) {
  using R = RowsCfg<D, ROWS>;
  constexpr int KB = D / 16, DT = D / 32, RC = D / 8;
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][R::ELEMS];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][R::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const NaGeom& g = a.na;
  const int32_t H = g.grid_h, W = g.grid_w, N = a.Nq;
  const float c = a.c;

  // (head, plane, group of 4 rows), the items of one head kept on one XCD
  const int32_t groups = a.patch_ny, per_head = g.grid_d * groups;
  const int32_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int32_t bh = item / per_head, rest = item - bh * per_head;
  const int32_t z = rest / groups;
  const RowGroup rg = na_row_group(g, rest - z * groups, false);
  const int32_t y = rg.rho + rg.stride * (rg.u0 + wave);  // this wavefront's grid row
  const bool row_in = rg.u0 + wave < rg.len;
  const bool q_ok = row_in && col < W;
  const int32_t my_q = (z * H + y) * W + col;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * (uint32_t)(D * 2);

  // ---- the lane's query, loaded first; used after the first stage has landed
  const int32_t q_row = q_ok ? my_q : 0;
  u32x4_t qraw[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    qraw[kb] = *reinterpret_cast<const u32x4_t*>(a.q + head + (size_t)q_row * D + kb * 16 + half * 8);

  const Band bz = na_band(z, z, g.grid_d, g.kernel_d, g.rad_d, g.wrap_d, g.dil_d);
  const Band by = rg.band;  // by.count <= R::ROWS
  // Planes are visited from the work-group's own plane (always in its window, so its
  // stage can be requested before any mask is built) through the band, circularly.
  int32_t i_own = z - bz.start;
  i_own += i_own < 0 ? g.grid_d : 0;
  auto plane_at = [&](int32_t j) {  // plane of the j-th band cell visited
    int32_t i = i_own + j;
    i -= i >= bz.count ? bz.count : 0;
    const int32_t zk = bz.start + i;
    return zk >= g.grid_d ? zk - g.grid_d : zk;
  };

  // ---- a stage: the band rows of one plane; LDS chunk p holds chunk (p % RC) ^ swizzle of
  // key p / RC = 32 r + x (band row r, column x); columns past W and rows past the band
  // read as zero (an offset past the head)
  const i32x4_t k_rsrc = head_rsrc(a.k + head, head_bytes);
  const i32x4_t v_rsrc = head_rsrc(a.v + head, head_bytes);
  auto load_stage = [&](int32_t zk, int stage) {
    const uint32_t k_base = __builtin_amdgcn_readfirstlane(lds_addr(k_lds[stage]) + wave * 1024);
    const uint32_t v_base = __builtin_amdgcn_readfirstlane(lds_addr(v_lds[stage]) + wave * 1024);
#pragma unroll
    for (int j = 0; j < R::LOADS; ++j) {
      const int32_t p = j * 256 + tid;
      const int32_t key = p / RC, r = key / 32, x = key % 32;
      const int32_t chunk = (p % RC) ^ chunk_swizzle<D>(key);
      uint32_t voff = head_bytes;
      if (r < by.count && x < W) {
        const int32_t yk = row_group_row(rg, r);
        voff = (uint32_t)((zk * H + yk) * W + x) * (uint32_t)(D * 2) + (uint32_t)chunk * 16u;
      }
      dma_lds16(k_rsrc, k_base + (uint32_t)j * 4096u, voff, 0u);
      dma_lds16(v_rsrc, v_base + (uint32_t)j * 4096u, voff, 0u);
    }
  };

  load_stage(z, 0);

  // window masks per axis (rows and planes are the same for every lane of a wavefront)
  const GridMasks gm = na_grid_masks(z, imin(y, H - 1), imin(col, W - 1), g);
  // the lane's columns (bit x of the low word, x < W <= 32) as a per-element bias: 0 for a
  // key in the window, -inf for the rest (and for a lane outside the grid)
  const uint32_t cm16 = q_ok ? lane_block_bits((uint32_t)gm.x0, half) : 0u;
  float bias[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) bias[e] = ((cm16 >> e) & 1u) ? 0.f : -INFINITY;
  uint32_t rows_vis = 0;  // bit r: band row r in this wavefront's row window
  for (int32_t r = 0; r < by.count; ++r) {
    rows_vis |= (uint32_t)bit128(gm.y0, gm.y1, row_group_row(rg, r)) << r;
  }
  rows_vis = row_in ? __builtin_amdgcn_readfirstlane(rows_vis) : 0u;
  auto next_plane = [&](int32_t j) {  // first visit from j whose plane is in the window (uniform)
    while (j < bz.count && __builtin_amdgcn_readfirstlane((int)bit128(gm.z0, gm.z1, plane_at(j))) == 0) ++j;
    return j;
  };

  // LDS read offsets (as in the tile kernel)
  const int k_swz = chunk_swizzle<D>(col);
  int v_row[2], v_off[2][DT];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v_row[h] = h * 8 + half * 4 + ((lane & 15) >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dcol = dt * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
      v_off[h][dt] = (((dcol >> 3) ^ chunk_swizzle<D>(v_row[h])) << 3) + (dcol & 7);
    }
  }

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = q_ok ? -FLT_MAX : 0.f, l_run = 0.f;  // row_update sets a lane's maximum at its first visible key
  bf16x8_t qf[KB];
  for (int32_t i = 0, it = 0, stage = 0; i < bz.count; ++it, stage ^= 1) {
    const int32_t i_next = next_plane(i + 1);
    const bool more = i_next < bz.count;
    // the next plane's rows go into the other stage (last read before the previous barrier);
    // on the first pass they are issued after the wait, so that Q's wait does not take them in
    if (it > 0 && more) load_stage(plane_at(i_next), stage ^ 1);
    if (it > 0 && more)
      wait_tile_loads<2 * R::LOADS>();
    else
      wait_tile_loads<0>();
    __syncthreads();
    if (it == 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4_t x = qraw[kb];
        asm volatile("" : "+v"(x));  // keeps the wait for Q after the first stage's copy has been issued
        x ^= a.q_sign;               // negative scale: flip Q's sign bits, use |scale|
        qf[kb] = __builtin_bit_cast(bf16x8_t, q_ok ? x : u32x4_t{0, 0, 0, 0});
      }
      if (more) load_stage(plane_at(i_next), stage ^ 1);
    }
    // this wavefront's visible rows of the stage, in order, one at a time: the next row's
    // scores are issued before this row's exponentials
    const uint16_t* ks = k_lds[stage];
    const uint16_t* vs = v_lds[stage];
    uint32_t rem = rows_vis;
    if (rem != 0u) {
      int32_t r = __builtin_ctz(rem);
      f32x16_t s_nx = row_scores<D>(ks + r * 32 * D, qf, col, half, k_swz);
      while (true) {
        const f32x16_t s = s_nx;
        const int32_t rc = r;
        rem &= rem - 1u;
        const bool nxt = rem != 0u;
        if (nxt) {
          r = __builtin_ctz(rem);
          s_nx = row_scores<D>(ks + r * 32 * D, qf, col, half, k_swz);
        }
        row_update<D>(s, vs + rc * 32 * D, bias, true, c, v_row, v_off, oacc, m_run, l_run);
        if (!nxt) break;
      }
    }
    __syncthreads();  // every wavefront is done with this stage before it is refilled
    i = i_next;
  }

  // ---- delayed division and store (lane `col` of the first half-wave also writes the logsumexp)
  const float l_tot = swap_halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* __restrict__ oh = a.o + head;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4_t ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (__bf16)(oacc[dt][g4 * 4 + e] * inv);
        *reinterpret_cast<u32x2_t*>(oh + (size_t)my_q * D + dt * 32 + g4 * 8 + half * 4) = __builtin_bit_cast(u32x2_t, ob);
      }
    if (a.lse != nullptr && half == 0) a.lse[(size_t)bh * N + my_q] = row_lse(m_run, l_tot);
  }
}

template <int D, int MASK, bool SPLIT>
static hipError_t launch_one(const KernelArgs& a, int32_t n_wg, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, MASK, SPLIT>), dim3(n_wg), dim3(Cfg<D>::THREADS), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const KernelArgs& a, int32_t mask, int32_t n_wg, int32_t rem, hipStream_t stream) {
  if (a.ws_parts != nullptr) {  // remainder split, no mask: the counters, then the parts' kernel
    hipLaunchKernelGGL(attn_split_clear_kernel, dim3(1), dim3(256), 0, stream, a.split_count, rem);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_one<D, MASK_NONE, true>(a, n_wg, stream);
  }
  switch (mask) {
    case MASK_NONE: return launch_one<D, MASK_NONE, false>(a, n_wg, stream);
    case MASK_CAUSAL: return launch_one<D, MASK_CAUSAL, false>(a, n_wg, stream);
    case MASK_NA: return launch_one<D, MASK_NA, false>(a, n_wg, stream);
    case MASK_NA_BLOCKS: return launch_one<D, MASK_NA_BLOCKS, false>(a, n_wg, stream);
    case MASK_NA_GRID: return launch_one<D, MASK_NA_GRID, false>(a, n_wg, stream);
    case MASK_NA_PATCH:
      if constexpr (D == 32 || D == 64) {
        hipLaunchKernelGGL((attn_fwd_na_patch_kernel<D>), dim3(n_wg), dim3(PatchCfg<D>::THREADS), 0, stream, a);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    case MASK_NA_ROWS:
      if constexpr (rows_lds_rows(D) > 0) {
        if (a.rows_stage == rows_lds_rows(D)) {
          hipLaunchKernelGGL((attn_fwd_na_rows_kernel<D, rows_lds_rows(D)>), dim3(n_wg), dim3(256), 0, stream, a);
          return hipGetLastError();
        }
      }
      if constexpr (rows_wide_lds(D) > 0) {
        if (a.rows_stage == rows_wide_lds(D)) {
          hipLaunchKernelGGL((attn_fwd_na_rows_kernel<D, rows_wide_lds(D)>), dim3(n_wg), dim3(256), 0, stream, a);
          return hipGetLastError();
        }
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// The split workspace of attn_fwd_ex_static: one array per device, kept until the
// process ends and shared by every call on that device (calls that overlap on one
// device race for it). It needs no initial content.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void* addr[kDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // host code sees `scratch` only as a stand-in: the device address comes from the runtime
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_fwd(const KernelArgs& a, int32_t d, int32_t mask, int32_t n_wg, int32_t rem, hipStream_t stream) {
  switch (d) {
    case 32: return launch_d<32>(a, mask, n_wg, rem, stream);
    case 64: return launch_d<64>(a, mask, n_wg, rem, stream);
    case 128: return launch_d<128>(a, mask, n_wg, rem, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
