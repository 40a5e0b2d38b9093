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
// 64 tokens stream through a double-buffered LDS ring shared by the 4
// wavefronts; the next tile's global loads are in flight while the current
// tile is computed.
//
// Per key tile and wavefront:
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, K from LDS (A operand), Q held
//                   in registers for the whole loop (B operand). Each lane then
//                   holds 16 keys of one query column per 32-key block, so
//                   row reductions are in-lane plus one exchange between the
//                   two half-waves (v_permlane32_swap).
//   running max     m_new = max(m, c * rowmax(S)), alpha = 2^(m - m_new), with
//                   c = |scale| * log2(e) (exp2 replaces exp).
//   P = 2^(c S - m) fp32, rounded to bfloat16 for the second product;
//                   l = alpha * l + rowsum of the rounded P, kept per lane.
//   O^T = V^T P^T   v_mfma_f32_32x32x16_bf16 with P straight from registers
//                   (B operand) and V read from LDS with ds_read_b64_tr_b16,
//                   which hands each lane 4 consecutive keys of one d column.
//                   The key order inside a 16-key MFMA block follows the
//                   accumulator layout of S^T; the V reads use the same order.
// Finally O / l (delayed division), rounded to bfloat16 (nearest even).
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "attn.h"
#include "launch.hpp"
#include "tile_plan.hpp"

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

template <int D>
struct Cfg {
  static constexpr int BM = 128;     // queries per work-group (4 wavefronts x 32)
  static constexpr int BN = 64;      // keys per tile
  static constexpr int THREADS = 256;
  // LDS row strides in 16-bit elements. K rows are read 16 bytes per lane,
  // 32 rows at a time: a stride of 36 (D=64) or 20 (D=32) banks spreads 16
  // consecutive rows over all 64 banks. V rows are read 8 bytes per lane by
  // the transposing load, 4 rows x 64 bytes per half-wave: a stride of
  // 64 bytes modulo 256 puts those 4 rows on disjoint banks.
  static constexpr int KSTR = D + 8;
  static constexpr int VSTR = D == 64 ? 96 : 32;
  static constexpr int K_TILE = BN * KSTR;
  static constexpr int V_TILE = BN * VSTR;
  static constexpr int CHUNKS_PER_ROW = D / 8;                       // 16-byte chunks
  static constexpr int CHUNKS_PER_THREAD = BN * CHUNKS_PER_ROW / THREADS;
  static_assert(BN * CHUNKS_PER_ROW % THREADS == 0, "tile chunks must split evenly");
};

static_assert(Cfg<64>::BM == kBlockM && Cfg<32>::BM == kBlockM, "launch geometry and kernel tile must agree");

__device__ __forceinline__ float swap_halves_max(float x) {
  // each lane ends up with the max of itself and the lane 32 positions away
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__device__ __forceinline__ void load_tile_regs(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                                               int32_t N, int32_t tile, int tid,
                                               u32x4_t (&kr)[Cfg<D>::CHUNKS_PER_THREAD],
                                               u32x4_t (&vr)[Cfg<D>::CHUNKS_PER_THREAD]) {
  using C = Cfg<D>;
#pragma unroll
  for (int j = 0; j < C::CHUNKS_PER_THREAD; ++j) {
    const int c = tid + j * C::THREADS;
    const int row = c / C::CHUNKS_PER_ROW, col = c % C::CHUNKS_PER_ROW;
    const int32_t key = tile * C::BN + row;
    if (key < N) {
      const size_t off = (size_t)key * D + col * 8;
      kr[j] = *reinterpret_cast<const u32x4_t*>(kh + off);
      vr[j] = *reinterpret_cast<const u32x4_t*>(vh + off);
    } else {
      kr[j] = u32x4_t{0, 0, 0, 0};
      vr[j] = u32x4_t{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile_lds(uint16_t* ks, uint16_t* vs, int tid,
                                               const u32x4_t (&kr)[Cfg<D>::CHUNKS_PER_THREAD],
                                               const u32x4_t (&vr)[Cfg<D>::CHUNKS_PER_THREAD]) {
  using C = Cfg<D>;
#pragma unroll
  for (int j = 0; j < C::CHUNKS_PER_THREAD; ++j) {
    const int c = tid + j * C::THREADS;
    const int row = c / C::CHUNKS_PER_ROW, col = c % C::CHUNKS_PER_ROW;
    *reinterpret_cast<u32x4_t*>(ks + row * C::KSTR + col * 8) = kr[j];
    *reinterpret_cast<u32x4_t*>(vs + row * C::VSTR + col * 8) = vr[j];
  }
}

// Integer division for the small divisors of the grid geometry.
__device__ __forceinline__ void divmod_u32(uint32_t n, uint32_t d, int32_t& q, int32_t& r) {
  q = (int32_t)(n / d);
  r = (int32_t)(n - (uint32_t)q * d);
}

template <int D, int MASK>
__global__ __launch_bounds__(256) void attn_fwd_kernel(KernelArgs a) {
  using C = Cfg<D>;
  constexpr int KB = D / 16;     // 16-wide contraction blocks over d for S^T
  constexpr int DT = D / 32;     // 32-row output tiles over d for O^T
  constexpr int SB = C::BN / 32; // 32-key blocks per key tile

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][C::K_TILE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][C::V_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column owned by this lane
  const int half = lane >> 5;  // which half-wave

  const WorkItem w = work_item(MASK, blockIdx.x, gridDim.x, a.n_qtiles, a.BH);
  const int32_t N = a.N;
  const int32_t q0 = w.qtile * C::BM;
  const size_t head_off = (size_t)w.bh * (size_t)N * D;
  const uint16_t* __restrict__ qh = a.q + head_off;
  const uint16_t* __restrict__ kh = a.k + head_off;
  const uint16_t* __restrict__ vh = a.v + head_off;
  uint16_t* __restrict__ oh = a.o + head_off;

  // ---- Q fragment: B operand of S^T = K Q^T; lane holds d = 16kb + 8*half + 0..7 of its query
  const int32_t my_q = q0 + wave * 32 + col;
  bf16x8_t qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    u32x4_t x = u32x4_t{0, 0, 0, 0};
    if (my_q < N) {
      x = *reinterpret_cast<const u32x4_t*>(qh + (size_t)my_q * D + kb * 16 + half * 8);
      x ^= a.q_sign;  // negative scale: flip Q's sign bits, use |scale|
    }
    qf[kb] = __builtin_bit_cast(bf16x8_t, x);
  }

  // ---- neighbourhood coordinates of this lane's query
  int32_t yq = 0, xq = 0;
  if (MASK == MASK_NA2D) divmod_u32((uint32_t)my_q, (uint32_t)a.na.grid_w, yq, xq);

  const int32_t n_kv = a.n_kvtiles;
  const KvRun run = kv_run(MASK, N, C::BM, C::BN, q0, a.na);

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -FLT_MAX;  // running max of c * S (finite sentinel: no inf - inf)
  float l_run = 0.f;       // this lane's share of the row sum
  const float c = a.c;

  u32x4_t kr[C::CHUNKS_PER_THREAD], vr[C::CHUNKS_PER_THREAD];
  load_tile_regs<D>(kh, vh, N, kv_tile_at(run, 0, n_kv), tid, kr, vr);
  store_tile_lds<D>(k_lds[0], v_lds[0], tid, kr, vr);
  __syncthreads();

  for (int32_t i = 0; i < run.count; ++i) {
    const int buf = i & 1;
    const int32_t t = kv_tile_at(run, i, n_kv);
    const bool has_next = i + 1 < run.count;
    if (has_next) load_tile_regs<D>(kh, vh, N, kv_tile_at(run, i + 1, n_kv), tid, kr, vr);

    const uint16_t* ks = k_lds[buf];
    const uint16_t* vs = v_lds[buf];

    // ---- S^T = K Q^T: lane holds keys 32sb + 8(r/4) + 4*half + r%4 of its query column
    f32x16_t s[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      s[sb] = f32x16_t{};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4_t kx = *reinterpret_cast<const u32x4_t*>(ks + (sb * 32 + col) * C::KSTR + kb * 16 + half * 8);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx), qf[kb], s[sb], 0, 0, 0);
      }
    }

    // ---- element mask on tiles that need it (uniform branch)
    const bool masked = tile_needs_mask(MASK, N, C::BN, q0, t);
    if (masked) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int32_t key = t * C::BN + sb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          bool ok = key < N;
          if (MASK == MASK_CAUSAL) ok = ok && key <= my_q;
          if (MASK == MASK_NA2D) {
            int32_t yk, xk;
            divmod_u32((uint32_t)key, (uint32_t)a.na.grid_w, yk, xk);
            ok = ok && na_axis_ok(yq, yk, a.na.grid_h, a.na.kernel_h, a.na.rad_h, a.na.wrap_h) &&
                 na_axis_ok(xq, xk, a.na.grid_w, a.na.kernel_w, a.na.rad_w, a.na.wrap_w);
          }
          if (!ok) s[sb][r] = -INFINITY;
        }
      }
    }

    // ---- running max over this tile
    float mx = s[0][0];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
    mx = swap_halves_max(mx);
    const float cand = mx == -INFINITY ? -FLT_MAX : mx * c;
    const float m_new = fmaxf(m_run, cand);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    // ---- P = 2^(c S - m), rounded to bfloat16 for the second product. The row
    // sum adds the same rounded values (two per v_dot2 against (1, 1)), so the
    // weights that multiply V are exactly the ones the final division uses.
    bf16x8_t pb[SB][2];
    float psum = 0.f;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][kb2 * 8 + e], c, -m_new));
          float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][kb2 * 8 + e + 1], c, -m_new));
          if (masked) {
            p0 = s[sb][kb2 * 8 + e] == -INFINITY ? 0.f : p0;
            p1 = s[sb][kb2 * 8 + e + 1] == -INFINITY ? 0.f : p1;
          }
          const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
          pb[sb][kb2][e] = pp[0];
          pb[sb][kb2][e + 1] = pp[1];
          psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
        }
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          // slot 8*half + e of this block holds key 32sb + 16kb2 + 8(e/4) + 4*half + e%4
          bf16x8_t vf;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int key = sb * 32 + kb2 * 16 + h * 8 + half * 4 + ((lane & 15) >> 2);
            const int dcol = dt * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
            const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)((lds_u16*)vs + key * C::VSTR + dcol));
            const bf16x4_t xb = __builtin_bit_cast(bf16x4_t, x);
#pragma unroll
            for (int e = 0; e < 4; ++e) vf[h * 4 + e] = xb[e];
          }
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[sb][kb2], oacc[dt], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile_lds<D>(k_lds[buf ^ 1], v_lds[buf ^ 1], tid, kr, vr);
    __syncthreads();
  }

  // ---- delayed division and store: lane holds d = 32dt + 8(r/4) + 4*half + r%4
  const float l_tot = swap_halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (my_q < N) {
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
  }
}

template <int D, int MASK>
static hipError_t launch_one(const KernelArgs& a, int32_t n_wg, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, MASK>), dim3(n_wg), dim3(Cfg<D>::THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const KernelArgs& a, int32_t d, int32_t mask, int32_t n_wg, hipStream_t stream) {
  if (d == 64) {
    if (mask == MASK_CAUSAL) return launch_one<64, MASK_CAUSAL>(a, n_wg, stream);
    if (mask == MASK_NA2D) return launch_one<64, MASK_NA2D>(a, n_wg, stream);
    return launch_one<64, MASK_NONE>(a, n_wg, stream);
  }
  if (mask == MASK_CAUSAL) return launch_one<32, MASK_CAUSAL>(a, n_wg, stream);
  if (mask == MASK_NA2D) return launch_one<32, MASK_NA2D>(a, n_wg, stream);
  return launch_one<32, MASK_NONE>(a, n_wg, stream);
}

int32_t tile_keys() { return Cfg<64>::BN; }

}  // namespace attn
