// Device building blocks shared by the forward and backward kernels: vector
// types, the LDS row swizzle, half-wave reductions, buffer resources and the
// global -> LDS tile copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, fully unrolled.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// Rows live unpadded in LDS; the 16-byte chunks of a row are permuted by an XOR
// with a function of the row so that both read patterns are free of bank
// conflicts (64 banks of 4 bytes):
//  * S^T = K Q^T reads 16 bytes per lane, 16 consecutive rows at one logical
//    chunk per 16 lanes: the even rows and the odd rows must each land on 8
//    different chunk slots;
//  * the transposing V read takes 8 bytes per lane, 4 consecutive rows x 4
//    chunks per half-wave: rows r and r+2 must fall in opposite halves of the
//    8 chunk slots.
// d = 128 (16 chunks per row, a row spans every bank): the 16 rows of one K read
// need 16 different slots, and the 4 rows of one transposing V read (4 chunks
// each) need 4 different slot quarters: row r uses slot c ^ ((r & 3) << 2 | (r >> 2) & 3).
// d = 64 (8 chunks per row): row r uses slot c ^ (((r >> 1) & 1) << 2 | (r >> 2) & 3).
// d = 32 (4 chunks per row, 4 rows per 256 bytes): slot c ^ ((r >> 2) & 3).
// Every form depends on r mod 16 only.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  return (row >> 2) & 3;
}

template <int D>
__device__ __forceinline__ int lds_index(int row, int chunk, int within) {
  return row * D + ((chunk ^ chunk_swizzle<D>(row)) << 3) + within;
}

// Each lane-pair (l, l + 32) holds the same query column; combine across the two half-waves.
__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Global -> LDS copy of one K or V tile without passing through registers
// (buffer_load_dwordx4 ... lds): every instruction of a wavefront fills one
// contiguous 1 KB block of the tile, lane L writing its bytes [16L, 16L + 16).
// Each lane therefore fetches the global chunk that the swizzle places at its
// slot; that per-lane byte offset inside a tile is the same for every tile, and
// the tile's start is a scalar offset, so a load costs no vector arithmetic.
// The buffer resource spans one head (Nkv rows): rows past Nkv read as zero in
// hardware, and their keys are masked.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource (4 scalar dwords) over `bytes` bytes at `base`: stride 0,
// so offsets at or past `bytes` read as zero.
__device__ __forceinline__ i32x4_t head_rsrc(const uint16_t* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16-byte buffer load into LDS at the wave-uniform byte address `lds` (lane L
// writes bytes [lds + 16L, lds + 16L + 16)). Issued as inline assembly so the
// compiler's wait insertion does not treat it as a store that may alias every
// later LDS read: left to the compiler, each step waited for the next tile's
// loads before its first read of the current tile. Completion is awaited
// explicitly (wait_tile_loads) before the barrier that publishes the tile.
__device__ __forceinline__ void dma_lds16(i32x4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) { return (uint32_t)(uintptr_t)(lptr_t)p; }

// Race check of the hand-managed tile rings. Built with ATTN_SERIAL_TILES=1, every
// kernel issues each tile load only after the computation of its step and waits
// for all of this wavefront's loads (vmcnt(0)) before the barrier that publishes
// them: no load is in flight while any tile is read. The arithmetic is unchanged,
// so that build must agree bit for bit with the pipelined one; a wait count or
// barrier that let a step read a tile before it landed would show as a mismatch.
#ifndef ATTN_SERIAL_TILES
#define ATTN_SERIAL_TILES 0
#endif
constexpr bool kSerialTiles = ATTN_SERIAL_TILES != 0;

// Wait until at most N of this wavefront's tile loads are still in flight (loads
// complete in issue order). Every step issues the same number of loads, so a
// fixed count names exactly the tiles the next step reads.
template <int N>
__device__ __forceinline__ void wait_tile_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace attn
