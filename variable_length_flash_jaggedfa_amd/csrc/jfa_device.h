// Device helpers shared by the gfx950 kernels of libjfa.
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_bf16, one wave of 64
// lanes, lane = 32*g + li with g in {0,1}, li in [0,32)):
//   A operand (32 x 16, M x K): lane holds 8 bf16 of row m = li, k-chunk g.
//   B operand (16 x 32, K x N): lane holds 8 bf16 of column n = li, k-chunk g.
//   C/D (32 x 32 fp32): lane holds 16 floats; register r is row
//       (r/4)*8 + 4*g + (r%4), column li.
// The hardware's order of k inside a chunk is the same for A and B, so any
// consistent assignment of contraction indices to (g, element) is valid; the
// kernels rely on that when they feed an accumulator tile back in as an operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jfa_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two floats -> two bf16 (round to nearest even), packed low/high
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// 2^x on the transcendental unit
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// combine a value with the one held by lane (lane ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A value every lane of the wave holds, moved to a scalar register (the
// compiler cannot prove this for loads from buffers the kernel may also write).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// A schedule or offsets entry the whole wave reads at one address, loaded into a
// scalar register through the scalar data cache. The pointer is taken as constant
// memory, which the compiler may read with scalar loads wherever the address is
// uniform: the schedule and offsets are written before the launch and never
// while a kernel runs. (Through the vector path, each tile's two dependent
// lookups cost two round trips to L2 and a wait on every vector load in flight.)
__device__ __forceinline__ int sload(const int* p) {
  return *(const __attribute__((address_space(4))) int*)p;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

// 16-bit element e (0..7) of a 16-byte vector
__device__ __forceinline__ uint32_t half_of(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Persistent-slot index of this workgroup. Workgroups are dispatched round-robin
// over the 8 XCDs, so workgroup w runs on XCD w % 8; renumbering makes slots
// s and s+1 share an XCD (and its L2) whenever the grid is a multiple of 8.
__device__ __forceinline__ int xcd_slot(int wg, int grid) {
  if (grid % 8) return wg;
  return (wg % 8) * (grid / 8) + wg / 8;
}

// Key position inside a 16-key group as stored in transposed LDS tiles: bits 2
// and 3 swapped, so that the 8 keys one lane group feeds to an MFMA k-chunk
// (taken from an accumulator tile) are contiguous.
__device__ __forceinline__ int kperm(int j) {
  return (j & ~0xC) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace jfa_dev
