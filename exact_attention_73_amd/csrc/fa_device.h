// Device-side helpers shared by the gfx950 kernels of this library.
//
// Matrix-instruction conventions used throughout (CDNA4, wave64):
//
//  v_mfma_f32_32x32x16_bf16  D(32x32,f32) += A(32x16,bf16) * B(16x32,bf16)
//    A: lane L holds row (L & 31), eight consecutive k of k-group (L >> 5)
//    B: lane L holds column (L & 31), the same eight k
//    D: lane L, register r holds row 8*(r/4) + 4*(L>>5) + (r&3), column L&31
//  v_mfma_f32_32x32x64_f8f6f4 (E4M3 operands): the same, with 32 k per lane.
//
// Only the row/column placement matters for correctness: whatever order the
// hardware pairs k inside a lane group, A and B are always filled with the
// same k at the same (lane group, item) slot, so the contraction covers each
// k exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescale of the online softmax (bf16 forward and decode): the exponent
// reference of a row moves only when its max grows by more than this many
// log2 units, so P <= 2^kLazyLog2 and O, l are rescaled only then.
constexpr float kLazyLog2 = 8.f;

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// E4M3 x E4M3 with E8M0 block exponents (127 = 2^0) for A and B.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine lane L's value with lane L ^ 32's (the other half of the wave)
// without a trip through LDS: v_permlane32_swap exchanges lanes 32..63 of its
// first operand with lanes 0..31 of its second, so with x in both, the two
// results hold x[L] and x[L ^ 32] in every lane (which one is which depends on
// the half; max and + do not care, and give the same bits in both halves).
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fmax3(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

// Round two floats to bf16 (nearest even) and pack them, low word = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 h = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Byte permute of two dwords (v_perm_b32): selector bytes 0-3 pick from lo,
// 4-7 from hi.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Workgroup index remapped so that each of the 8 XCDs (which receive
// workgroups round-robin by index) walks a contiguous slice of the work
// list; neighbouring work items then share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
  if (n & 7) return bid;
  return (bid & 7) * (n >> 3) + (bid >> 3);
}

// Causal workgroup order of the ping-pong kernels (bf16 and FP8).  Workgroups reach the 8
// XCDs round-robin by index, so XCD x runs workgroups x, x + 8, ...  Heads
// are pinned to XCDs (x takes heads x, x + 8, ...) and each XCD walks its
// heads four at a time, the heaviest query tiles first within each group of
// four (heads alternating).  Against a global heavy-first order (every head
// in flight on every XCD) this cuts the K/V bytes fetched from HBM from
// 2.5-3.3 to 1.5-1.8 times the algorithmic bytes at N = 2048-4096, at equal
// speed; walking one head at a time reaches 1.0 but leaves the heavy tiles
// of each XCD's last head for the end (10-20 % slower).  Grids whose head
// count does not split into such groups keep the global order.
__device__ __forceinline__ void causal_order(int BH, int nq, int& bh, int& qt) {
  constexpr int G = 4;
  if ((BH & 7) == 0 && ((BH >> 3) % G) == 0) {
    const int x = (int)blockIdx.x & 7, j = (int)blockIdx.x >> 3;
    const int g = j / (G * nq), r = j - g * (G * nq);
    qt = nq - 1 - r / G;
    bh = x + 8 * (g * G + r % G);
  } else {
    qt = nq - 1 - (int)blockIdx.x / BH;
    bh = (int)blockIdx.x % BH;
  }
}

}  // namespace fa
