// Shared device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tdl {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

// LDS (address space 3) pointer, the destination type of direct-to-LDS loads
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
constexpr float kF16Max = 65504.f;

// fp32 -> fp16, round to nearest even, saturating at +-65504.
__device__ __forceinline__ f16 f32_to_f16_sat(float v) {
  return (f16)fminf(fmaxf(v, -kF16Max), kF16Max);
}

// Element type of an MFMA operand: bf16 or fp16 (same rate on gfx950; fp16
// keeps 11 significant bits, bf16 8).
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  typedef bf16x8 v8;
  __device__ static f32x4 mma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static bf16 from_f32(float v) { return (bf16)v; }
};
template <> struct Mfma<f16> {
  typedef f16x8 v8;
  __device__ static f32x4 mma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static f16 from_f32(float v) { return f32_to_f16_sat(v); }
};
constexpr int kBlockTokens = 16;

__device__ __forceinline__ float bf16_to_f32(bf16 v) { return (float)v; }
// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ bf16 f32_to_bf16(float v) { return (bf16)v; }

__device__ __forceinline__ uint16_t bf16_bits(bf16 v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ bf16 bits_bf16(uint16_t v) { return __builtin_bit_cast(bf16, v); }

// Lanes l and l ^ 32 (l ^ 16) combined on the VALU, without the LDS
// permute (whose wait also waits for every LDS access issued before it):
// given the same register twice, v_permlane32_swap (v_permlane16_swap, over
// rows of 16 lanes) leaves each lane the pair {x[l], x[l ^ 32]} ({x[l],
// x[l ^ 16]}), so the max or the sum of the pair is the same on both lanes.
// The whole wave must be active.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP move within rows of 16 lanes (quad_perm, row_mirror, row_half_mirror)
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the wave, the same value on every lane, all on the VALU: lanes
// l ^ 1 and l ^ 2 by quad permutations; then the half-row and row mirrors
// (lane i with 7 - i, then with 15 - i), which pair lanes whose groups
// already agree; then lanes l ^ 16 and l ^ 32.  The whole wave must be
// active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x140>(v);  // row_mirror
  return sum_xor32(sum_xor16(v));
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// 16x16x32 bf16 MFMA: D = A(16x32) * B(32x16) + C.  Lane l supplies 8 values
// of row l%16 of A and of column l%16 of B; both use the same k order, so any
// pairing that loads A and B alike contracts correctly.  D: lane l holds
// rows 4*(l/16)+0..3 of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16 bf16 MFMA: lane l supplies A[l%16][4*(l/16)+0..3] and
// B[4*(l/16)+0..3][l%16]; D as above.
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// The same two shapes with fp16 operands.
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace tdl
