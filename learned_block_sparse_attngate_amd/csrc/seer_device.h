// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, MFMA wrapper and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seer {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;      // gate pooling window == attention tile edge
constexpr int kWave = 64;       // CDNA wavefront size

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two fp32 -> packed bf16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t p = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, p);
}

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate (gfx950).
// Lane l supplies A[l % 32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l % 32];
// it receives C[8*(r/4) + 4*(l/32) + r%4][l % 32] in element r.
__device__ __forceinline__ f32x16_t mfma_32x32x16(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Combine the values of lanes l and l ^ 32 (both lanes get the result).
// v_permlane32_swap with the same register as both operands leaves one
// lane-half's own value and the partner's value in the two results, in an
// order that differs between the halves; max and + are symmetric, so the
// order does not matter and both lanes compute bit-identical results.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

}  // namespace seer
