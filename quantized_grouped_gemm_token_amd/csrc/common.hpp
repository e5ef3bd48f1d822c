// Device helpers shared by the W4A8 MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 128;      // INT4 group size along K
constexpr float kFp8Max = 448.0f;

// E4M3FN code of an fp32 value: round to nearest, ties to even, saturating at
// +-448, sign kept on zero (OCP 8-bit floating point, E4M3 variant).  Integer
// arithmetic on the fp32 bit pattern, so the result is the same on every
// device.  NaN inputs are outside the domain.
//  * |v| >= 448                 -> 0x7E (the largest finite magnitude)
//  * |v| <  2^-5                -> rint(|v| * 2^9): in this range E4M3 is
//    evenly spaced by 2^-9 (subnormals, then the first normal binade), so the
//    code is the value in units of 2^-9; 2^-5 itself is code 0x10
//  * otherwise                  -> keep 3 mantissa bits with round-half-even on
//    the 20 dropped bits and rebias the exponent from 127 to 7 (a mantissa
//    carry moves into the exponent field, which is the right next code)
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {              // 448.0f
    code = 0x7eu;
  } else if (a < 0x3d000000u) {        // 2^-5
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return code | sign;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// SwiGLU of one gate/up pair in fp32: silu(g) * u, silu(g) = g / (1 + e^-g)
// (no clamp), with the hardware exponential and reciprocal (each within 1
// ulp; the result within a few ulp of the exact value, far below the FP8 or
// INT8 step that follows).  The SwiGLU kernel and the fused gate/up
// epilogues both use this one expression, so they produce the same bits.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Max of v over each row of 16 lanes (one MFMA D column group), left in
// every lane of the row: DPP row rotations by 8, 4, 2 and 1 (register
// moves, no LDS round trip).
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, true)));   // row_ror:8
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, true)));   // row_ror:4
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xf, 0xf, true)));   // row_ror:2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, true)));   // row_ror:1
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

}  // namespace w4a8
