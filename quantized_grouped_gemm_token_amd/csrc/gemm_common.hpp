// Pieces shared by the grouped W4A8 GEMM kernels.
//
// The GEMM never dequantizes the INT4 weights to BF16 ("GLM-5.3-W4A8" card,
// section 量化方式: the INT4 weights become FP8 inside the kernel and feed the
// FP8 matrix cores).  On gfx950 that FP8 conversion is free:
//
//   * a stored nibble u = q + 8 (0..15), zero-extended to a byte and read as
//     E4M3, is exactly u * 2^-9: E4M3 spaces its subnormals and its first
//     normal binade evenly by 2^-9, so the bytes 0x00..0x0F are linear;
//   * so  sum_k a_k q_k = 2^9 * sum_k a_k (u_k 2^-9)  -  8 * sum_k a_k.
//     The second term is one more MFMA of the same A tile against a constant
//     B of -2^-6 (E4M3 0x88), used as the accumulator input C of the real
//     MFMA:  D = A x U(2^-9) + A x (-2^-6)  = 2^-9 * A x Q   (every product
//     is exact, the sums are fp32);
//   * then acc += s[n, g] * D per 128-wide group (one fp32 FMA per output per
//     group), and the 2^9 goes into the epilogue with the token scale.
//
// The only work per weight is splitting the nibbles of a word into bytes
// (in the GEMM storage's nibble order: two ANDs and a shift per 8 weights).
#pragma once

#include "common.hpp"

namespace w4a8 {

typedef int v8i __attribute__((ext_vector_type(8)));     // 32 E4M3 bytes
typedef float v4f __attribute__((ext_vector_type(4)));   // 16x16 fp32 tile, 4 per lane

constexpr int kBiasWord = (int)0x88888888u;                // four E4M3 -2^-6
constexpr float kUnitScale = 512.0f;                        // 2^9

// v_mfma_f32_16x16x128_f8f6f4 with both operands E4M3 and no block scaling.
// Lane l supplies A row (l % 16) and B column (l % 16), K elements
// 32 * (l / 16) .. +32 of the 128 (the same K map for both operands);
// D lane l holds column l % 16, rows 4 * (l / 16) .. +3.
__device__ __forceinline__ v4f mfma16x16x128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// v_mfma_scale_f32_16x16x128_f8f6f4 with A E4M3 (unit block scales) and B
// MXFP4: E2M1 codes with E8M0 block scales applied by the matrix core.
// With an FP4 B the matrix core reads the K elements of the two operands in
// different orders:
//   B: lane l supplies column l % 16, K elements 32 (l / 16) .. +32 as 16
//      packed bytes (element k in the low nibble of byte k/2 when k is even)
//      in the first four dwords of the operand; byte 0 of its scale operand
//      is the E8M0 scale of exactly those 32 elements (one MX block);
//   A: lane l supplies row l % 16, K bytes 16 (l / 16) .. +16 in its first
//      four dwords and K bytes 64 + 16 (l / 16) .. +16 in the last four.
// D as in the FP8 form.  The products are exact; D = C + sum in fp32.
__device__ __forceinline__ v4f mfma_mx(v8i a, i32x4 b, v4f c, int scale_b) {
  const v8i bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 0, 4, 0, 0x7F7F7F7F, 0, scale_b);
}

// The three weight forms of the grouped GEMM kernels.
enum WeightForm : int {
  kFormG128 = 0,      // INT4 group 128 (uint4b8 in int32 words) x FP8 activations, fp32 group scales
  kFormChannel = 1,   // INT4 per channel x INT8 activations, int32 accumulation
  kFormMx = 2,        // MXFP4 group 32 x FP8 activations, E8M0 block scales in the matrix core
};

// INT8 matrix-core products for the per-channel variant (int32 accumulation).
// 16x16x64: lane l supplies A row (l % 16) and B column (l % 16), K elements
// 16 * (l / 16) .. +16 of the 64; D as in the 16x16 FP8 form.
// A 32-byte FP8 operand of a lane becomes two INT8 operands (its 16-byte
// halves, with the same split on both sides), so the kernels keep their FP8
// data layout: the two products cover the same K elements between them.
__device__ __forceinline__ i32x4 mfma_i8_16x16x64(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 32 nibbles of the GEMM storage (word c holds k = 8c .. 8c+7 in the nibble
// order k0 k4 k1 k5 k2 k6 k3 k7) -> 32 bytes u_k in K order, each read by the
// MFMA as u_k * 2^-9: one mask for k0..k3 and a shift and a mask for k4..k7.
__device__ __forceinline__ v8i nibbles_to_fp8(i32x4 w) {
  v8i r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    r[2 * c] = (int)((uint32_t)w[c] & 0x0f0f0f0fu);             // u0 u1 u2 u3
    r[2 * c + 1] = (int)(((uint32_t)w[c] >> 4) & 0x0f0f0f0fu);  // u4 u5 u6 u7
  }
  return r;
}
// The same from the row-major stored words (the nibble of k at bits 4 (k mod 8)):
// a mask and a shift give the even elements k0 k2 k4 k6 and the odd ones
// k1 k3 k5 k7, and two byte permutes interleave them into K order.
__device__ __forceinline__ v8i nibbles_rowmajor_to_fp8(i32x4 w) {
  v8i r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t ev = (uint32_t)w[c] & 0x0f0f0f0fu;           // u0 u2 u4 u6
    const uint32_t od = ((uint32_t)w[c] >> 4) & 0x0f0f0f0fu;    // u1 u3 u5 u7
    r[2 * c] = (int)__builtin_amdgcn_perm(od, ev, 0x05010400u);      // u0 u1 u2 u3
    r[2 * c + 1] = (int)__builtin_amdgcn_perm(od, ev, 0x07030602u);  // u4 u5 u6 u7
  }
  return r;
}
// Fused SwiGLU: the gate/up GEMM reads its weight rows interleaved by 16, so
// that two neighbouring 16-column blocks of a tile hold the gate and the up
// rows of the same 16 output columns.  Tile column v reads weight row
//   gate_up_row(v) = (v / 16 odd ? half : 0) + 16 (v / 32) + v % 16,
// half = I (gate rows 0..I-1, up rows I..2I-1), and feeds output column
// 16 (v / 32) + v % 16 of act = silu(gate) * up.
__device__ __forceinline__ int gate_up_row(int v, int half) { return ((v >> 4) & 1) * half + 16 * (v >> 5) + (v & 15); }

__device__ __forceinline__ v8i bias_operand() {
  v8i b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = kBiasWord;
  return b;
}

}  // namespace w4a8
