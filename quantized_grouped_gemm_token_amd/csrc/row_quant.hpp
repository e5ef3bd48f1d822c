// Per-row activation quantizer of layer step 1, as device code shared by the
// quantizer kernels and the fused front of the layer (front.hip).
#pragma once

#include "common.hpp"

namespace w4a8 {

// Row quantizers of the two activation formats.
//  * FP8 (the group-128 variant): scale = fl32(amax / 448), code = E4M3(fl32(x / scale)).
//  * INT8 (the per-channel variant, "GLM-5.3-Channel-INT4-w4a8" card, section 1:
//    dynamic per-token INT8): scale = fl32(amax / 127), code =
//    clamp(round-half-even(fl32(x / scale)), -127, 127); the kernels also
//    write the sum of each row's codes, which the integer GEMM needs to undo
//    the +8 offset of the stored weight nibbles.
template <bool kInt8>
struct RowCodec {
  static constexpr float kMax = kInt8 ? 127.0f : kFp8Max;
  // the byte of v = x / scale; adds the integer code to sum
  __device__ static __forceinline__ uint32_t code(float v, int& sum) {
    if constexpr (kInt8) {
      const int c = (int)fminf(fmaxf(rintf(v), -127.0f), 127.0f);
      sum += c;
      return (uint32_t)c & 0xFFu;
    } else {
      return e4m3_encode(v);
    }
  }
};

// ---- one row per 256-thread workgroup ------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowMaxChunks = 8;          // 16-byte chunks per thread

// max over the workgroup (v >= 0 in every thread); red holds 4 floats
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// sum over the workgroup, valid in thread 0; red holds 4 ints (not the ones block_max used)
__device__ __forceinline__ int block_sum_int(int v, int* red) {
  v = wave_sum_int(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// step 1 for one row, by a 256-thread workgroup: thread t holds the chunks
// t, t + 256, .. (8 bf16 each) of the row
template <bool kInt8, int kPer>
__device__ __forceinline__ void quant_act_row(int64_t row, const uint16_t* __restrict__ x, int64_t H, int64_t ld,
                                              uint8_t* __restrict__ q, float* __restrict__ s,
                                              int32_t* __restrict__ rowsum) {
  using C = RowCodec<kInt8>;
  __shared__ float red[4];
  __shared__ int reds[4];
  const int chunks = (int)(H >> 3);
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * ld);
  uint4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = (int)threadIdx.x + kRowThreads * i;
    v[i] = c < chunks ? xr[c] : make_uint4(0u, 0u, 0u, 0u);   // zeros count nothing in the max
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
  }
  amax = block_max(amax, red);
  const float scale = amax > 0.0f ? amax / C::kMax : 1.0f;
  uint2* qr = reinterpret_cast<uint2*>(q + row * H);
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = (int)threadIdx.x + kRowThreads * i;
    if (c < chunks) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t out[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t c0 = C::code(bf16_lo(w[j]) / scale, sum);
        const uint32_t c1 = C::code(bf16_hi(w[j]) / scale, sum);
        out[j >> 1] |= (c0 | (c1 << 8)) << (16 * (j & 1));
      }
      qr[c] = make_uint2(out[0], out[1]);
    }
  }
  if constexpr (kInt8) sum = block_sum_int(sum, reds);
  if (threadIdx.x == 0) {
    s[row] = scale;
    if constexpr (kInt8) rowsum[row] = sum;
  }
}

}  // namespace w4a8
