// Weight quantizer: the offline step that produces the layer's expert weights.
//
// "GLM-5.3-W4A8" card, section 量化方式: after the FP8 blocks are dequantized
// to float32, every routed-expert weight is quantized to symmetric INT4 with
// group size 128 along K; each group's scale is the one, among 11 shrink
// ratios from 1.00 down to 0.70, whose reconstruction has the smallest squared
// error; the result is packed as uint4b8 nibbles (q + 8) in int32 words.
//
// Per group:  amax = max |w| (1 if the group is all zero);
//             s_r  = fl32(r * amax / 7) for r = 1.00, 0.97, ..., 0.70;
//             q_r  = clamp(round-half-even(w / s_r), -8, 7);
//             keep the r with the smallest sum (w - q_r s_r)^2, the larger r on ties.
// The quotient is rounded as the exact value would be, and the squared
// errors are summed in fp64, so the choice does not depend on fp32 rounding.
//
// One wave per group: lane l holds weights 2l and 2l+1 (one 8-byte load), and
// writes byte l of the group's 64 packed bytes (low nibble k = 2l, high nibble
// k = 2l + 1), which is exactly the int32 word layout (nibble k at bits
// 4 (k mod 8) of word k / 8, little-endian).
#include "common.hpp"
#include "kernels.hpp"

namespace w4a8 {

constexpr int kShrinkCount = 11;
__constant__ double kShrink[kShrinkCount] = {1.00, 0.97, 0.94, 0.91, 0.88, 0.85, 0.82, 0.79, 0.76, 0.73, 0.70};

// round(w / s) to the nearest integer, ties to even, as the exact quotient
// rounds.  The fp32 quotient is within one of that integer; w - (q +- 1/2) s
// is exact in fp64 whenever it is near zero (q +- 1/2 has 5 significant bits
// and s 24, so the product is exact, and w is then within a factor of two of
// it), so its sign decides the neighbouring integer exactly.
__device__ __forceinline__ float rne_quotient(float w, float s) {
  float q = rintf(w / s);
  const double wd = w, sd = s;
  const double above = wd - ((double)q + 0.5) * sd;   // > 0: the quotient exceeds q + 1/2
  if (above > 0.0 || (above == 0.0 && (((int)q) & 1))) return q + 1.0f;
  const double below = wd - ((double)q - 0.5) * sd;   // < 0: the quotient is under q - 1/2
  if (below < 0.0 || (below == 0.0 && (((int)q) & 1))) return q - 1.0f;
  return q;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__global__ __launch_bounds__(256) void wquant_kernel(const float* __restrict__ w, int64_t groups, int G,
                                                     int mse_clip, uint8_t* __restrict__ packed,
                                                     float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  for (int64_t gi = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); gi < groups; gi += waves) {
    // group gi = (row gi / G, group gi % G): its 128 weights are contiguous
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(w + gi * kGroup) + lane);
    float amax = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
    if (amax == 0.0f) amax = 1.0f;
    double best_err = 0.0;
    float best_s = 0.0f;
    const int nr = mse_clip ? kShrinkCount : 1;
    for (int i = 0; i < nr; ++i) {
      const float s = (float)(kShrink[i] * (double)amax / 7.0);
      const float q0 = fminf(fmaxf(rne_quotient(v.x, s), -8.0f), 7.0f);
      const float q1 = fminf(fmaxf(rne_quotient(v.y, s), -8.0f), 7.0f);
      const double e0 = (double)v.x - (double)q0 * (double)s;
      const double e1 = (double)v.y - (double)q1 * (double)s;
      const double err = wave_sum_f64(e0 * e0 + e1 * e1);
      if (i == 0 || err < best_err) {   // wave-uniform: every lane holds the same sum
        best_err = err;
        best_s = s;
      }
    }
    const int u0 = (int)fminf(fmaxf(rne_quotient(v.x, best_s), -8.0f), 7.0f) + 8;
    const int u1 = (int)fminf(fmaxf(rne_quotient(v.y, best_s), -8.0f), 7.0f) + 8;
    packed[gi * (kGroup / 2) + lane] = (uint8_t)(u0 | (u1 << 4));
    if (lane == 0) scales[gi] = best_s;
  }
}

// Per-channel RTN ("GLM-5.3-Channel-INT4-w4a8" card, section 1: RTN, static,
// per channel): one scale per weight row, s = fl32(amax / 7) (1/7 for an
// all-zero row), q = clamp(round-half-even(w / s), -8, 7) from the exact
// quotient.  One 256-thread block per row: the row's amax, then its codes.
__global__ __launch_bounds__(256) void wquant_channel_kernel(const float* __restrict__ w, int64_t rows,
                                                             int64_t K, uint8_t* __restrict__ packed,
                                                             float* __restrict__ scales) {
  __shared__ float part[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const f32x2* wr = reinterpret_cast<const f32x2*>(w + row * K);
    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < K / 2; c += 256) {
      const f32x2 v = wr[c];
      amax = fmaxf(amax, fmaxf(fabsf(v.x), fabsf(v.y)));
    }
    amax = wave_max(amax);
    if (lane == 0) part[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    if (amax == 0.0f) amax = 1.0f;
    const float s = (float)((double)amax / 7.0);
    for (int64_t c = threadIdx.x; c < K / 2; c += 256) {
      const f32x2 v = wr[c];
      const int u0 = (int)fminf(fmaxf(rne_quotient(v.x, s), -8.0f), 7.0f) + 8;
      const int u1 = (int)fminf(fmaxf(rne_quotient(v.y, s), -8.0f), 7.0f) + 8;
      packed[row * (K / 2) + c] = (uint8_t)(u0 | (u1 << 4));
    }
    if (threadIdx.x == 0) scales[row] = s;
    __syncthreads();   // part[] is reused by the next row
  }
}

// MXFP4 (Open Compute Project microscaling format), the 4-bit alternative the
// "GLM-5.3-W4A8" card compares against in section 量化方式 (groups of 32):
// E2M1 elements with one E8M0 scale per 32 consecutive weights along K.
// Per block:  amax = max |w| (1 if the block is all zero);
//             X = floor(log2 amax) - 2 (2 = the exponent of E2M1's top
//             binade), clamped to [-127, 127]; scale byte X + 127;
//             code = E2M1 of w * 2^-X: nearest of 0, .5, 1, 1.5, 2, 3, 4, 6,
//             ties to the code with mantissa bit 0, saturating at 6, with the
//             sign bit of w (so -0 and tiny negatives keep it).
// w * 2^-X is exact (a power-of-two scaling; a result too small to stay
// normal lies far below the first rounding threshold, 0.25).
// Eight lanes per block: each holds 4 consecutive weights (one 16-byte load)
// and writes their 2 packed bytes (element k in the low nibble of byte k / 2
// when k is even); the block's max comes from DPP moves inside the 8 lanes.
__device__ __forceinline__ uint32_t e2m1_code(float w, float x) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(w) >> 28) & 8u);
}

__global__ __launch_bounds__(256) void wquant_mxfp4_kernel(const float* __restrict__ w, int64_t pieces,
                                                           uint16_t* __restrict__ packed,
                                                           uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;   // a multiple of 8: a block's lanes move together
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < pieces; t += stride) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(w) + t);
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xf, 0xf, true)));    // quad [1,0,3,2]
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xf, 0xf, true)));    // quad [2,3,0,1]
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xf, 0xf, true)));   // half-row mirror
    if (m == 0.0f) m = 1.0f;
    int e;
    (void)frexpf(m, &e);                                    // m = f 2^e, f in [0.5, 1): floor(log2 m) = e - 1
    const int X = min(max(e - 3, -127), 127);
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = e2m1_code(v[i], ldexpf(v[i], -X));
    packed[t] = (uint16_t)(c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12));
    if ((t & 7) == 0) scales[t >> 3] = (uint8_t)(X + 127);
  }
}

hipError_t launch_wquant_mxfp4(const float* w, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales,
                               hipStream_t stream) {
  const int64_t pieces = rows * K / 4;
  if (pieces == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 8192);
  hipLaunchKernelGGL(wquant_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, pieces,
                     reinterpret_cast<uint16_t*>(packed), scales);
  return hipGetLastError();
}

// 4-bit weights into the layout the grouped GEMMs read (a pure permutation of
// bytes; INT4 words and MXFP4 bytes alike hold 64 bytes per row and 128-wide
// K group).  Per expert e (G = K/128 groups):
//   w: the 64 packed bytes of K group g of rows 16b .. 16b+15 become one 1 KB
//      piece at ((e (N/16) + b) G + g) 1024 + 64 (row % 16), so that one
//      16-row x 128-K operand block is a single contiguous load;
//   s: the 4 scale bytes of row n and group g (one fp32 group scale, or four
//      E8M0 block scales) move to ((e G + g) N + n) 4, so that the scales of
//      one group of all rows are contiguous (skipped when s is null).
// One thread per 16 weight bytes and one per 4 scale bytes.
// INT4 words in the GEMM storage hold their eight nibbles k0..k7 in the order
// k0 k4 k1 k5 k2 k6 k3 k7 (bits 0..31), so that w & 0x0f0f0f0f holds k0..k3
// and (w >> 4) & 0x0f0f0f0f holds k4..k7, one per byte
__device__ __forceinline__ uint32_t nibble_split(uint32_t w) {
  auto spread = [](uint32_t x) {      // nibble i of a 16-bit value -> nibble 2i
    x = (x | (x << 8)) & 0x00ff00ffu;
    return (x | (x << 4)) & 0x0f0f0f0fu;
  };
  return spread(w & 0xffffu) | (spread(w >> 16) << 4);
}

template <bool kSplit>
__global__ __launch_bounds__(256) void prepack_kernel(const u32x4* __restrict__ w, const uint32_t* __restrict__ s,
                                                      int64_t E, int64_t N, int64_t G, u32x4* __restrict__ wb,
                                                      uint32_t* __restrict__ sb) {
  const int64_t nw = E * N * G * 4, ns = s ? E * N * G : 0;   // 16-byte pieces, 4-byte scale words
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nw + ns; t += stride) {
    if (t < nw) {
      // source piece t: row r = t / (4G) of all E N rows, group g, chunk c
      const int64_t r = t / (4 * G), rem = t - r * 4 * G, g = rem >> 2, c = rem & 3;
      const int64_t e = r / N, n = r - e * N;
      u32x4 v = __builtin_nontemporal_load(w + t);
      if constexpr (kSplit) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = nibble_split(v[i]);
      }
      wb[(((e * (N / 16) + n / 16) * G + g) * 16 + n % 16) * 4 + c] = v;
    } else {
      const int64_t u = t - nw, r = u / G, g = u - r * G, e = r / N, n = r - e * N;
      sb[(e * G + g) * N + n] = s[u];
    }
  }
}

hipError_t launch_prepack(const void* w, const void* s, int64_t E, int64_t N, int64_t K, int nibble_split,
                          void* wb, void* sb, hipStream_t stream) {
  const int64_t G = K / 128, total = E * N * G * (s ? 5 : 4);
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 16384);
  auto kernel = nibble_split ? prepack_kernel<true> : prepack_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(w),
                     reinterpret_cast<const uint32_t*>(s), E, N, G, reinterpret_cast<u32x4*>(wb),
                     reinterpret_cast<uint32_t*>(sb));
  return hipGetLastError();
}

hipError_t launch_wquant_channel(const float* w, int64_t rows, int64_t K, int32_t* packed, float* scales,
                                 hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(rows, 65536);
  hipLaunchKernelGGL(wquant_channel_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, rows, K,
                     reinterpret_cast<uint8_t*>(packed), scales);
  return hipGetLastError();
}

hipError_t launch_wquant(const float* w, int64_t rows, int64_t K, int mse_clip, int32_t* packed, float* scales,
                         hipStream_t stream) {
  const int G = (int)(K / kGroup);
  const int64_t groups = rows * G;
  if (groups == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((groups + 3) / 4, 65536);
  hipLaunchKernelGGL(wquant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, groups, G, mse_clip,
                     reinterpret_cast<uint8_t*>(packed), scales);
  return hipGetLastError();
}

}  // namespace w4a8
