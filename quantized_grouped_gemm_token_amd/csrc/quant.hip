// Per-row dynamic quantization: the activation quantizer (layer step 1) and
// SwiGLU followed by re-quantization (layer step 5), to FP8 or to INT8.
//
// Per-token FP8 activations, quantized at run time: "GLM-5.3-W4A8" model
// card (gpustack), section 量化方式 and the table of section 与其他 4-bit
// 版本的差异.  Scale = fl32(amax / 448); code = E4M3(fl32(x / scale)).
//
// Rows of up to 2048 16-byte chunks (H <= 16384 bf16, I <= 8192 fp32) take
// one 256-thread workgroup each: every thread loads all of its chunks at
// once and keeps them in registers, so a row costs one memory round trip and
// the codes come from registers.  Longer rows take one wave per row, four
// rows per block, reading the row twice (amax, then codes; the second pass
// hits L2).  Divisions are IEEE fp32 (the library is built with correctly
// rounded fp32 division) so the codes are bit-exact.
#include "common.hpp"
#include "kernels.hpp"
#include "row_quant.hpp"

namespace w4a8 {

// ---- step 1: bf16 activations ------------------------------------------
template <bool kInt8>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                        int64_t H, int64_t ld, uint8_t* __restrict__ q,
                                                        float* __restrict__ s, int32_t* __restrict__ rowsum) {
  using C = RowCodec<kInt8>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * ld);   // 8 bf16 per uint4
  const int64_t chunks = H >> 3;
  float amax = 0.0f;
  for (int64_t c = lane; c < chunks; c += kWave) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  }
  amax = wave_max(amax);
  const float scale = amax > 0.0f ? amax / C::kMax : 1.0f;
  uint2* qr = reinterpret_cast<uint2*>(q + row * H);
  int sum = 0;
  for (int64_t c = lane; c < chunks; c += kWave) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c0 = C::code(bf16_lo(w[i]) / scale, sum);
      const uint32_t c1 = C::code(bf16_hi(w[i]) / scale, sum);
      out[i >> 1] |= (c0 | (c1 << 8)) << (16 * (i & 1));
    }
    qr[c] = make_uint2(out[0], out[1]);
  }
  if constexpr (kInt8) sum = wave_sum_int(sum);
  if (lane == 0) {
    s[row] = scale;
    if constexpr (kInt8) rowsum[row] = sum;
  }
}

// ---- step 5: silu(gate) * up, then the row quantizer -------------------

template <bool kInt8>
__global__ __launch_bounds__(256) void swiglu_quant_kernel(const float* __restrict__ h, int64_t M, int64_t I,
                                                           uint8_t* __restrict__ q, float* __restrict__ s,
                                                           int32_t* __restrict__ rowsum) {
  using C = RowCodec<kInt8>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4* gate = reinterpret_cast<const float4*>(h + row * 2 * I);
  const float4* up = reinterpret_cast<const float4*>(h + row * 2 * I + I);
  const int64_t chunks = I >> 2;
  float amax = 0.0f;
  for (int64_t c = lane; c < chunks; c += kWave) {
    const float4 g = gate[c], u = up[c];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(silu_mul(g.x, u.x)), fabsf(silu_mul(g.y, u.y))),
                             fmaxf(fabsf(silu_mul(g.z, u.z)), fabsf(silu_mul(g.w, u.w)))));
  }
  amax = wave_max(amax);
  const float scale = amax > 0.0f ? amax / C::kMax : 1.0f;
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * I);
  int sum = 0;
  for (int64_t c = lane; c < chunks; c += kWave) {
    const float4 g = gate[c], u = up[c];
    const uint32_t c0 = C::code(silu_mul(g.x, u.x) / scale, sum);
    const uint32_t c1 = C::code(silu_mul(g.y, u.y) / scale, sum);
    const uint32_t c2 = C::code(silu_mul(g.z, u.z) / scale, sum);
    const uint32_t c3 = C::code(silu_mul(g.w, u.w) / scale, sum);
    qr[c] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  }
  if constexpr (kInt8) sum = wave_sum_int(sum);
  if (lane == 0) {
    s[row] = scale;
    if constexpr (kInt8) rowsum[row] = sum;
  }
}

// ---- step 5 after a fused gate/up epilogue -------------------------------
// The fused gate/up GEMM already wrote act = silu(gate) * up (fp32 [M][I])
// and partial row maxima of |act| (pmax [M][I/64]); this is the second half
// of the SwiGLU kernel above: the same scale and codes, from the same values.
template <bool kInt8>
__global__ __launch_bounds__(256) void requant_kernel(const float* __restrict__ act, const float* __restrict__ pmax,
                                                      int64_t M, int64_t I, uint8_t* __restrict__ q,
                                                      float* __restrict__ s, int32_t* __restrict__ rowsum) {
  using C = RowCodec<kInt8>;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int64_t slots = I >> 6;
  float m = 0.0f;
  for (int64_t c = lane; c < slots; c += kWave) m = fmaxf(m, pmax[row * slots + c]);
  m = wave_max(m);
  const f32x4* ar = reinterpret_cast<const f32x4*>(act + row * I);
  const float scale = m > 0.0f ? m / C::kMax : 1.0f;
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * I);
  int sum = 0;
  for (int64_t c = lane; c < (I >> 2); c += kWave) {
    const f32x4 v = __builtin_nontemporal_load(ar + c);
    const uint32_t c0 = C::code(v[0] / scale, sum);
    const uint32_t c1 = C::code(v[1] / scale, sum);
    const uint32_t c2 = C::code(v[2] / scale, sum);
    const uint32_t c3 = C::code(v[3] / scale, sum);
    qr[c] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  }
  if constexpr (kInt8) sum = wave_sum_int(sum);
  if (lane == 0) {
    s[row] = scale;
    if constexpr (kInt8) rowsum[row] = sum;
  }
}

// ---- one row per 256-thread workgroup (row_quant.hpp) -------------------
template <bool kInt8, int kPer>
__global__ __launch_bounds__(kRowThreads) void quant_act_row_kernel(const uint16_t* __restrict__ x, int64_t H,
                                                                    int64_t ld, uint8_t* __restrict__ q,
                                                                    float* __restrict__ s,
                                                                    int32_t* __restrict__ rowsum) {
  quant_act_row<kInt8, kPer>(blockIdx.x, x, H, ld, q, s, rowsum);
}

// step 5 after a fused gate/up epilogue: thread t holds the chunks t, t + 256,
// .. (4 fp32 each) of act row blockIdx.x; the row maximum comes from pmax
template <bool kInt8, int kPer>
__global__ __launch_bounds__(kRowThreads) void requant_row_kernel(const float* __restrict__ act,
                                                                  const float* __restrict__ pmax, int64_t I,
                                                                  uint8_t* __restrict__ q, float* __restrict__ s,
                                                                  int32_t* __restrict__ rowsum) {
  using C = RowCodec<kInt8>;
  __shared__ float red[4];
  __shared__ int reds[4];
  const int64_t row = blockIdx.x;
  const int chunks = (int)(I >> 2), slots = (int)(I >> 6);
  const f32x4* ar = reinterpret_cast<const f32x4*>(act + row * I);
  f32x4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = (int)threadIdx.x + kRowThreads * i;
    if (c < chunks) v[i] = __builtin_nontemporal_load(ar + c);
  }
  float m = 0.0f;
  for (int c = (int)threadIdx.x; c < slots; c += kRowThreads) m = fmaxf(m, pmax[row * slots + c]);
  m = block_max(m, red);
  const float scale = m > 0.0f ? m / C::kMax : 1.0f;
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * I);
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = (int)threadIdx.x + kRowThreads * i;
    if (c < chunks) {
      const uint32_t c0 = C::code(v[i][0] / scale, sum);
      const uint32_t c1 = C::code(v[i][1] / scale, sum);
      const uint32_t c2 = C::code(v[i][2] / scale, sum);
      const uint32_t c3 = C::code(v[i][3] / scale, sum);
      qr[c] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  }
  if constexpr (kInt8) sum = block_sum_int(sum, reds);
  if (threadIdx.x == 0) {
    s[row] = scale;
    if constexpr (kInt8) rowsum[row] = sum;
  }
}

// the row kernel with the fewest chunks per thread that covers `chunks`, or false
template <bool kInt8>
static bool launch_quant_act_row(const uint16_t* x, int64_t T, int64_t H, int64_t ld, uint8_t* q, float* s,
                                 int32_t* rowsum, hipStream_t stream) {
  const int64_t per = ((H >> 3) + kRowThreads - 1) / kRowThreads;
  const dim3 grid((unsigned)T), block(kRowThreads);
  switch (per) {
    case 1: hipLaunchKernelGGL((quant_act_row_kernel<kInt8, 1>), grid, block, 0, stream, x, H, ld, q, s, rowsum); return true;
    case 2: hipLaunchKernelGGL((quant_act_row_kernel<kInt8, 2>), grid, block, 0, stream, x, H, ld, q, s, rowsum); return true;
    case 3: hipLaunchKernelGGL((quant_act_row_kernel<kInt8, 3>), grid, block, 0, stream, x, H, ld, q, s, rowsum); return true;
    case 4: hipLaunchKernelGGL((quant_act_row_kernel<kInt8, 4>), grid, block, 0, stream, x, H, ld, q, s, rowsum); return true;
    case 5: case 6: hipLaunchKernelGGL((quant_act_row_kernel<kInt8, 6>), grid, block, 0, stream, x, H, ld, q, s, rowsum); return true;
    case 7: case 8: hipLaunchKernelGGL((quant_act_row_kernel<kInt8, 8>), grid, block, 0, stream, x, H, ld, q, s, rowsum); return true;
    default: return false;
  }
}

template <bool kInt8>
static bool launch_requant_row(const float* act, const float* pmax, int64_t M, int64_t I, uint8_t* q, float* s,
                               int32_t* rowsum, hipStream_t stream) {
  const int64_t per = ((I >> 2) + kRowThreads - 1) / kRowThreads;
  const dim3 grid((unsigned)M), block(kRowThreads);
  switch (per) {
    case 1: hipLaunchKernelGGL((requant_row_kernel<kInt8, 1>), grid, block, 0, stream, act, pmax, I, q, s, rowsum); return true;
    case 2: hipLaunchKernelGGL((requant_row_kernel<kInt8, 2>), grid, block, 0, stream, act, pmax, I, q, s, rowsum); return true;
    case 3: case 4: hipLaunchKernelGGL((requant_row_kernel<kInt8, 4>), grid, block, 0, stream, act, pmax, I, q, s, rowsum); return true;
    case 5: case 6: case 7: case 8: hipLaunchKernelGGL((requant_row_kernel<kInt8, 8>), grid, block, 0, stream, act, pmax, I, q, s, rowsum); return true;
    default: return false;
  }
}

hipError_t launch_requant(const float* act, const float* pmax, int64_t M, int64_t I, uint8_t* q, float* s,
                          hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (launch_requant_row<false>(act, pmax, M, I, q, s, nullptr, stream)) return hipGetLastError();
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(requant_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, act, pmax, M, I, q, s,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_requant_i8(const float* act, const float* pmax, int64_t M, int64_t I, int8_t* q, float* s,
                             int32_t* rowsum, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (launch_requant_row<true>(act, pmax, M, I, reinterpret_cast<uint8_t*>(q), s, rowsum, stream))
    return hipGetLastError();
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(requant_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, act, pmax, M, I,
                     reinterpret_cast<uint8_t*>(q), s, rowsum);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t H, int64_t ld, uint8_t* q, float* s,
                            hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (launch_quant_act_row<false>(x, T, H, ld, q, s, nullptr, stream)) return hipGetLastError();
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(quant_act_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x, T, H, ld, q, s,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_quant_act_i8(const uint16_t* x, int64_t T, int64_t H, int64_t ld, int8_t* q, float* s,
                               int32_t* rowsum, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (launch_quant_act_row<true>(x, T, H, ld, reinterpret_cast<uint8_t*>(q), s, rowsum, stream))
    return hipGetLastError();
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(quant_act_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x, T, H, ld,
                     reinterpret_cast<uint8_t*>(q), s, rowsum);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* h, int64_t M, int64_t I, uint8_t* q, float* s, hipStream_t stream) {
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(swiglu_quant_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, h, M, I, q, s,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_swiglu_i8(const float* h, int64_t M, int64_t I, int8_t* q, float* s, int32_t* rowsum,
                            hipStream_t stream) {
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(swiglu_quant_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, h, M, I,
                     reinterpret_cast<uint8_t*>(q), s, rowsum);
  return hipGetLastError();
}

}  // namespace w4a8
