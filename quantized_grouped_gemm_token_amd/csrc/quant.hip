// Per-row dynamic quantization: the activation quantizer (layer step 1) and
// SwiGLU followed by re-quantization (layer step 5), to FP8 or to INT8.
//
// Per-token FP8 activations, quantized at run time: "GLM-5.3-W4A8" model
// card (gpustack), section 量化方式 and the table of section 与其他 4-bit
// 版本的差异.  Scale = fl32(amax / 448); code = E4M3(fl32(x / scale)).
//
// One wave per row, four rows per 256-thread block.  Both kernels read the
// row twice (amax, then codes); the second pass hits L2.  Divisions are IEEE
// fp32 (the library is built with correctly rounded fp32 division) so the
// codes are bit-exact.
#include "common.hpp"
#include "kernels.hpp"

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

hipError_t launch_requant(const float* act, const float* pmax, int64_t M, int64_t I, uint8_t* q, float* s,
                          hipStream_t stream) {
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(requant_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, act, pmax, M, I, q, s,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_requant_i8(const float* act, const float* pmax, int64_t M, int64_t I, int8_t* q, float* s,
                             int32_t* rowsum, hipStream_t stream) {
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(requant_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, act, pmax, M, I,
                     reinterpret_cast<uint8_t*>(q), s, rowsum);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t H, int64_t ld, uint8_t* q, float* s,
                            hipStream_t stream) {
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(quant_act_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x, T, H, ld, q, s,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_quant_act_i8(const uint16_t* x, int64_t T, int64_t H, int64_t ld, int8_t* q, float* s,
                               int32_t* rowsum, hipStream_t stream) {
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
