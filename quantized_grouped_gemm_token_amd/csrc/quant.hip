// Per-row dynamic FP8 quantization: the activation quantizer (layer step 1)
// and SwiGLU followed by re-quantization (layer step 5).
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

// ---- step 1: bf16 activations ------------------------------------------
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                        int64_t H, int64_t ld, uint8_t* __restrict__ q,
                                                        float* __restrict__ s) {
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
  const float scale = amax > 0.0f ? amax / kFp8Max : 1.0f;
  uint2* qr = reinterpret_cast<uint2*>(q + row * H);
  for (int64_t c = lane; c < chunks; c += kWave) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c0 = e4m3_encode(bf16_lo(w[i]) / scale);
      const uint32_t c1 = e4m3_encode(bf16_hi(w[i]) / scale);
      out[i >> 1] |= (c0 | (c1 << 8)) << (16 * (i & 1));
    }
    qr[c] = make_uint2(out[0], out[1]);
  }
  if (lane == 0) s[row] = scale;
}

// ---- step 5: silu(gate) * up, then per-row FP8 -------------------------
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__global__ __launch_bounds__(256) void swiglu_quant_kernel(const float* __restrict__ h, int64_t M, int64_t I,
                                                           uint8_t* __restrict__ q, float* __restrict__ s) {
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
  const float scale = amax > 0.0f ? amax / kFp8Max : 1.0f;
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * I);
  for (int64_t c = lane; c < chunks; c += kWave) {
    const float4 g = gate[c], u = up[c];
    const uint32_t c0 = e4m3_encode(silu_mul(g.x, u.x) / scale);
    const uint32_t c1 = e4m3_encode(silu_mul(g.y, u.y) / scale);
    const uint32_t c2 = e4m3_encode(silu_mul(g.z, u.z) / scale);
    const uint32_t c3 = e4m3_encode(silu_mul(g.w, u.w) / scale);
    qr[c] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
  }
  if (lane == 0) s[row] = scale;
}

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t H, int64_t ld, uint8_t* q, float* s,
                            hipStream_t stream) {
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, T, H, ld, q, s);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* h, int64_t M, int64_t I, uint8_t* q, float* s, hipStream_t stream) {
  const int64_t blocks = (M + 3) / 4;
  hipLaunchKernelGGL(swiglu_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, h, M, I, q, s);
  return hipGetLastError();
}

}  // namespace w4a8
