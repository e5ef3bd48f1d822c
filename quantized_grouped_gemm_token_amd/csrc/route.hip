// Layer step 2: top-k softmax routing (one wave per token).
//
// 256 routed experts per MoE layer ("从 755GB 到 395GB", Bitdeer AI blog,
// section 我们量化了什么); the router stays BF16 outside this layer
// ("GLM-5.3-W4A8" card, section 量化方式), so the logits are an input.
//
// Each lane keeps up to 16 logits (E <= 1024) in registers.  The k winners
// are picked one at a time by a wave-wide arg-max ordered by (logit desc,
// index asc), which gives the ids in descending order with ties to the lower
// expert.  The weights need only the selected logits when renormalised: the
// full softmax denominator cancels.
#include "common.hpp"
#include "kernels.hpp"

namespace w4a8 {

constexpr int kRouteMaxSlots = 16;      // 16 * 64 = 1024 experts
constexpr int kRouteWaves = 4;

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                         int k, int renormalize, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  extern __shared__ unsigned char route_smem[];
  float* sel_v = reinterpret_cast<float*>(route_smem);                 // [4][k]
  int* sel_i = reinterpret_cast<int*>(route_smem) + kRouteWaves * k;   // [4][k]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kRouteWaves + wave;
  const bool active = t < T;
  float* my_v = sel_v + wave * k;
  int* my_i = sel_i + wave * k;

  float v[kRouteMaxSlots];
  const float* lr = logits + (active ? t : 0) * (int64_t)E;
#pragma unroll
  for (int s = 0; s < kRouteMaxSlots; ++s) {
    const int e = lane + s * kWave;
    v[s] = (active && e < E) ? lr[e] : 0.0f;
  }
  uint32_t taken = 0;   // bit s: slot s already selected
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < kRouteMaxSlots; ++s) {
      const int e = lane + s * kWave;
      const bool ok = e < E && !((taken >> s) & 1u);
      if (ok && (v[s] > bv || (v[s] == bv && e < bi))) {
        bv = v[s];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      my_v[j] = bv;
      my_i[j] = bi;
    }
  }
  __syncthreads();
  const float m = my_v[0];           // the largest logit
  float denom = 0.0f;
  if (renormalize) {
    for (int j = lane; j < k; j += kWave) denom += expf(my_v[j] - m);
  } else {
#pragma unroll
    for (int s = 0; s < kRouteMaxSlots; ++s)
      if (lane + s * kWave < E) denom += expf(v[s] - m);
  }
  denom = wave_sum(denom);
  if (!active) return;
  for (int j = lane; j < k; j += kWave) {
    ids[t * k + j] = my_i[j];
    w[t * k + j] = expf(my_v[j] - m) / denom;
  }
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renormalize, int32_t* ids, float* w,
                        hipStream_t stream) {
  const int64_t blocks = (T + kRouteWaves - 1) / kRouteWaves;
  const size_t smem = (size_t)kRouteWaves * k * (sizeof(float) + sizeof(int));
  hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)blocks), dim3(256), smem, stream, logits, T, E, k,
                     renormalize, ids, w);
  return hipGetLastError();
}

}  // namespace w4a8
