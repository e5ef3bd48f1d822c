// Layer step 2: top-k softmax routing (one wave per token).
//
// 256 routed experts per MoE layer ("从 755GB 到 395GB", Bitdeer AI blog,
// section 我们量化了什么); the router stays BF16 outside this layer
// ("GLM-5.3-W4A8" card, section 量化方式), so the logits are an input.
//
// Each lane keeps up to 16 logits (E <= 1024) in registers (as many slots as
// E needs).  The k winners are picked one at a time by a wave-wide arg-max
// ordered by (logit desc, index asc), which gives the ids in descending order
// with ties to the lower expert.  The arg-max runs on DPP row rotations and
// four lane reads, without LDS round trips.  The weights need only the selected logits when renormalised: the
// full softmax denominator cancels.
#include "common.hpp"
#include "kernels.hpp"

namespace w4a8 {

constexpr int kRouteMaxSlots = 16;      // 16 * 64 = 1024 experts
constexpr int kRouteWaves = 4;

// (value, index) order of the selection: a larger logit first, equal logits by the lower expert
__device__ __forceinline__ bool route_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// one step of the row reduction: the pair of the lane `kCtl` (a DPP row rotation) away
template <int kCtl>
__device__ __forceinline__ void route_row_step(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), kCtl, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_mov_dpp(bi, kCtl, 0xf, 0xf, false);
  if (route_better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

// the best (value, index) pair of the wave, in every lane: DPP rotations within
// each row of 16 lanes, then the four row leaders read as uniform values
__device__ __forceinline__ void route_wave_best(float& bv, int& bi) {
  route_row_step<0x128>(bv, bi);   // row_ror:8
  route_row_step<0x124>(bv, bi);   // row_ror:4
  route_row_step<0x122>(bv, bi);   // row_ror:2
  route_row_step<0x121>(bv, bi);   // row_ror:1
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), r));
    const int ri = __builtin_amdgcn_readlane(bi, r);
    if (route_better(rv, ri, v, i)) {
      v = rv;
      i = ri;
    }
  }
  bv = v;
  bi = i;
}

// S logit slots per lane (E <= 64 S): slot s of lane l is expert l + 64 s
template <int S>
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

  float v[S];
  const float* lr = logits + (active ? t : 0) * (int64_t)E;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = lane + s * kWave;
    v[s] = (active && e < E) ? lr[e] : 0.0f;
  }
  uint32_t taken = 0;   // bit s: slot s already selected
  for (int j = 0; j < k; ++j) {
    // the lane's best untaken slot: slots ascend in expert index, so a strict
    // comparison keeps the lower index among equal logits
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int e = lane + s * kWave;
      if (e < E && !((taken >> s) & 1u) && v[s] > bv) {
        bv = v[s];
        bi = e;
      }
    }
    route_wave_best(bv, bi);
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
    for (int s = 0; s < S; ++s)
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
  const dim3 grid((unsigned)blocks), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, smem, stream, logits, T, E, k, renormalize, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, smem, stream, logits, T, E, k, renormalize, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, smem, stream, logits, T, E, k, renormalize, ids, w);
  else if (E <= 512)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, smem, stream, logits, T, E, k, renormalize, ids, w);
  else
    hipLaunchKernelGGL(route_topk_kernel<kRouteMaxSlots>, grid, block, smem, stream, logits, T, E, k,
                       renormalize, ids, w);
  return hipGetLastError();
}

}  // namespace w4a8
