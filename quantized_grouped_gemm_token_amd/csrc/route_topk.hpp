// Top-k softmax routing of layer step 2 (one wave per token), as device code
// shared by the routing kernel and the fused front of the layer.
#pragma once

#include "common.hpp"

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

// the tokens 4 block .. 4 block + 3 of a 256-thread workgroup, one per wave,
// with S logit slots per lane (E <= 64 S): slot s of lane l is expert l + 64 s.
// route_smem: 8 k words per wave
template <int S>
__device__ __forceinline__ void route_block(int64_t block, const float* __restrict__ logits, int64_t T, int E, int k,
                                            int renormalize, int32_t* __restrict__ ids, float* __restrict__ w,
                                            unsigned char* route_smem) {
  float* sel_v = reinterpret_cast<float*>(route_smem);                 // [4][k]
  int* sel_i = reinterpret_cast<int*>(route_smem) + kRouteWaves * k;   // [4][k]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = block * kRouteWaves + wave;
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

}  // namespace w4a8
