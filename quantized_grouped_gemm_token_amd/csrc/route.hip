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
#include "route_topk.hpp"

namespace w4a8 {

// S logit slots per lane (E <= 64 S), four tokens per workgroup (route_topk.hpp)
template <int S>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                         int k, int renormalize, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  extern __shared__ unsigned char route_smem[];
  route_block<S>(blockIdx.x, logits, T, E, k, renormalize, ids, w, route_smem);
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
