// Layer steps 1, 2 and 3 in one launch, for decode batches (T k <= 4096 routed
// rows, H <= 8192).
//
// Steps 1 and 2 share no data, so one grid holds both: workgroups 0 .. T-1
// quantize one activation row each (row_quant.hpp), the next ceil(T/4) route
// four tokens each (route_topk.hpp).  Step 3 needs every routed id: each
// routing workgroup, once its ids are written, makes them visible to the
// device and counts itself on a device counter; the one that arrives last
// sorts the routed rows (the one-block form of permute_small.hpp) and puts
// the counter back to zero for the next call.  Nothing waits on the
// counter, so no workgroup can stall on another.  The results are those of
// the three separate kernels, which share this device code.
#include "common.hpp"
#include "kernels.hpp"
#include "permute_small.hpp"
#include "route_topk.hpp"
#include "row_quant.hpp"

#include <type_traits>

namespace w4a8 {

template <bool kInt8, int kPer, int S>
__global__ __launch_bounds__(256) void front_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t H, int64_t ld,
                                                    uint8_t* __restrict__ q, float* __restrict__ s,
                                                    int32_t* __restrict__ rowsum, const float* __restrict__ logits,
                                                    int E, int k, int renormalize, int32_t* __restrict__ ids,
                                                    float* __restrict__ w, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ row_token, int32_t* __restrict__ inv_pos,
                                                    uint32_t* __restrict__ counter, int route_blocks) {
  if ((int64_t)blockIdx.x < T) {
    quant_act_row<kInt8, kPer>(blockIdx.x, x, H, ld, q, s, rowsum);
    return;
  }
  extern __shared__ unsigned char front_smem[];
  route_block<S>((int64_t)blockIdx.x - T, logits, T, E, k, renormalize, ids, w, front_smem);
  __shared__ uint32_t arrived;
  __threadfence();                        // this workgroup's ids and weights are visible to the device
  __syncthreads();
  if (threadIdx.x == 0) arrived = atomicAdd(counter, 1u);
  __syncthreads();
  if (arrived != (uint32_t)(route_blocks - 1)) return;
  __threadfence();                        // the last one: every workgroup's ids are visible here
  permute_small(ids, T * k, k, E, offsets, row_token, inv_pos);
  if (threadIdx.x == 0) *counter = 0u;
}

template <bool kInt8, int kPer, int S>
static void launch_front_variant(const FrontArgs& f, hipStream_t stream) {
  const int route_blocks = (int)((f.T + kRouteWaves - 1) / kRouteWaves);
  const size_t smem = (size_t)kRouteWaves * f.k * (sizeof(float) + sizeof(int));
  hipLaunchKernelGGL((front_kernel<kInt8, kPer, S>), dim3((unsigned)(f.T + route_blocks)), dim3(256), smem, stream,
                     f.x, f.T, f.H, f.ld, f.q, f.s, f.rowsum, f.logits, f.E, f.k, f.renormalize, f.ids, f.w,
                     f.offsets, f.row_token, f.inv_pos, f.counter, route_blocks);
}

template <bool kInt8, int kPer>
static void launch_front_slots(const FrontArgs& f, hipStream_t stream) {
  if (f.E <= 64) launch_front_variant<kInt8, kPer, 1>(f, stream);
  else if (f.E <= 128) launch_front_variant<kInt8, kPer, 2>(f, stream);
  else if (f.E <= 256) launch_front_variant<kInt8, kPer, 4>(f, stream);
  else if (f.E <= 512) launch_front_variant<kInt8, kPer, 8>(f, stream);
  else launch_front_variant<kInt8, kPer, kRouteMaxSlots>(f, stream);
}

bool front_fits(int64_t T, int64_t H, int k) {
  return T >= 1 && T * k <= kPermSmallMax && ((H >> 3) + kRowThreads - 1) / kRowThreads <= 4;
}

hipError_t launch_front(const FrontArgs& f, bool int8, hipStream_t stream) {
  const int64_t per = ((f.H >> 3) + kRowThreads - 1) / kRowThreads;
  auto go = [&](auto I8) {
    constexpr bool kI8 = decltype(I8)::value;
    if (per <= 1) launch_front_slots<kI8, 1>(f, stream);
    else if (per == 2) launch_front_slots<kI8, 2>(f, stream);
    else if (per == 3) launch_front_slots<kI8, 3>(f, stream);
    else launch_front_slots<kI8, 4>(f, stream);
  };
  if (int8) go(std::true_type{});
  else go(std::false_type{});
  return hipGetLastError();
}

}  // namespace w4a8
