// Layer step 3: group the routed rows by expert (a stable counting sort).
//
// The pages' engines dispatch tokens to experts across GPUs (expert
// parallelism is required for W4A8: "GLM-5.3-W4A8" card, sections 性能 and
// 部署); inside one GPU that dispatch is this permutation.
//
// Up to 4096 routed indices (decode batches) take one launch that does all
// three steps in one block; more take three launches, all deterministic (no
// order-dependent atomics):
//   1. count   -- one block per 1024 routed indices: per-expert counts of the
//                 block, written to counts[e][b];
//   2. scan    -- one block: exclusive prefix sum over counts in (expert,
//                 block) order with a wavefront-level scan; gives each
//                 (expert, block) its first output row, and the expert
//                 offsets (= the entry of block 0);
//   3. scatter -- one block per 1024 indices again: the stable rank of each
//                 index among the block's earlier indices with the same
//                 expert (ballot-based peer matching inside a wave, per-wave
//                 counts across waves), added to the (expert, block) base.
#include "common.hpp"
#include "kernels.hpp"
#include "permute_small.hpp"

#include <atomic>

namespace w4a8 {

__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(const int32_t* __restrict__ ids, int64_t R,
                                                                      int E, int nblk,
                                                                      int32_t* __restrict__ counts) {
  __shared__ int cnt[kPermMaxE];
  for (int e = threadIdx.x; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kPermBlock;
  for (int i = threadIdx.x; i < kPermBlock; i += kPermThreads) {
    const int64_t f = base + i;
    if (f < R) {
      const int e = ids[f];
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // integer counts: order does not matter
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) counts[(int64_t)e * nblk + blockIdx.x] = cnt[e];
}

// Exclusive scan over n = E * nblk counts (expert-major) in place; offsets[e]
// is the scan value of (e, block 0); offsets[E] = R.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ counts, int64_t n, int E,
                                                             int nblk, int have_counts,
                                                             int32_t* __restrict__ offsets) {
  __shared__ int wave_tot[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t c0 = 0; c0 < n; c0 += 1024) {
    const int64_t i = c0 + tid;
    const int v = (have_counts && i < n) ? counts[i] : 0;
    const int incl = wave_inclusive_scan(v, lane);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      const int wt = lane < 16 ? wave_tot[lane] : 0;
      const int wincl = wave_inclusive_scan(wt, lane);
      if (lane < 16) wave_tot[lane] = wincl - wt;     // exclusive prefix of wave totals
    }
    __syncthreads();
    const int carry = carry_s;
    const int excl = carry + wave_tot[wave] + incl - v;
    if (i < n) {
      counts[i] = excl;
      if (i % nblk == 0) offsets[i / nblk] = excl;
    }
    __syncthreads();
    if (tid == 1023) carry_s = excl + v;
    __syncthreads();
  }
  if (tid == 0) offsets[E] = carry_s;
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(const int32_t* __restrict__ ids, int64_t R,
                                                                        int k, int E, int nblk,
                                                                        const int32_t* __restrict__ bases,
                                                                        int32_t* __restrict__ row_token,
                                                                        int32_t* __restrict__ inv_pos) {
  __shared__ int run[kPermMaxE];                     // next free row of each expert for this block
  __shared__ int wcnt[kPermWaves][kPermMaxE];        // per-wave counts of the current round
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) {
    run[e] = bases[(int64_t)e * nblk + blockIdx.x];
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  permute_scatter_rounds(ids, R, k, E, (int64_t)blockIdx.x * kPermBlock, run, wcnt, row_token, inv_pos);
}

// all three steps in one block when R <= kPermSmallMax (permute_small.hpp)
__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(const int32_t* __restrict__ ids, int64_t R,
                                                                      int k, int E,
                                                                      int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ row_token,
                                                                      int32_t* __restrict__ inv_pos) {
  permute_small(ids, R, k, E, offsets, row_token, inv_pos);
}

int64_t permute_workspace_bytes(int64_t R, int E) {
  const int64_t nblk = (R + kPermBlock - 1) / kPermBlock;
  return (nblk > 0 ? nblk : 1) * (int64_t)E * (int64_t)sizeof(int32_t);
}

// ---- the workspace of w4a8_moe_permute_noalloc, for callers that cannot
// allocate device memory: a buffer the library holds on each GPU until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device buffer: kernels and copies get its device address from
// permute_scratch(), taken once per device with hipGetSymbolAddress.
static __device__ __align__(256) int32_t scratch[kPermScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<int32_t*> g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t permute_scratch(int32_t** ptr) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    p = static_cast<int32_t*>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_permute(const int32_t* ids, int64_t R, int k, int E, int32_t* offsets, int32_t* row_token,
                          int32_t* inv_pos, int32_t* counts, hipStream_t stream) {
  if (R <= kPermSmallMax) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids, R, k, E, offsets,
                       row_token, inv_pos);
    return hipGetLastError();
  }
  const int64_t nblk64 = (R + kPermBlock - 1) / kPermBlock;
  const int nblk = (int)(nblk64 > 0 ? nblk64 : 1);
  if (R > 0)
    hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(kPermThreads), 0, stream, ids, R, E, nblk, counts);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, counts, (int64_t)E * nblk, E, nblk,
                     (int)(R > 0), offsets);
  if (R > 0) {
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(kPermThreads), 0, stream, ids, R, k, E, nblk,
                       counts, row_token, inv_pos);
  }
  return hipGetLastError();
}

}  // namespace w4a8
