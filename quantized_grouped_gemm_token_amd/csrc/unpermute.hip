// Layer step 7: routing-weighted combine of each token's k expert outputs.
//
// y[t, :] = sum_j w[t, j] * o[inv_pos[t*k + j], :], fp32, j ascending (a
// fixed order, so the result is deterministic).  A routed index that was
// not routed (inv_pos < 0) contributes nothing.
//
// Grid: (T tokens, H / 1024 column chunks); each thread owns 4 columns.
#include "common.hpp"
#include "kernels.hpp"

namespace w4a8 {

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void unpermute_kernel(const float* __restrict__ o,
                                                        const int32_t* __restrict__ inv_pos,
                                                        const float* __restrict__ w, int k, int64_t H,
                                                        void* __restrict__ y) {
  const int64_t t = blockIdx.x;
  const int64_t col = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  if (col >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // eight expert rows at a time: all their loads in flight (an unrouted or
  // missing row loads row 0 and is skipped), then the sums in j order
  constexpr int kU = 8;
  for (int j0 = 0; j0 < k; j0 += kU) {
    int p[kU];
    f32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) p[u] = j0 + u < k ? inv_pos[t * k + j0 + u] : -1;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o + (int64_t)max(p[u], 0) * H + col));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (p[u] < 0) continue;
      const float wj = w[t * k + j0 + u];
      acc.x = fmaf(wj, v[u][0], acc.x);
      acc.y = fmaf(wj, v[u][1], acc.y);
      acc.z = fmaf(wj, v[u][2], acc.z);
      acc.w = fmaf(wj, v[u][3], acc.w);
    }
  }
  if (BF16_OUT) {
    const uint32_t lo = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
    const uint32_t hi = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + t * H + col) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + t * H + col) = acc;
  }
}

// The routing-weighted scatter in the down GEMM's epilogue (the token-major
// form of step 7): for each routed index f = t k + j with inv_pos[f] = p, the
// GEMM stores its row p as row f (row_src[p] = f), scaled by a_scale[p] w[f]
// (row_scale[p], which it takes in place of its token scales); then
// combine_kernel sums each token's k rows, contiguous in memory, in j order.
__global__ __launch_bounds__(256) void row_sources_kernel(const int32_t* __restrict__ inv_pos,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ a_scale, int64_t R,
                                                          int64_t M_total, int32_t* __restrict__ row_src,
                                                          float* __restrict__ row_scale) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= R) return;
  const int32_t p = inv_pos[f];
  if (p < 0 || p >= M_total) return;          // not routed (an id out of range)
  row_src[p] = (int32_t)f;
  row_scale[p] = a_scale[p] * w[f];
}

// y[t, :] = sum over the routed j (inv_pos[t k + j] >= 0), j ascending, of
// o_tok[t k + j, :]: fp32 adds, the first one onto 0.  Grid as unpermute_kernel.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_tok,
                                                      const int32_t* __restrict__ inv_pos, int k, int64_t H,
                                                      void* __restrict__ y) {
  const int64_t t = blockIdx.x;
  const int64_t col = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  if (col >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int kU = 8;
  for (int j0 = 0; j0 < k; j0 += kU) {
    bool use[kU];
    f32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) use[u] = j0 + u < k && inv_pos[t * k + j0 + u] >= 0;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      v[u] = use[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o_tok + (t * k + j0 + u) * H + col))
                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (!use[u]) continue;
      acc.x += v[u][0];
      acc.y += v[u][1];
      acc.z += v[u][2];
      acc.w += v[u][3];
    }
  }
  if (BF16_OUT) {
    const uint32_t lo = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
    const uint32_t hi = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + t * H + col) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + t * H + col) = acc;
  }
}

hipError_t launch_row_sources(const int32_t* inv_pos, const float* w, const float* a_scale, int64_t R,
                              int64_t M_total, int32_t* row_src, float* row_scale, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(row_sources_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, stream, inv_pos, w,
                     a_scale, R, M_total, row_src, row_scale);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o_tok, const int32_t* inv_pos, int64_t T, int k, int64_t H, void* y,
                          int bf16_out, hipStream_t stream) {
  const dim3 grid((unsigned)T, (unsigned)((H + 1023) / 1024));
  if (bf16_out)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream, o_tok, inv_pos, k, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream, o_tok, inv_pos, k, H, y);
  return hipGetLastError();
}

hipError_t launch_unpermute(const float* o, const int32_t* inv_pos, const float* w, int64_t T, int k, int64_t H,
                            void* y, int bf16_out, hipStream_t stream) {
  const dim3 grid((unsigned)T, (unsigned)((H + 1023) / 1024));
  if (bf16_out)
    hipLaunchKernelGGL(unpermute_kernel<true>, grid, dim3(256), 0, stream, o, inv_pos, w, k, H, y);
  else
    hipLaunchKernelGGL(unpermute_kernel<false>, grid, dim3(256), 0, stream, o, inv_pos, w, k, H, y);
  return hipGetLastError();
}

}  // namespace w4a8
