// Grouped W4A8 GEMM, weight-streaming form: for few rows per expert (decode).
//
// With a handful of tokens per expert the GEMM is bound by reading the INT4
// weights from HBM once.  Each wave owns NSUB x 16 weight rows (output
// columns) of one expert and streams them along K with 16-byte loads: lane l
// reads the 16 bytes (32 nibbles) of column l % 16 for the K quarter l / 16
// of each 128-wide group, which is exactly its B operand of the
// 16x16x128 FP8 MFMA -- no LDS, no shuffles.  The expert's rows (A, FP8
// codes, gathered through a_rows) come from L2 in 16-row tiles.
//
// Grid: (ceil(N / (64 * NSUB)), E); 256 threads = 4 waves side by side in N.
// An expert with no rows returns at once; one with more than 16 * MSUB rows
// loops over M blocks, re-streaming its weights (the tiled kernel is the one
// for many rows per expert).
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace w4a8 {

template <int NSUB, int MSUB, int U>
struct StreamStage {
  i32x4 wb[U][NSUB];
  float sc[U][NSUB];
  v8i av[U][MSUB];
};

template <int NSUB, int MSUB, int U>
__device__ __forceinline__ void stream_load(StreamStage<NSUB, MSUB, U>& st, const int32_t* const (&wrow)[NSUB],
                                            const float* const (&srow)[NSUB],
                                            const uint8_t* const (&arow)[MSUB], int g0) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int g = g0 + u;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      st.wb[u][s] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wrow[s] + g * 16));
      st.sc[u][s] = srow[s][g];
    }
#pragma unroll
    for (int t = 0; t < MSUB; ++t) st.av[u][t] = *reinterpret_cast<const v8i*>(arow[t] + g * kGroup);
  }
}

template <int NSUB, int MSUB, int U>
__device__ __forceinline__ void stream_compute(const StreamStage<NSUB, MSUB, U>& st, v4f (&acc)[MSUB][NSUB]) {
  const v8i kb = bias_operand();
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    v4f bias[MSUB];
#pragma unroll
    for (int t = 0; t < MSUB; ++t) bias[t] = mfma16x16x128(st.av[u][t], kb, zero);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const v8i b = nibbles_to_fp8(st.wb[u][s]);
#pragma unroll
      for (int t = 0; t < MSUB; ++t) {
        const v4f d = mfma16x16x128(st.av[u][t], b, bias[t]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][s][r] = fmaf(st.sc[u][s], d[r], acc[t][s][r]);
      }
    }
  }
}

template <int NSUB, int MSUB, int U>
__global__ __launch_bounds__(256) void gg_stream_kernel(const uint8_t* __restrict__ a,
                                                        const float* __restrict__ a_scale,
                                                        const int32_t* __restrict__ a_rows,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ w_packed,
                                                        const float* __restrict__ w_scale, int64_t N, int64_t K,
                                                        float* __restrict__ out) {
  const int e = blockIdx.y;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  if (r1 <= r0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int64_t n_base = ((int64_t)blockIdx.x * 4 + wave) * (16 * NSUB);
  if (n_base >= N) return;
  const int G = (int)(K >> 7);
  const int64_t kw = K >> 3;   // int32 words per weight row

  const int32_t* wrow[NSUB];
  const float* srow[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int64_t n = n_base + s * 16 + col;
    wrow[s] = w_packed + ((int64_t)e * N + n) * kw + kq * 4;
    srow[s] = w_scale + ((int64_t)e * N + n) * G;
  }

  for (int m0 = r0; m0 < r1; m0 += 16 * MSUB) {
    const uint8_t* arow[MSUB];
#pragma unroll
    for (int t = 0; t < MSUB; ++t) {
      const int p = min(m0 + t * 16 + col, r1 - 1);   // rows past the end repeat the last one (not stored)
      const int64_t src = a_rows ? a_rows[p] : p;
      arow[t] = a + src * K + kq * 32;
    }
    v4f acc[MSUB][NSUB];
#pragma unroll
    for (int t = 0; t < MSUB; ++t)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[t][s] = v4f{0.f, 0.f, 0.f, 0.f};

    int g0 = 0;
    for (; g0 + U <= G; g0 += U) {
      StreamStage<NSUB, MSUB, U> st;
      stream_load(st, wrow, srow, arow, g0);
      stream_compute(st, acc);
    }
    for (; g0 < G; ++g0) {
      StreamStage<NSUB, MSUB, 1> st;
      stream_load(st, wrow, srow, arow, g0);
      stream_compute(st, acc);
    }

#pragma unroll
    for (int t = 0; t < MSUB; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = m0 + t * 16 + kq * 4 + r;
        if (p < r1) {
          const int64_t src = a_rows ? a_rows[p] : p;
          const float rs = a_scale[src] * kUnitScale;
#pragma unroll
          for (int s = 0; s < NSUB; ++s) out[(int64_t)p * N + n_base + s * 16 + col] = acc[t][s][r] * rs;
        }
      }
    }
  }
}

hipError_t launch_gg_stream(const GemmArgs& g, hipStream_t stream) {
  constexpr int NSUB = 2, U = 4;
  const dim3 block(256);
  const dim3 grid((unsigned)((g.N + 64 * NSUB - 1) / (64 * NSUB)), (unsigned)g.E);
  if (g.M_total <= 4 * g.E)
    hipLaunchKernelGGL((gg_stream_kernel<NSUB, 1, U>), grid, block, 0, stream, g.a, g.a_scale, g.a_rows,
                       g.offsets, g.w_packed, g.w_scale, g.N, g.K, g.out);
  else
    hipLaunchKernelGGL((gg_stream_kernel<NSUB, 4, U>), grid, block, 0, stream, g.a, g.a_scale, g.a_rows,
                       g.offsets, g.w_packed, g.w_scale, g.N, g.K, g.out);
  return hipGetLastError();
}

}  // namespace w4a8
