// Grouped W4A8 GEMM, weight-streaming form: for few rows per expert (decode).
//
// With a handful of tokens per expert the GEMM is bound by reading the 4-bit
// weights from HBM once, so the kernel is built around the load pattern HBM
// serves best.  The weights come in the GEMM storage, where the 64 packed
// bytes of one 128-wide K group of 16 rows are one contiguous 1 KB piece: one
// 16-byte load per lane and group reads a whole piece (lane = col + 16 kq
// takes row col, bytes 16 kq .. +15, i.e. K elements 32 kq .. +31), and that
// is exactly the lane's MFMA B operand (INT4: after splitting the nibbles
// into bytes; MXFP4: as it is).  A wave owns NS subtiles of 16 weight rows
// (output columns) of one expert and walks K two groups at a time, so each
// subtile streams 2 KB per step.
//
// The 4 waves of a workgroup share the expert's activation rows (FP8 codes,
// up to 16 rows per M block, gathered through a_rows): they are staged in
// LDS once per chunk of CH group pairs, directly in MFMA operand order, double
// buffered, with one barrier per chunk.  Per-group scales are group-major: a
// lane reads the word of its row for each group.
//
// MXFP4 weights (group 32): the group's word of E8M0 block scales is shifted
// so that the lane's quarter is byte 0, and the matrix core applies it: the
// products accumulate straight into acc.  The activations are staged in the
// K order the FP4 form of the instruction reads (16-byte chunks q and q + 4
// for lane group q).
//
// Grid: (ceil(N / (64 NS)), E); 256 threads = 4 waves side by side in N.  An
// expert with no rows returns at once; one with more than 16 rows loops over
// M blocks, re-streaming its weights (the tiled kernel is the one for many
// rows per expert).
//
// The same kernel reads the weights in the row-major stored format too (the
// grouped GEMM calls without "_prepacked"): the lane's operand of a group is
// then 16 bytes of its own row, so a wave's load covers 64 bytes of 16 rows.
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace w4a8 {

constexpr int kStreamThreads = 256;

// LDS image of the activation tile of one chunk: for each group h of the
// chunk and MFMA lane L, the 32 bytes lane L feeds to the MFMA (row L % 16,
// K bytes 32 (L / 16) .. +31 of group h; MX form: K bytes 16 (L / 16) .. +15
// and 64 + 16 (L / 16) .. +15).
template <int CH>
struct StreamSmem {
  uint8_t a[2][2 * CH][64][32];
  float rmax[4][16];                 // fused form: row max |act| of each wave's 16 output columns
};

// Chunk of activations -> registers: thread t loads rows t / 16 (16 B chunks
// t % 16, +16, +32, ... of the chunk's 256*CH bytes per row).
template <int CH>
struct AChunk {
  static constexpr int kPerThread = (16 * 256 * CH) / (16 * kStreamThreads);   // 16-byte pieces per thread
  i32x4 v[kPerThread];
};

// A thread whose row is past the expert's last one stages zeros instead: the
// products of such a row are never stored, and each output row depends only
// on its own activation row, so its bytes need not be read.
template <int CH>
__device__ __forceinline__ void a_chunk_load(AChunk<CH>& r, const uint8_t* arow_t, bool row_valid, int g0,
                                             int ngroups) {
  const int c0 = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < AChunk<CH>::kPerThread; ++i) {
    const int c = c0 + 16 * i;               // 16-byte piece of the chunk's row bytes
    if (c * 16 < ngroups * kGroup)
      r.v[i] = row_valid ? *reinterpret_cast<const i32x4*>(arow_t + g0 * kGroup + c * 16) : i32x4{0, 0, 0, 0};
  }
}

template <int CH, bool kMx>
__device__ __forceinline__ void a_chunk_store(const AChunk<CH>& r, StreamSmem<CH>& sm, int buf, int ngroups) {
  const int row = threadIdx.x >> 4, c0 = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < AChunk<CH>::kPerThread; ++i) {
    const int c = c0 + 16 * i;
    const int k = c * 16;                    // byte within the chunk's row
    if (k < ngroups * kGroup) {
      const int h = k >> 7, kk = k & 127;    // group within the chunk, K within the group
      const int q = kMx ? (kk >> 4) & 3 : kk >> 5, o = kMx ? (kk >> 6) * 16 : kk & 31;   // lane group, byte in it
      *reinterpret_cast<i32x4*>(&sm.a[buf][h][row + 16 * q][o]) = r.v[i];
    }
  }
}

// the lane's 16 weight bytes of groups g and g + 1 for each subtile
template <int NS>
struct WPair {
  i32x4 wa[NS], wb[NS];
};

// kGStride: bytes between a lane's weights of two consecutive groups (1024 in
// the GEMM storage, 64 in the row-major stored format)
template <int NS, int kGStride>
__device__ __forceinline__ void w_pair_load(WPair<NS>& w, const uint8_t* const (&pw)[NS], int g) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    w.wa[s] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(pw[s] + g * kGStride));
    w.wb[s] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(pw[s] + (g + 1) * kGStride));
  }
}

// the lane's 32 weight bytes u_k in K order, from the GEMM storage or (kRM) the row-major words
template <bool kRM>
__device__ __forceinline__ v8i split_nibbles(i32x4 w) {
  if constexpr (kRM) return nibbles_rowmajor_to_fp8(w);
  else return nibbles_to_fp8(w);
}

// group-128 INT4 form of one group pair: A operands from LDS, the +8 offset
// removed by the bias MFMAs (accumulator input), then acc += s * D per group
template <int NS, bool kRM>
__device__ __forceinline__ void pair_compute(const WPair<NS>& w, const float (&s0)[NS], const float (&s1)[NS],
                                             const uint8_t* a0, const uint8_t* a1, v4f (&acc)[NS]) {
  const v8i av0 = *reinterpret_cast<const v8i*>(a0);
  const v8i av1 = *reinterpret_cast<const v8i*>(a1);
  const v8i kb = bias_operand();
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const v4f c0 = mfma16x16x128(av0, kb, zero);
  const v4f c1 = mfma16x16x128(av1, kb, zero);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const v4f d0 = mfma16x16x128(av0, split_nibbles<kRM>(w.wa[s]), c0);
    const v4f d1 = mfma16x16x128(av1, split_nibbles<kRM>(w.wb[s]), c1);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(s1[s], d1[r], fmaf(s0[s], d0[r], acc[s][r]));
  }
}

// the MXFP4 form of one group pair: sb0 / sb1 hold the lane's E8M0 scale
// bytes (byte 0) of groups g and g + 1
template <int NS>
__device__ __forceinline__ void pair_compute_mx(const WPair<NS>& w, const int (&sb0)[NS], const int (&sb1)[NS],
                                                const uint8_t* a0, const uint8_t* a1, v4f (&acc)[NS]) {
  const v8i av0 = *reinterpret_cast<const v8i*>(a0);
  const v8i av1 = *reinterpret_cast<const v8i*>(a1);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    acc[s] = mfma_mx(av0, w.wa[s], acc[s], sb0[s]);
    acc[s] = mfma_mx(av1, w.wb[s], acc[s], sb1[s]);
  }
}

// the per-channel INT8 form of one group pair: int32 products, no scales
// (the nibbles u = q + 8 are the INT8 B operand; the offset is removed with
// the activation row sums in the epilogue)
template <int NS, bool kRM>
__device__ __forceinline__ void pair_compute_i8(const WPair<NS>& w, const uint8_t* a0, const uint8_t* a1,
                                                i32x4 (&acc)[NS]) {
  const v8i av0 = *reinterpret_cast<const v8i*>(a0);
  const v8i av1 = *reinterpret_cast<const v8i*>(a1);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const v8i b0 = split_nibbles<kRM>(w.wa[s]), b1 = split_nibbles<kRM>(w.wb[s]);
    acc[s] = mfma_i8_16x16x64(av0.lo, b0.lo, acc[s]);
    acc[s] = mfma_i8_16x16x64(av0.hi, b0.hi, acc[s]);
    acc[s] = mfma_i8_16x16x64(av1.lo, b1.lo, acc[s]);
    acc[s] = mfma_i8_16x16x64(av1.hi, b1.hi, acc[s]);
  }
}

// kForm: kFormChannel, the per-channel variant (INT8 activations with row sums
// a_rowsum, one scale per weight row in w_scale [E][N]); kFormG128, the
// group-128 FP8 form (w_scale [E][K/128][N]); kFormMx, MXFP4 weights (w_scale
// holds the E8M0 words, [E][K/128][N]).
// kSwiglu: the fused gate/up form: a wave's two subtiles are the gate and the
// up rows of the same 16 output columns (gate_up_row), and the epilogue
// writes act = silu(gate) * up [M][N/2] and the workgroup's max |act| of each
// row (its 64 output columns) to pmax[p][blockIdx.x].
// kRM: the weights come in the row-major stored format instead of the GEMM
// storage (int32 [E][N][K/8] uint4b8 words or u8 [E][N][K/2] E2M1 codes, scales
// [E][N][K/128] fp32 or [E][N][K/32] E8M0 bytes): each lane still loads its own
// 16-byte operand per group (row col, bytes 16 kq .. +15 of the row's group),
// a wave's load then reading 64 bytes of each of 16 rows instead of one 1 KB
// piece, and the INT4 nibbles need two byte permutes more to reach K order.
// N % 16 == 0 is enough there: a subtile past N loads row 0 and stores nothing.
// At least 3 waves per SIMD (3 workgroups per CU): the kernel is bound by the
// weight loads it has in flight.  Without the bound the group-128 form put its
// accumulators in AGPRs on top of 156 VGPRs and ran 2 waves per SIMD.
template <int NS, int CH, int kForm, bool kSwiglu, bool kRM>
__global__ __launch_bounds__(kStreamThreads, 3) void gg_stream_kernel(const uint8_t* __restrict__ a,
                                                                   const float* __restrict__ a_scale,
                                                                   const int32_t* __restrict__ a_rowsum,
                                                                   const int32_t* __restrict__ a_rows,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ w_packed,
                                                                   const float* __restrict__ w_scale, int64_t N,
                                                                   int64_t K, float* __restrict__ out,
                                                                   float* __restrict__ pmax) {
  static_assert(!kSwiglu || NS == 2, "fused SwiGLU pairs the two subtiles of a wave");
  constexpr bool kInt8 = kForm == kFormChannel;
  constexpr bool kMx = kForm == kFormMx;
  __shared__ StreamSmem<CH> sm;
  const int e = blockIdx.y;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  if (r1 <= r0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int col = lane & 15, kq = lane >> 4;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * (16 * NS);
  const bool active = n0 < N;                // waves past N only help stage activations
  const int G = (int)(K >> 7);
  const int64_t row_bytes = K >> 1;

  // subtile s: weight rows nb .. nb+15 are the G pieces of 1 KB from their block's base;
  // the lane reads row col, bytes 16 kq .. +15 of each.  Group scales: word (g, nb + col).
  // Row-major (kRM): row nb + col, bytes 64 g + 16 kq .. +15; scales word (nb + col, g).
  constexpr int kGStride = kRM ? 64 : 1024;
  const int64_t sstride = kRM ? 1 : N;         // scale words between two groups of a column
  const uint8_t* pw[NS];
  const uint32_t* srow[NS];
  bool sub_ok[NS];                             // subtile s holds columns below N
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    sub_ok[s] = n0 + 16 * s < N;
    const int64_t nb = sub_ok[s] ? (kSwiglu ? (int64_t)gate_up_row((int)(n0 + 16 * s), (int)(N / 2)) : n0 + 16 * s) : 0;
    if constexpr (kRM) {
      pw[s] = reinterpret_cast<const uint8_t*>(w_packed) + ((int64_t)e * N + nb + col) * row_bytes + kq * 16;
      srow[s] = reinterpret_cast<const uint32_t*>(w_scale) + ((int64_t)e * N + nb + col) * G;
    } else {
      pw[s] = reinterpret_cast<const uint8_t*>(w_packed) + ((int64_t)e * N + nb) * row_bytes + col * 64 + kq * 16;
      srow[s] = reinterpret_cast<const uint32_t*>(w_scale) + (int64_t)e * N * G + nb + col;
    }
  }

  for (int m0 = r0; m0 < r1; m0 += 16) {
    // activation row staged by this thread (rows past the end are zeros; never stored)
    const int p_t = min(m0 + (int)(threadIdx.x >> 4), r1 - 1);
    const bool row_valid = m0 + (int)(threadIdx.x >> 4) < r1;
    const uint8_t* arow_t = a + (int64_t)(a_rows ? a_rows[p_t] : p_t) * K;
    using Acc = std::conditional_t<kInt8, i32x4, v4f>;
    Acc acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = Acc{0, 0, 0, 0};

    const int nchunks = (G + 2 * CH - 1) / (2 * CH);
    {
      AChunk<CH> ar;
      a_chunk_load(ar, arow_t, row_valid, 0, min(G, 2 * CH));
      a_chunk_store<CH, kMx>(ar, sm, 0, min(G, 2 * CH));
    }
    __syncthreads();
    for (int ci = 0; ci < nchunks; ++ci) {
      const int g0 = ci * 2 * CH;
      const int ng = min(2 * CH, G - g0);    // groups in this chunk
      const int buf = ci & 1;
      AChunk<CH> next;
      const bool has_next = ci + 1 < nchunks;
      const int ng_next = has_next ? min(2 * CH, G - g0 - 2 * CH) : 0;
      if (has_next) a_chunk_load(next, arow_t, row_valid, g0 + 2 * CH, ng_next);
      if (active) {
        // group scales of this chunk (bits: fp32, or MX words shifted so that byte 0 is the lane's quarter)
        uint32_t sc[NS][2 * CH];
        if constexpr (!kInt8) {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int h = 0; h < 2 * CH; ++h) {
              sc[s][h] = h < ng ? srow[s][(int64_t)(g0 + h) * sstride] : 0u;
              if constexpr (kMx) sc[s][h] >>= 8 * kq;
            }
          }
        }
        const int npairs = ng >> 1;
#pragma unroll
        for (int u = 0; u < CH; u += 2) {
          if (u < npairs) {
            WPair<NS> w0, w1;
            const bool two = u + 1 < npairs;
            w_pair_load<NS, kGStride>(w0, pw, g0 + 2 * u);
            if (two) w_pair_load<NS, kGStride>(w1, pw, g0 + 2 * u + 2);
            const uint8_t* a00 = &sm.a[buf][2 * u][lane][0];
            const uint8_t* a01 = &sm.a[buf][2 * u + 1][lane][0];
            const uint8_t* a10 = &sm.a[buf][2 * u + 2][lane][0];
            const uint8_t* a11 = &sm.a[buf][2 * u + 3][lane][0];
            if constexpr (kInt8) {
              pair_compute_i8<NS, kRM>(w0, a00, a01, acc);
              if (two) pair_compute_i8<NS, kRM>(w1, a10, a11, acc);
            } else if constexpr (kMx) {
              int s0[NS], s1[NS];
#pragma unroll
              for (int s = 0; s < NS; ++s) { s0[s] = (int)sc[s][2 * u]; s1[s] = (int)sc[s][2 * u + 1]; }
              pair_compute_mx(w0, s0, s1, a00, a01, acc);
              if (two) {
#pragma unroll
                for (int s = 0; s < NS; ++s) { s0[s] = (int)sc[s][2 * u + 2]; s1[s] = (int)sc[s][2 * u + 3]; }
                pair_compute_mx(w1, s0, s1, a10, a11, acc);
              }
            } else {
              float s0[NS], s1[NS];
#pragma unroll
              for (int s = 0; s < NS; ++s) {
                s0[s] = __uint_as_float(sc[s][2 * u]);
                s1[s] = __uint_as_float(sc[s][2 * u + 1]);
              }
              pair_compute<NS, kRM>(w0, s0, s1, a00, a01, acc);
              if (two) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                  s0[s] = __uint_as_float(sc[s][2 * u + 2]);
                  s1[s] = __uint_as_float(sc[s][2 * u + 3]);
                }
                pair_compute<NS, kRM>(w1, s0, s1, a10, a11, acc);
              }
            }
          }
        }
        if (ng & 1) {   // a last single group
          const int h = ng - 1;
          const v8i av = *reinterpret_cast<const v8i*>(&sm.a[buf][h][lane][0]);
          const v4f c = (kInt8 || kMx) ? v4f{0.f, 0.f, 0.f, 0.f}
                                       : mfma16x16x128(av, bias_operand(), v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const i32x4 wq = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(pw[s] + (g0 + h) * kGStride));
            if constexpr (kInt8) {
              const v8i b = split_nibbles<kRM>(wq);
              acc[s] = mfma_i8_16x16x64(av.lo, b.lo, acc[s]);
              acc[s] = mfma_i8_16x16x64(av.hi, b.hi, acc[s]);
            } else if constexpr (kMx) {
              acc[s] = mfma_mx(av, wq, acc[s], (int)sc[s][h]);
            } else {
              const v4f d = mfma16x16x128(av, split_nibbles<kRM>(wq), c);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(__uint_as_float(sc[s][h]), d[r], acc[s][r]);
            }
          }
        }
      }
      if (has_next) a_chunk_store<CH, kMx>(next, sm, buf ^ 1, ng_next);
      __syncthreads();
    }

    if (active) {
      if constexpr (kInt8) {
        // out = a_scale * w_scale * (sum a u - 8 sum a): the integer part is exact
        float ws[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int v = sub_ok[s] ? (int)(n0 + 16 * s) + col : 0;
          ws[s] = w_scale[(int64_t)e * N + (kSwiglu ? gate_up_row(v, (int)(N / 2)) : v)];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = m0 + kq * 4 + r;
          if constexpr (kSwiglu) {
            // gate and up of output column n0 / 2 + col (rows past r1 compute on a repeated row, unstored)
            const int pc = min(p, r1 - 1);
            const int64_t src = a_rows ? a_rows[pc] : pc;
            const int off = 8 * a_rowsum[src];
            const float as = a_scale[src];
            const float y = silu_mul((float)(acc[0][r] - off) * as * ws[0], (float)(acc[1][r] - off) * as * ws[1]);
            const float m = max16(p < r1 ? fabsf(y) : 0.0f);
            if (p < r1) out[(int64_t)p * (N / 2) + n0 / 2 + col] = y;
            if (col == 0) sm.rmax[wave][kq * 4 + r] = m;
          } else if (p < r1) {
            const int64_t src = a_rows ? a_rows[p] : p;
            const int off = 8 * a_rowsum[src];
            const float as = a_scale[src];
#pragma unroll
            for (int s = 0; s < NS; ++s)
              if (sub_ok[s]) out[(int64_t)p * N + n0 + 16 * s + col] = (float)(acc[s][r] - off) * as * ws[s];
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = m0 + kq * 4 + r;
          if constexpr (kSwiglu) {
            const int pc = min(p, r1 - 1);
            const int64_t src = a_rows ? a_rows[pc] : pc;
            const float rs = a_scale[src] * (kMx ? 1.0f : kUnitScale);
            const float y = silu_mul(acc[0][r] * rs, acc[1][r] * rs);
            const float m = max16(p < r1 ? fabsf(y) : 0.0f);
            if (p < r1) out[(int64_t)p * (N / 2) + n0 / 2 + col] = y;
            if (col == 0) sm.rmax[wave][kq * 4 + r] = m;
          } else if (p < r1) {
            const int64_t src = a_rows ? a_rows[p] : p;
            const float rs = a_scale[src] * (kMx ? 1.0f : kUnitScale);
#pragma unroll
            for (int s = 0; s < NS; ++s)
              if (sub_ok[s]) out[(int64_t)p * N + n0 + 16 * s + col] = acc[s][r] * rs;
          }
        }
      }
    }
    if constexpr (kSwiglu) {
      // the workgroup's row maxima over its 4 waves (a wave past N counts 0)
      if (!active && lane < 16) sm.rmax[wave][lane] = 0.0f;
      __syncthreads();
      if (threadIdx.x < 16 && m0 + (int)threadIdx.x < r1) {
        const float m = fmaxf(fmaxf(sm.rmax[0][threadIdx.x], sm.rmax[1][threadIdx.x]),
                              fmaxf(sm.rmax[2][threadIdx.x], sm.rmax[3][threadIdx.x]));
        pmax[(int64_t)(m0 + threadIdx.x) * gridDim.x + blockIdx.x] = m;
      }
    }
  }
}

template <int NS, int CH, int kForm, bool kSwiglu>
static void launch_variant(const GemmArgs& g, hipStream_t stream) {
  const dim3 grid((unsigned)((g.N + 64 * NS - 1) / (64 * NS)), (unsigned)g.E);
  auto kernel = g.row_major ? gg_stream_kernel<NS, CH, kForm, kSwiglu, true> : gg_stream_kernel<NS, CH, kForm, kSwiglu, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kStreamThreads), 0, stream, g.a,
                     g.a_scale, g.a_rowsum, g.a_rows, g.offsets, g.w_packed, g.w_scale, g.N, g.K, g.out, g.pmax);
}

hipError_t launch_gg_stream(const GemmArgs& g, hipStream_t stream) {
  if (g.pmax) {
    // the fused gate/up GEMM: chunks of 4 groups (128 VGPRs or fewer, so 4 waves
    // per SIMD; 1.1% faster at decode for the FP8 forms, 0.4% for the INT8 one)
    if (g.a_rowsum) launch_variant<2, 2, kFormChannel, true>(g, stream);
    else if (g.mx) launch_variant<2, 2, kFormMx, true>(g, stream);
    else launch_variant<2, 2, kFormG128, true>(g, stream);
  } else {
    // the plain form (the down GEMM, K = I): chunks of 4 groups for the FP8 forms
    // (2.4% faster in the layer at decode), of 8 for the INT8 one (1.6% faster)
    if (g.a_rowsum) launch_variant<2, 4, kFormChannel, false>(g, stream);
    else if (g.mx) launch_variant<2, 2, kFormMx, false>(g, stream);
    else launch_variant<2, 2, kFormG128, false>(g, stream);
  }
  return hipGetLastError();
}

}  // namespace w4a8
