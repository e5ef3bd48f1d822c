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
// expert with no rows returns at once.  In the multi-block form each weight
// load feeds up to MB = 4 M blocks of 16 rows: the workgroup picks MB from its
// expert's row count (1 for up to 16 rows, 2 for up to 32, else 4), so an
// expert's weights are streamed once for every 64 of its rows, and a skewed
// batch, whose hot experts get many of its rows, reads little more than the
// weights it touches.  Its LDS holds 2 buffers of 8 (group, M block)
// activation tiles of 2 KB: 4-group chunks for MB = 1 and 2, group-pair chunks
// for MB = 4.  The one-block form (MB = 1 only; batches of at most 8 rows per
// expert on average) keeps 2 buffers of one chunk's tiles and fewer registers,
// for 4 waves per SIMD.
// With the kernel choice taken on the device (sel_rows >= 0), every wave first
// reads the E + 1 expert offsets and the workgroup returns at once if an
// expert has more rows than the streaming kernel takes.
//
// The same kernel reads the weights in the row-major stored format too (the
// grouped GEMM calls without "_prepacked"): the lane's operand of a group is
// then 16 bytes of its own row, so a wave's load covers 64 bytes of 16 rows.
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace w4a8 {

constexpr int kStreamThreads = 256;
constexpr int kStreamTiles = 8;      // the most (group, M block) activation tiles per LDS buffer

// LDS image of the activation tiles of one chunk: for group h of the chunk,
// M block b and MFMA lane L, tile h MB + b holds the 32 bytes lane L feeds to
// the MFMA (row 16 b + L % 16, K bytes 32 (L / 16) .. +31 of group h; MX form:
// K bytes 16 (L / 16) .. +15 and 64 + 16 (L / 16) .. +15).
template <int kTiles, int kRows>
struct StreamSmem {
  uint8_t a[2][kTiles][64][32];
  float rmax[4][kRows];              // fused form: row max |act| of each wave's 16 output columns
};

// Chunk of activations -> registers: for each M block b, thread t loads row
// 16 b + t / 16 (16 B pieces t % 16, +16, +32, ... of the chunk's 256 CHB bytes per row).
template <int MB, int CHB>
struct AChunk {
  i32x4 v[MB][CHB];
};

// A thread whose row is past the expert's last one stages zeros instead: the
// products of such a row are never stored, and each output row depends only
// on its own activation row, so its bytes need not be read.
template <int MB, int CHB>
__device__ __forceinline__ void a_chunk_load(AChunk<MB, CHB>& r, const uint8_t* const (&arow)[MB],
                                             const bool (&row_valid)[MB], int g0, int ngroups) {
  const int c0 = threadIdx.x & 15;
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < CHB; ++i) {
      const int c = c0 + 16 * i;             // 16-byte piece of the chunk's row bytes
      if (c * 16 < ngroups * kGroup)
        r.v[b][i] = row_valid[b] ? *reinterpret_cast<const i32x4*>(arow[b] + g0 * kGroup + c * 16)
                                 : i32x4{0, 0, 0, 0};
    }
}

template <int MB, int CHB, bool kMx, typename Smem>
__device__ __forceinline__ void a_chunk_store(const AChunk<MB, CHB>& r, Smem& sm, int buf, int ngroups) {
  const int row = threadIdx.x >> 4, c0 = threadIdx.x & 15;
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < CHB; ++i) {
      const int c = c0 + 16 * i;
      const int k = c * 16;                  // byte within the chunk's row
      if (k < ngroups * kGroup) {
        const int h = k >> 7, kk = k & 127;  // group within the chunk, K within the group
        const int q = kMx ? (kk >> 4) & 3 : kk >> 5, o = kMx ? (kk >> 6) * 16 : kk & 31;   // lane group, byte in it
        *reinterpret_cast<i32x4*>(&sm.a[buf][h * MB + b][row + 16 * q][o]) = r.v[b][i];
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

__device__ __forceinline__ v8i lds_v8i(const uint8_t* p) { return *reinterpret_cast<const v8i*>(p); }

// group-128 INT4 form of one group pair for MB M blocks: per subtile the
// weight bytes are split once and serve every M block, whose A operands come
// from LDS (a0 / a1: block 0 of the two groups' tiles, block b 2 KB further);
// the +8 offset is removed by the bias MFMAs (accumulator input), then
// acc += s * D per group.  One block: the bias products serve every subtile.
// More blocks: one subtile at a time (the bias products again per subtile), so
// that few values are live.
template <int NS, int MB, bool kRM>
__device__ __forceinline__ void pair_compute(const WPair<NS>& w, const float (&s0)[NS], const float (&s1)[NS],
                                             const uint8_t* a0, const uint8_t* a1, v4f (&acc)[MB][NS]) {
  const v8i kb = bias_operand();
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if constexpr (MB == 1) {
    const v8i av0 = lds_v8i(a0), av1 = lds_v8i(a1);
    const v4f c0 = mfma16x16x128(av0, kb, zero), c1 = mfma16x16x128(av1, kb, zero);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const v4f d0 = mfma16x16x128(av0, split_nibbles<kRM>(w.wa[s]), c0);
      const v4f d1 = mfma16x16x128(av1, split_nibbles<kRM>(w.wb[s]), c1);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[0][s][r] = fmaf(s1[s], d1[r], fmaf(s0[s], d0[r], acc[0][s][r]));
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const v8i b0 = split_nibbles<kRM>(w.wa[s]), b1 = split_nibbles<kRM>(w.wb[s]);
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const v8i av0 = lds_v8i(a0 + 2048 * b), av1 = lds_v8i(a1 + 2048 * b);
      const v4f d0 = mfma16x16x128(av0, b0, mfma16x16x128(av0, kb, zero));
      const v4f d1 = mfma16x16x128(av1, b1, mfma16x16x128(av1, kb, zero));
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[b][s][r] = fmaf(s1[s], d1[r], fmaf(s0[s], d0[r], acc[b][s][r]));
      if constexpr (MB > 1) __builtin_amdgcn_sched_barrier(0);   // one M block at a time: few values live
    }
  }
}

// the MXFP4 form of one group pair: sb0 / sb1 hold the lane's E8M0 scale
// bytes (byte 0) of groups g and g + 1
template <int NS, int MB>
__device__ __forceinline__ void pair_compute_mx(const WPair<NS>& w, const int (&sb0)[NS], const int (&sb1)[NS],
                                                const uint8_t* a0, const uint8_t* a1, v4f (&acc)[MB][NS]) {
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const v8i av0 = lds_v8i(a0 + 2048 * b), av1 = lds_v8i(a1 + 2048 * b);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc[b][s] = mfma_mx(av0, w.wa[s], acc[b][s], sb0[s]);
      acc[b][s] = mfma_mx(av1, w.wb[s], acc[b][s], sb1[s]);
    }
  }
}

// the per-channel INT8 form of one group pair: int32 products, no scales
// (the nibbles u = q + 8 are the INT8 B operand; the offset is removed with
// the activation row sums in the epilogue)
template <int NS, int MB, bool kRM>
__device__ __forceinline__ void pair_compute_i8(const WPair<NS>& w, const uint8_t* a0, const uint8_t* a1,
                                                i32x4 (&acc)[MB][NS]) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const v8i b0 = split_nibbles<kRM>(w.wa[s]), b1 = split_nibbles<kRM>(w.wb[s]);
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const v8i av0 = lds_v8i(a0 + 2048 * b), av1 = lds_v8i(a1 + 2048 * b);
      acc[b][s] = mfma_i8_16x16x64(av0.lo, b0.lo, acc[b][s]);
      acc[b][s] = mfma_i8_16x16x64(av0.hi, b0.hi, acc[b][s]);
      acc[b][s] = mfma_i8_16x16x64(av1.lo, b1.lo, acc[b][s]);
      acc[b][s] = mfma_i8_16x16x64(av1.hi, b1.hi, acc[b][s]);
      if constexpr (MB > 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// the most rows of the experts base + 4 lane .. +3 (offsets: E + 1 row starts)
__device__ __forceinline__ int lane_max_rows(const int32_t* __restrict__ offsets, int E, int base) {
  const int i0 = base + 4 * (int)(threadIdx.x & 63);
  int o[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) o[j] = offsets[min(i0 + j, E)];   // past E: offsets[E], no rows
  int most = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) most = max(most, o[j + 1] - o[j]);
  return most;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
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
// CH: group pairs per chunk for MB = 1 (MB = 2 takes up to 2, MB = 4 one).
// kMaxMB: the most M blocks a weight load feeds (1, or 4 with the row-count
// choice); the one-block kernel keeps its registers and LDS small.
// At least 4 waves per SIMD for the one-block kernel, 3 for the multi-block one:
// the kernel is bound by the weight loads it has in flight.  Without a bound the
// group-128 form put its accumulators in AGPRs on top of 156 VGPRs and ran 2
// waves per SIMD.
template <int NS, int CH, int kForm, bool kSwiglu, bool kRM, int kMaxMB>
__global__ __launch_bounds__(kStreamThreads, kMaxMB == 1 ? 4 : 3) void gg_stream_kernel(const uint8_t* __restrict__ a,
                                                                   const float* __restrict__ a_scale,
                                                                   const int32_t* __restrict__ a_rowsum,
                                                                   const int32_t* __restrict__ a_rows,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ w_packed,
                                                                   const float* __restrict__ w_scale, int64_t N,
                                                                   int64_t K, float* __restrict__ out,
                                                                   float* __restrict__ pmax, int E, int sel_rows,
                                                                   const int32_t* __restrict__ out_rows) {
  static_assert(!kSwiglu || NS == 2, "fused SwiGLU pairs the two subtiles of a wave");
  static_assert(2 * CH <= kStreamTiles, "the chunk's tiles must fit the LDS buffer");
  constexpr bool kInt8 = kForm == kFormChannel;
  constexpr bool kMx = kForm == kFormMx;
  __shared__ StreamSmem<kMaxMB == 1 ? 2 * CH : kStreamTiles, 16 * kMaxMB> sm;
  const int e = blockIdx.y;
  // the choice on the device: the tiled kernel takes a batch with an expert of more than
  // sel_rows rows (the offsets are loaded with the expert's own, in one round trip)
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const int lane_most = sel_rows >= 0 ? lane_max_rows(offsets, E, 0) : 0;   // experts 0 .. 255
  if (r1 <= r0) return;
  if (sel_rows >= 0) {
    int most = lane_most;
    for (int base = 256; base < E; base += 256) most = max(most, lane_max_rows(offsets, E, base));
    if (wave_max(most) > sel_rows) return;   // every wave alike
  }
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
  float ws[NS];                                // INT8 form: the per-channel weight scales
  if constexpr (kInt8) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int v = sub_ok[s] ? (int)(n0 + 16 * s) + col : 0;
      ws[s] = w_scale[(int64_t)e * N + (kSwiglu ? gate_up_row(v, (int)(N / 2)) : v)];
    }
  }

  // The rows in passes of MB M blocks (16 MB rows), each weight load feeding all of them;
  // CHB group pairs per chunk (2 CHB groups), the chunk's 2 CHB MB activation tiles in LDS.
  auto rows_pass = [&](auto MB_, auto CHB_) {
    constexpr int MB = decltype(MB_)::value;
    constexpr int CHB = decltype(CHB_)::value;
    static_assert(2 * CHB * MB <= kStreamTiles, "tiles per buffer");
    for (int m0 = r0; m0 < r1; m0 += 16 * MB) {
      // activation rows staged by this thread (rows past the end are zeros; never stored)
      const uint8_t* arow[MB];
      bool row_valid[MB];
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int p_t = m0 + 16 * b + (int)(threadIdx.x >> 4);
        row_valid[b] = p_t < r1;
        const int pc = min(p_t, r1 - 1);
        arow[b] = a + (int64_t)(a_rows ? a_rows[pc] : pc) * K;
      }
      using Acc = std::conditional_t<kInt8, i32x4, v4f>;
      Acc acc[MB][NS];
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[b][s] = Acc{0, 0, 0, 0};

      const int nchunks = (G + 2 * CHB - 1) / (2 * CHB);
      {
        AChunk<MB, CHB> ar;
        a_chunk_load(ar, arow, row_valid, 0, min(G, 2 * CHB));
        a_chunk_store<MB, CHB, kMx>(ar, sm, 0, min(G, 2 * CHB));
      }
      __syncthreads();
      for (int ci = 0; ci < nchunks; ++ci) {
        const int g0 = ci * 2 * CHB;
        const int ng = min(2 * CHB, G - g0);    // groups in this chunk
        const int buf = ci & 1;
        AChunk<MB, CHB> next;
        const bool has_next = ci + 1 < nchunks;
        const int ng_next = has_next ? min(2 * CHB, G - g0 - 2 * CHB) : 0;
        if (has_next) a_chunk_load(next, arow, row_valid, g0 + 2 * CHB, ng_next);
        if (active) {
          // group scales of this chunk (bits: fp32, or MX words shifted so that byte 0 is the lane's quarter)
          uint32_t sc[NS][2 * CHB];
          if constexpr (!kInt8) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
#pragma unroll
              for (int h = 0; h < 2 * CHB; ++h) {
                sc[s][h] = h < ng ? srow[s][(int64_t)(g0 + h) * sstride] : 0u;
                if constexpr (kMx) sc[s][h] >>= 8 * kq;
              }
            }
          }
          const int npairs = ng >> 1;
          // tile of group h, M block 0, for this lane
          auto tile = [&](int h) { return &sm.a[buf][h * MB][lane][0]; };
#pragma unroll
          for (int u = 0; u < CHB; u += 2) {
            if (u < npairs) {
              WPair<NS> w0, w1;
              const bool two = u + 1 < npairs;
              w_pair_load<NS, kGStride>(w0, pw, g0 + 2 * u);
              if (two) w_pair_load<NS, kGStride>(w1, pw, g0 + 2 * u + 2);
              if constexpr (kInt8) {
                pair_compute_i8<NS, MB, kRM>(w0, tile(2 * u), tile(2 * u + 1), acc);
                if (two) pair_compute_i8<NS, MB, kRM>(w1, tile(2 * u + 2), tile(2 * u + 3), acc);
              } else if constexpr (kMx) {
                int s0[NS], s1[NS];
#pragma unroll
                for (int s = 0; s < NS; ++s) { s0[s] = (int)sc[s][2 * u]; s1[s] = (int)sc[s][2 * u + 1]; }
                pair_compute_mx<NS, MB>(w0, s0, s1, tile(2 * u), tile(2 * u + 1), acc);
                if (two) {
#pragma unroll
                  for (int s = 0; s < NS; ++s) { s0[s] = (int)sc[s][2 * u + 2]; s1[s] = (int)sc[s][2 * u + 3]; }
                  pair_compute_mx<NS, MB>(w1, s0, s1, tile(2 * u + 2), tile(2 * u + 3), acc);
                }
              } else {
                float s0[NS], s1[NS];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                  s0[s] = __uint_as_float(sc[s][2 * u]);
                  s1[s] = __uint_as_float(sc[s][2 * u + 1]);
                }
                pair_compute<NS, MB, kRM>(w0, s0, s1, tile(2 * u), tile(2 * u + 1), acc);
                if (two) {
#pragma unroll
                  for (int s = 0; s < NS; ++s) {
                    s0[s] = __uint_as_float(sc[s][2 * u + 2]);
                    s1[s] = __uint_as_float(sc[s][2 * u + 3]);
                  }
                  pair_compute<NS, MB, kRM>(w1, s0, s1, tile(2 * u + 2), tile(2 * u + 3), acc);
                }
              }
            }
          }
          if (ng & 1) {   // a last single group
            const int h = ng - 1;
            i32x4 wq[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s)
              wq[s] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(pw[s] + (g0 + h) * kGStride));
#pragma unroll
            for (int b = 0; b < MB; ++b) {
              const v8i av = lds_v8i(tile(h) + 2048 * b);
              const v4f c = (kInt8 || kMx) ? v4f{0.f, 0.f, 0.f, 0.f}
                                           : mfma16x16x128(av, bias_operand(), v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int s = 0; s < NS; ++s) {
                if constexpr (kInt8) {
                  const v8i bq = split_nibbles<kRM>(wq[s]);
                  acc[b][s] = mfma_i8_16x16x64(av.lo, bq.lo, acc[b][s]);
                  acc[b][s] = mfma_i8_16x16x64(av.hi, bq.hi, acc[b][s]);
                } else if constexpr (kMx) {
                  acc[b][s] = mfma_mx(av, wq[s], acc[b][s], (int)sc[s][h]);
                } else {
                  const v4f d = mfma16x16x128(av, split_nibbles<kRM>(wq[s]), c);
#pragma unroll
                  for (int r = 0; r < 4; ++r) acc[b][s][r] = fmaf(__uint_as_float(sc[s][h]), d[r], acc[b][s][r]);
                }
              }
            }
          }
        }
        if (has_next) a_chunk_store<MB, CHB, kMx>(next, sm, buf ^ 1, ng_next);
        __syncthreads();
      }

      if (active) {
#pragma unroll
        for (int b = 0; b < MB; ++b) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rb = 16 * b + kq * 4 + r;   // row within the pass
            const int p = m0 + rb;
            if constexpr (kSwiglu) {
              // gate and up of output column n0 / 2 + col (rows past r1 compute on zero rows, unstored)
              const int pc = min(p, r1 - 1);
              const int64_t src = a_rows ? a_rows[pc] : pc;
              float yg, yu;
              if constexpr (kInt8) {
                const int off = 8 * a_rowsum[src];
                const float as = a_scale[src];
                yg = (float)(acc[b][0][r] - off) * as * ws[0];
                yu = (float)(acc[b][1][r] - off) * as * ws[1];
              } else {
                const float rs = a_scale[src] * (kMx ? 1.0f : kUnitScale);
                yg = acc[b][0][r] * rs;
                yu = acc[b][1][r] * rs;
              }
              const float y = silu_mul(yg, yu);
              const float m = max16(p < r1 ? fabsf(y) : 0.0f);
              if (p < r1) out[(int64_t)p * (N / 2) + n0 / 2 + col] = y;
              if (col == 0) sm.rmax[wave][rb] = m;
            } else if (p < r1) {
              const int64_t src = a_rows ? a_rows[p] : p;
              const int64_t dp = out_rows ? out_rows[p] : p;   // the row of out (the scatter form: a token-major slot)
              if constexpr (kInt8) {
                const int off = 8 * a_rowsum[src];
                const float as = a_scale[src];
#pragma unroll
                for (int s = 0; s < NS; ++s)
                  if (sub_ok[s]) out[dp * N + n0 + 16 * s + col] = (float)(acc[b][s][r] - off) * as * ws[s];
              } else {
                const float rs = a_scale[src] * (kMx ? 1.0f : kUnitScale);
#pragma unroll
                for (int s = 0; s < NS; ++s)
                  if (sub_ok[s]) out[dp * N + n0 + 16 * s + col] = acc[b][s][r] * rs;
              }
            }
          }
        }
      }
      if constexpr (kSwiglu) {
        // the workgroup's row maxima over its 4 waves (a wave past N counts 0)
        if (!active && lane < 16 * MB) sm.rmax[wave][lane] = 0.0f;
        __syncthreads();
        if (threadIdx.x < 16 * MB && m0 + (int)threadIdx.x < r1) {
          const float m = fmaxf(fmaxf(sm.rmax[0][threadIdx.x], sm.rmax[1][threadIdx.x]),
                                fmaxf(sm.rmax[2][threadIdx.x], sm.rmax[3][threadIdx.x]));
          pmax[(int64_t)(m0 + threadIdx.x) * gridDim.x + blockIdx.x] = m;
        }
      }
    }
  };
  // M blocks per weight load, by the expert's rows (every workgroup of the expert picks the same)
  const int rows = r1 - r0;
  if constexpr (kMaxMB >= 4) {
    if (rows > 32) {
      rows_pass(std::integral_constant<int, 4>{}, std::integral_constant<int, 1>{});
      return;
    }
    if (rows > 16) {
      rows_pass(std::integral_constant<int, 2>{}, std::integral_constant<int, (CH < 2 ? CH : 2)>{});
      return;
    }
  }
  rows_pass(std::integral_constant<int, 1>{}, std::integral_constant<int, CH>{});
}

// The multi-block kernel when the average expert has more than 8 rows.  The
// one-block kernel runs at 4 waves per SIMD, the multi-block one at 3: measured
// on the decode shape (H 6144, I 2048, 256 experts, top-8), uniform routing, the
// layer took 1.5% less time with the one-block kernel at 128 tokens and 0.8% less
// at 256; with one block per weight load the layer took 7% more time than the
// multi-block kernel at 384 tokens, 24% at 512, 56% at 1024, and 33-72% on
// Zipf-skewed routing.
template <int NS, int CH, int kForm, bool kSwiglu>
static void launch_variant(const GemmArgs& g, hipStream_t stream) {
  const dim3 grid((unsigned)((g.N + 64 * NS - 1) / (64 * NS)), (unsigned)g.E);
  const bool multi = g.M_total > 8 * (int64_t)g.E;
  auto kernel = multi ? (g.row_major ? gg_stream_kernel<NS, CH, kForm, kSwiglu, true, 4>
                                     : gg_stream_kernel<NS, CH, kForm, kSwiglu, false, 4>)
                      : (g.row_major ? gg_stream_kernel<NS, CH, kForm, kSwiglu, true, 1>
                                     : gg_stream_kernel<NS, CH, kForm, kSwiglu, false, 1>);
  hipLaunchKernelGGL(kernel, grid, dim3(kStreamThreads), 0, stream, g.a,
                     g.a_scale, g.a_rowsum, g.a_rows, g.offsets, g.w_packed, g.w_scale, g.N, g.K, g.out, g.pmax,
                     g.E, (int)g.sel_rows, g.out_rows);
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
