// The stable counting sort of layer step 3, as device code shared by the
// permutation kernels and the fused front of the layer.
#pragma once

#include "common.hpp"

namespace w4a8 {

constexpr int kPermBlock = 1024;        // routed indices per block
constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kPermMaxE = 1024;

// inclusive scan of one value per lane across the wave
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// The stable scatter of the kPermBlock indices from `base`: run[e] holds the
// next free row of expert e for them (advanced here), wcnt is zero.  Rounds of
// 256 indices in index order; within a round the rank of an index among the
// round's earlier indices with the same expert comes from ballot-based peer
// matching inside a wave and per-wave counts across waves.
__device__ __forceinline__ void permute_scatter_rounds(const int32_t* __restrict__ ids, int64_t R, int k, int E,
                                                       int64_t base, int* run, int (*wcnt)[kPermMaxE],
                                                       int32_t* __restrict__ row_token,
                                                       int32_t* __restrict__ inv_pos) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int kRounds = kPermBlock / kPermThreads;
  int keys[kRounds];                                // every round's id loaded at once: one wait, not one per round
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
    const int64_t f = base + (int64_t)round * kPermThreads + tid;
    keys[round] = f < R ? ids[f] : kPermMaxE;       // sentinel key for the tail
  }
#pragma unroll
  for (int round = 0; round < kRounds; ++round) {
    const int64_t f = base + (int64_t)round * kPermThreads + tid;   // rounds, then threads: index order
    const bool valid = f < R;
    int key = keys[round];
    if ((unsigned)key >= (unsigned)E) key = kPermMaxE;
    if (valid && key == kPermMaxE) inv_pos[f] = -1;   // an id outside [0, E) is not routed
    const bool routed = key != kPermMaxE;
    // lanes holding the same key: match 11 key bits with ballots
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const uint64_t m = __ballot((key >> b) & 1);
      peers &= ((key >> b) & 1) ? m : ~m;
    }
    const int rank_in_wave = __popcll(peers & lt_mask);
    const bool leader = (peers & lt_mask) == 0;
    const int n_in_wave = __popcll(peers);
    if (routed && leader) wcnt[wave][key] = n_in_wave;
    __syncthreads();
    if (routed) {
      int pos = run[key] + rank_in_wave;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][key];
      row_token[pos] = (int32_t)(f / k);
      inv_pos[f] = pos;
    }
    __syncthreads();
    if (routed && leader) {
      atomicAdd(&run[key], n_in_wave);               // integer adds: order does not matter
      wcnt[wave][key] = 0;
    }
    __syncthreads();
  }
}

// All three steps in one block when R <= kPermSmallMax: counts in LDS, the
// exclusive scan over experts (4 consecutive experts per thread, then a
// wavefront scan and the 4 wave totals), then the scatter of each block of
// kPermBlock indices in order (run[] carries every expert's next row across them).
constexpr int64_t kPermSmallMax = 4 * kPermBlock;
__device__ __forceinline__ void permute_small(const int32_t* __restrict__ ids, int64_t R, int k, int E,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
                                              int32_t* __restrict__ inv_pos) {
  __shared__ int run[kPermMaxE];
  __shared__ int wcnt[kPermWaves][kPermMaxE];
  __shared__ int wave_tot[kPermWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < kPermMaxE; e += kPermThreads) {
    run[e] = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  // every id of this thread loaded at once (R <= kPermSmallMax: at most 16 each), then counted
  constexpr int kMaxPer = (int)(kPermSmallMax / kPermThreads);
  int mine[kMaxPer];
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int64_t i = tid + (int64_t)j * kPermThreads;
    mine[j] = i < R ? ids[i] : -1;
  }
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j)
    if ((unsigned)mine[j] < (unsigned)E) atomicAdd(&run[mine[j]], 1);   // integer counts: order does not matter
  __syncthreads();
  // thread t: experts 4t .. 4t + 3 (counts past E are 0)
  int c[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = run[4 * tid + j];
    local += c[j];
  }
  const int incl = wave_inclusive_scan(local, lane);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int excl = incl - local;
  for (int w = 0; w < wave; ++w) excl += wave_tot[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < E) offsets[e] = excl;
    run[e] = excl;                                   // the first row of expert e
    excl += c[j];
  }
  if (tid == kPermThreads - 1) offsets[E] = excl;    // E <= 4 * 256: the last thread ends the scan
  __syncthreads();
  for (int64_t base = 0; base < R; base += kPermBlock)
    permute_scatter_rounds(ids, R, k, E, base, run, wcnt, row_token, inv_pos);
}

}  // namespace w4a8
