// Grouped W4A8 GEMM, tiled form: for many rows per expert (prefill).
//
// A persistent kernel (one 256-thread workgroup per CU) walks the ragged
// list of tiles of all experts.  A tile is up to 128 rows of one expert (an
// "M block") by 256 output columns; wave w owns columns 64w..64w+63 for all
// of the tile's rows (8 row subtiles x 4 column subtiles of 16x16 MFMA
// outputs, 128 fp32 accumulators per lane).  Because every wave covers every
// row, a short last M block costs only its own 16-row subtiles.
//
// K is walked one 128-wide group at a time through a 4-stage LDS ring filled
// by direct global-to-LDS loads (no registers), issued 3 groups ahead:
//   * the activation rows (FP8 codes, gathered through a_rows) in MFMA
//     operand order -- 16 KB per group;
//   * each wave's own packed INT4 weights of the group (lane col + 16 kq
//     takes quarter kq of weight row col: exactly its MFMA B operand);
//   * each wave's 64 group scales.
// Each wave turns its weights into MFMA B operands in registers (nibbles read
// as E4M3 bytes u * 2^-9, see gemm_common.hpp), and the +8 offset of the
// uint4b8 nibbles is removed with the per-row group sums of the activations,
// computed once per workgroup by one extra MFMA per row subtile, one group
// ahead, and shared through LDS.  Each group's partial product is scaled into
// the fp32 accumulators with the weights' group scale.  One barrier per
// group.
//
// Tile order: each XCD runs windows of consecutive tiles of an expert at the
// same time (see the tile loop), so a weight tile and an activation block are
// fetched from HBM about once and served to the other tiles of the window by
// that XCD's L2.
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace w4a8 {

constexpr int kTileM = 128;           // rows per tile (M block)
constexpr int kTileN = 256;           // columns per tile (4 waves x 64)
constexpr int kTiledThreads = 256;
constexpr int kMaxExperts = 1024;
constexpr int kXcds = 8;              // accelerator complex dies of an MI355X (round-robin dispatch)

constexpr int kStages = 4;            // LDS ring depth (groups)

// One ring slot: everything one 128-wide K group of a tile needs.  The slots
// are separate LDS variables, addressed with compile-time slot numbers, so
// that the compiler can tell the slot being read from the slots still being
// filled and does not wait for every load in flight before each LDS read.
struct __attribute__((aligned(16))) RingSlot {
  // activations in MFMA operand order: lane L's 32 bytes are split in two
  // 16-byte planes so that every LDS read is 64 lanes x 16 consecutive bytes
  // (conflict free) and every direct load fills one plane
  uint8_t a[8][2][64][16];   // [row subtile][half][MFMA lane][16 B]
  uint8_t w[4][4][64][16];   // [wave][column subtile][lane][16 B] packed INT4
  float sc[4][64];           // [wave][column] group scales
};

template <int S>
__device__ __forceinline__ RingSlot& slot(RingSlot& r0, RingSlot& r1, RingSlot& r2, RingSlot& r3) {
  if constexpr (S == 0) return r0;
  else if constexpr (S == 1) return r1;
  else if constexpr (S == 2) return r2;
  else return r3;
}

// Workgroup barrier that leaves direct-to-LDS loads in flight: __syncthreads'
// release fence would wait for all of them.  The caller waits for what the
// other waves need (its LDS writes and the loads that must have landed); the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void barrier_loads_in_flight() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// buffer resource of a byte range (gfx9 dword 3: raw, untyped access)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// direct loads into LDS: lane l's bytes (at rsrc + voff + soff) go to lds + size * l
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ int tiles_of(int rows, int nb) { return ((rows + kTileM - 1) / kTileM) * nb; }

template <typename T>
__device__ __forceinline__ T lds_load(const void* p) {
  return *reinterpret_cast<const T*>(__builtin_assume_aligned(p, 16));
}

__global__ __launch_bounds__(kTiledThreads, 1) void gg_tiled_kernel(const uint8_t* __restrict__ a,
                                                                   const float* __restrict__ a_scale,
                                                                   const int32_t* __restrict__ a_rows,
                                                                   const int32_t* __restrict__ offsets, int E,
                                                                   const int32_t* __restrict__ w_packed,
                                                                   const float* __restrict__ w_scale, int64_t N,
                                                                   int64_t K, float* __restrict__ out) {
  __shared__ RingSlot ring0, ring1, ring2, ring3;
  __shared__ __attribute__((aligned(16))) float bias_sm[kStages][kTileM];   // -2^-6 * group code sums per row
  __shared__ int tile_start[kMaxExperts + 1];                              // first tile index of each expert
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps wave-indexed values scalar
  const int col = lane & 15, kq = lane >> 4;
  const int NB = (int)((N + kTileN - 1) / kTileN);
  const int G = (int)(K >> 7);
  const uint32_t row_bytes = (uint32_t)(K >> 1);

  // ---- tile numbering: exclusive prefix of per-expert tile counts (wave-level scans)
  {
    __shared__ int wsum[4];
    constexpr int kPer = kMaxExperts / kTiledThreads;   // experts per thread
    int cnt[kPer];
    int local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid * kPer + i;
      cnt[i] = e < E ? tiles_of(offsets[e + 1] - offsets[e], NB) : 0;
      local += cnt[i];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    int run = base + incl - local;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid * kPer + i;
      if (e < E) tile_start[e] = run;
      run += cnt[i];
    }
    if (tid == kTiledThreads - 1) tile_start[E] = run;   // the grand total
    __syncthreads();
  }
  const int total = tile_start[E];

  // Tile t runs on the XCD and in the round that keep data sharing local:
  // workgroups are dispatched round-robin over the XCDs, so workgroup w sits
  // on XCD w % X.  Each round hands the X XCDs consecutive windows of grid/X
  // tiles; tiles are numbered expert by expert, N block by N block, with the
  // M blocks of one N block adjacent, so a window (the tiles one XCD runs at
  // the same time) shares its weight tiles and activation blocks in that
  // XCD's L2.
  const int grid = gridDim.x;
  const bool xcd_windows = (grid % kXcds) == 0;
  const int window = grid / kXcds;
  const int my_slot = xcd_windows ? (int)(blockIdx.x % kXcds) * window + (int)(blockIdx.x / kXcds) : (int)blockIdx.x;
  for (int t = my_slot; t < total; t += grid) {
    // ---- which expert, M block and N block
    int lo_e = 0, hi_e = E;                    // tile_start[lo_e] <= t < tile_start[hi_e]
    while (hi_e - lo_e > 1) {
      const int mid = (lo_e + hi_e) >> 1;
      if (tile_start[mid] <= t) lo_e = mid; else hi_e = mid;
    }
    const int e = lo_e;
    const int r_e = offsets[e], rows_e = offsets[e + 1] - r_e;
    const int mbs = (rows_e + kTileM - 1) / kTileM;
    const int local = t - tile_start[e];
    const int mb = local % mbs;
    const int nb = local / mbs;
    const int r0 = r_e + mb * kTileM;
    const int mlen = min(kTileM, rows_e - mb * kTileM);
    const int nsub = (mlen + 15) >> 4;
    const int n0 = nb * kTileN + wave * 64;
    const bool active = n0 < N;

    // activation bytes this lane stages: row subtiles 2*wave, 2*wave+1, row lane % 16,
    // quarter lane / 16 of each group
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a, 0xffffffffu);
    uint32_t aoff[2];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const int rl = min(16 * (2 * wave + i2) + col, mlen - 1);
      const int p = r0 + rl;
      aoff[i2] = (uint32_t)(a_rows ? a_rows[p] : p) * (uint32_t)K + (uint32_t)(kq * 32);
    }
    // weights of this wave: expert e, columns n0 + 16j + col, quarter kq of each group
    const __amdgpu_buffer_rsrc_t rw =
        buffer_rsrc(reinterpret_cast<const uint8_t*>(w_packed) + (int64_t)e * N * row_bytes, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w_scale + (int64_t)e * N * G, (uint32_t)(N * G * 4));
    const int nw = active ? n0 : 0;   // a wave past the last column block loads (and ignores) block 0
    const uint32_t woff = (uint32_t)(nw + col) * row_bytes + kq * 16;
    const uint32_t soff = (uint32_t)(nw + lane) * (uint32_t)G * 4u;   // this lane's column for the scales

    // Stage group g into slot S: 4 activation loads, 4 weight loads and 1 scale
    // load per wave (a wave past the last column block loads column block 0,
    // so that every wave has the same 9 loads in flight).
    auto stage = [&](auto S_, int g) {
      RingSlot& sl = slot<decltype(S_)::value>(ring0, ring1, ring2, ring3);
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
        for (int half = 0; half < 2; ++half)
          dma16(ra, aoff[i2], (uint32_t)(g * kGroup + half * 16), &sl.a[2 * wave + i2][half][0][0]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16(rw, woff, (uint32_t)(16 * j) * row_bytes + (uint32_t)(g * 64), &sl.w[wave][j][0][0]);
      dma4(rs, soff, (uint32_t)g * 4u, &sl.sc[wave][0]);
    };
    // group sums of this wave's two row subtiles for the group in slot S -> bias_sm[S]
    auto row_sums = [&](auto S_) {
      constexpr int S = decltype(S_)::value;
      RingSlot& sl = slot<S>(ring0, ring1, ring2, ring3);
      const v8i kb = bias_operand();
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int i = 2 * wave + i2;
        if (i < nsub) {
          const uint8_t* ap = &sl.a[i][0][lane][0];
          const i32x4 x0 = lds_load<i32x4>(ap);
          const i32x4 x1 = lds_load<i32x4>(ap + 1024);
          const v8i av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          const v4f c = mfma16x16x128(av, kb, v4f{0.f, 0.f, 0.f, 0.f});
          if (col == 0) *reinterpret_cast<v4f*>(&bias_sm[S][16 * i + 4 * kq]) = c;
        }
      }
    };

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // one K group in slot S: prefetch group g+3, share the row sums of group
    // g+1, multiply group g, then wait until group g+2 has landed
    auto step = [&](auto S_, int g) {
      constexpr int S = decltype(S_)::value;
      if (g >= G) return;
      if (g + 3 < G) stage(std::integral_constant<int, (S + 3) % kStages>{}, g + 3);
      if (g + 1 < G) row_sums(std::integral_constant<int, (S + 1) % kStages>{});
      if (active) {
        RingSlot& sl = slot<S>(ring0, ring1, ring2, ring3);
        const uint8_t* abase = &sl.a[0][0][lane][0];               // + i*2K + half*1K
        const uint8_t* wbase = &sl.w[wave][0][lane][0];             // + j*1K
        const float* bbase = &bias_sm[S][4 * kq];                   // + 16i
        v8i b[4];
        float s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b[j] = nibbles_to_fp8(lds_load<i32x4>(wbase + j * 1024));
          s4[j] = sl.sc[wave][16 * j + col];
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          if (2 * ii < nsub) {
#pragma unroll
            for (int i = 2 * ii; i < 2 * ii + 2; ++i) {
              const i32x4 x0 = lds_load<i32x4>(abase + i * 2048);
              const i32x4 x1 = lds_load<i32x4>(abase + i * 2048 + 1024);
              const v8i av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
              const v4f cb = lds_load<v4f>(bbase + 16 * i);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const v4f d = mfma16x16x128(av, b[j], cb);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(s4[j], d[r], acc[i][j][r]);
              }
            }
          }
        }
      }
      // this wave's LDS writes done and group g+2 landed (only the 9 loads of
      // group g+3 may stay in flight), then the other waves' parts
      if (g + 3 < G) __builtin_amdgcn_s_waitcnt(0x0079);   // vmcnt(9) lgkmcnt(0)
      else __builtin_amdgcn_s_waitcnt(0);
      barrier_loads_in_flight();
    };

    // prologue: groups 0..2 in flight, group 0 landed and its row sums shared
    stage(std::integral_constant<int, 0>{}, 0);
    if (G > 1) stage(std::integral_constant<int, 1>{}, 1);
    if (G > 2) stage(std::integral_constant<int, 2>{}, 2);
    __builtin_amdgcn_s_waitcnt(0);
    barrier_loads_in_flight();
    row_sums(std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(0);
    barrier_loads_in_flight();

    for (int g = 0; g < G; g += kStages) {
      step(std::integral_constant<int, 0>{}, g);
      step(std::integral_constant<int, 1>{}, g + 1);
      step(std::integral_constant<int, 2>{}, g + 2);
      step(std::integral_constant<int, 3>{}, g + 3);
    }

    if (active) {
      // the lane's first output row; opaque to the optimizer so that the 32
      // row indices below are formed here rather than kept live in registers
      // through the whole kernel
      int row4 = 4 * kq;
      asm volatile("" : "+v"(row4));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < nsub) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rl = 16 * i + row4 + r;
            if (rl < mlen) {
              const int p = r0 + rl;
              const float rs = a_scale[a_rows ? a_rows[p] : p] * kUnitScale;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                __builtin_nontemporal_store(acc[i][j][r] * rs, out + (int64_t)p * N + n0 + 16 * j + col);
            }
          }
        }
      }
    }
  }
}

static int cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                hipSuccess && v > 0)
      cus = v;
    else
      cus = 256;
  }
  return cus;
}

hipError_t launch_gg_tiled(const GemmArgs& g, hipStream_t stream) {
  // the tiled kernel addresses its operands with 32-bit byte offsets
  constexpr int64_t k4G = (int64_t)1 << 32;
  if (g.M_total * g.K >= k4G || g.N * (g.K / 2) >= k4G || g.N * (g.K / 128) * 4 >= k4G)
    return launch_gg_stream(g, stream);
  hipLaunchKernelGGL(gg_tiled_kernel, dim3(cu_count()), dim3(kTiledThreads), 0, stream, g.a, g.a_scale,
                     g.a_rows, g.offsets, g.E, g.w_packed, g.w_scale, g.N, g.K, g.out);
  return hipGetLastError();
}

}  // namespace w4a8
