// Grouped W4A8 GEMM, tiled form: for many rows per expert (prefill).
//
// A persistent kernel (one workgroup of 8 waves per CU) walks the ragged
// list of tiles of all experts.  An expert's rows are cut into M blocks of
// equal height (rows / n, rounded): n = ceil(rows / 256) square ones, tiled by
// 256 output columns, or n = ceil(rows / 128) wide ones, tiled by 512 columns
// (at most 128 rows: half as many tiles per M block for the same weight bytes),
// whichever shape fills its tiles better (see square_mblocks).  Equal
// heights matter: the tiles that read the same weight columns, or the same
// activation rows, run at the same speed and stay in step through K, so the
// XCD's L2 serves the shared bytes to all of them.  With a full tile and a
// short remainder tile the remainder ran ahead, and its weight reads, then the
// full tile's, missed the L2 (2.4 GB more L2 misses per prefill launch).
//   square: wave w = 4 rg + cg owns the columns 64 cg .. +63 and the 16-row
//           A blocks rg, rg + 2, .., rg + 14 (interleaved, so that a short
//           tile still splits its rows over both row groups);
//   wide:   wave w owns the columns 64 w .. +63 and the A blocks 0 .. 7.
// Either way a wave computes up to 8 A blocks x 4 B blocks of 16x16x128
// products per K group, one MFMA each.
//
// K is walked one 128-wide group at a time through a 3-slot LDS ring (48 KB
// per slot) filled by direct global-to-LDS loads, two groups ahead.  Per group
// a slot holds the activation rows (FP8 codes, gathered through a_rows: 128
// bytes per row, 8 rows per load instruction) and then the weight columns (64
// packed bytes each, 16 columns per instruction).  The 16-byte chunks of a row
// or column are XOR-swizzled so that the MFMA operand reads are free of LDS
// bank conflicts.  The group scales of the tile's columns have a 3-slot ring
// of their own (one 4-byte load per column and group).
//
// Within a group the products are software-pipelined over the A blocks:
// the MFMAs of block i are issued between the group-scale FMAs of block i - 1
// (acc += s * D, one FMA per output), and the LDS reads of block i + 1 are in
// flight meanwhile.  The tile body is compiled for 0, 1, 2 and 4 to 8 blocks per
// wave, so that the hot loop has no per-block branches.
//
// The +8 offset of the uint4b8 nibbles is removed with the per-row sums of
// the activation codes of each group (see gemm_common.hpp): each wave loads
// exactly the activation rows whose sums it computes, with 16x16x128 MFMAs
// against the constant -2^-6, so the sums of group g + 1 are computed after
// the last A block of group g's products, once the wave's own loads of g + 1
// have landed, and are published by the one barrier per group.  They enter
// each product as its accumulator input.  Waiting there rather than halfway
// through the group leaves the loads nearly two groups of time to land: the
// kernel is bound by their latency (with the in-loop loads taken out, as a
// timing experiment, the gate/up GEMM ran 21% faster; without the scale FMAs
// and nibble splits, 5%).
//
// The weights come in the GEMM storage (16 columns x 128 K contiguous, scales
// group-major), so each weight load reads one contiguous 1 KB piece and each
// scale load 256 contiguous bytes: whole cache lines, where a row-major layout
// reads half a line per column and group and a line per scale word.
//
// MXFP4 weights (group 32) use the same ring: 64 packed bytes per column and
// group, and one 4-byte word of E8M0 scales per column and group (the four
// 32-element blocks of the group) in place of the fp32 group scale.  The matrix core applies the block scales itself, so the
// group's products accumulate straight into acc (no scale FMAs, no row sums:
// E2M1 is signed), the weight bytes are the B operand as they are, and the A
// operand is read as the 16-byte chunks q and q + 4 that the FP4 form of the
// instruction pairs with B's K quarter q.
//
// Tile order: an expert's square tiles go in groups of up to kGroupM = 4 M
// blocks; each group walks the expert's 256-column blocks in order, with its M
// blocks adjacent (one or two M blocks per expert, as at uniform prefill:
// column block by column block).  Wide tiles go by 512-column block.  Each
// XCD runs windows of 32 consecutive tiles at the same time, so a window of a
// hot expert covers about 4 M blocks x 8 column blocks: 4 activation blocks
// and 8 weight blocks, fetched from HBM about once and served to the other
// tiles of the window by that XCD's L2.  (Walking all M blocks of a column
// block first made every window read 32 activation blocks for one weight
// block: 15.9 GB of HBM traffic for the gate/up launch of a 16K-token prefill
// whose hottest expert has 15.9K rows, against 4.1 GB of algorithmic bytes.)
#include "gemm_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace w4a8 {

constexpr int kTM = 256;              // rows of a square tile
constexpr int kTN = 256;              // columns of a square tile
constexpr int kWideRows = 128;        // rows of a wide tile (the most a remainder has)
constexpr int kWideCols = 512;        // columns of a wide tile
constexpr int kMaxExperts = 1024;
constexpr int kGroupM = 4;            // M blocks per group in an expert's tile order
constexpr int kXcds = 8;              // accelerator complex dies of an MI355X (round-robin dispatch)
constexpr int kWaves = 8;             // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kABlocks = 8;           // 16-row A blocks per wave (at most)
constexpr int kBBlocks = 4;           // 16-column B blocks per wave
constexpr int kSlotBytes = kTM * kGroup + kTN * kGroup / 2;   // 48 KB: either tile shape's group
static_assert(kSlotBytes == kWideRows * kGroup + kWideCols * kGroup / 2, "slot sizes");

// One ring slot: the activation rows of one group, then its weight columns
// (column n of a 16-column load is at 64 n of its 1 KB piece in HBM).
//   a: row r, 16-byte chunk c (K bytes 16c..16c+15 of the group) at r*128 + 16*(c ^ swz_a(r))
//   w: column n, chunk c (packed bytes 16c..16c+15) at W + n*64 + 16*(c ^ swz_w(n)),
//      W = 256 * 128 (square tile) or 128 * 128 (wide tile)
// The three slots are separate LDS variables addressed with compile-time
// slot numbers, so that the compiler can tell the slot being read from the
// slots still being filled.
struct __attribute__((aligned(16))) RingSlot {
  uint8_t b[kSlotBytes];
};

// The swizzles.  A 16-byte LDS read of a wave is served a few lanes at a time:
// 8 lanes per cycle over 32 four-byte banks, or 16 lanes over 64 banks.  The
// operand reads have lane l read row (or column) l % 16 of a block at one chunk
// position, so the chunk slots of those rows must spread over the banks in
// either case:
//   rows (128 bytes apart): the slots of rows 0..7 and of rows 8..15 are all
//     different (8 lanes, 32 banks), and so are those of the even rows and of
//     the odd rows (16 lanes, 64 banks: rows 2i and 2i + 1 sit 32 banks apart);
//   columns (64 bytes apart, 4 slots): (n mod 2, slot) differs among columns
//     0..7 and among 8..15, and (n mod 4, slot) among 0..15.
// Both depend on the row or column modulo 16 only.
__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_w(int n) { return ((n >> 2) ^ (n >> 1)) & 3; }

template <int S, typename T>
__device__ __forceinline__ T& slot(T& r0, T& r1, T& r2) {
  if constexpr (S == 0) return r0;
  else if constexpr (S == 1) return r1;
  else return r2;
}

// Workgroup barrier that leaves direct-to-LDS loads in flight (__syncthreads'
// release fence would wait for all of them).  The caller waits for what the
// other waves need; the empty asm statements keep the compiler from moving
// memory accesses across.
__device__ __forceinline__ void barrier_loads_in_flight() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// buffer resource of a byte range (gfx9 dword 3: raw, untyped access)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// LDS byte address of a pointer into a __shared__ variable
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Direct loads into LDS: lane l's bytes (at rsrc + voff + soff) go to lds + size * l
// (M0 holds the wave's LDS base).  They are issued from inline assembly, which the
// compiler does not see as writing LDS: given the builtin, its wait insertion cannot
// always tell the ring slot being filled from the one being read, and adds a full
// vmcnt(0) before the group's LDS reads, which drains the prefetch.  The kernel orders
// these loads itself: its own vmcnt waits, then the barrier, before any wave reads
// the slot.  They write no register, so nothing the compiler allocates is in flight.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr(lds)), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}

template <typename T>
__device__ __forceinline__ T lds_load(const void* p) {
  return *reinterpret_cast<const T*>(__builtin_assume_aligned(p, 16));
}

// tiles of an expert with `rows` rows: M blocks of equal height, either
// ceil(rows / 256) square ones (per 256-column block) or ceil(rows / 128) wide
// ones (per 512 columns), whichever fills its tiles better.  Wide when
// rows mod 256 is 1..128 (and for 1..128 rows): 280 rows make three wide M
// blocks of 93-94 rows (24 tiles of 6 A blocks per wave at N = 4096) where two
// square ones of 140 rows ran 32 tiles of 5 blocks and loaded 256 activation
// rows per tile for 140.
__device__ __forceinline__ int square_mblocks(int rows) {
  if (rows <= kWideRows) return 0;
  const int nsq = (rows + kTM - 1) / kTM, nwide = (rows + kWideRows - 1) / kWideRows;
  return nwide < 2 * nsq ? 0 : nsq;
}
__device__ __forceinline__ int wide_mblocks(int rows) {
  return rows > 0 && square_mblocks(rows) == 0 ? (rows + kWideRows - 1) / kWideRows : 0;
}
__device__ __forceinline__ int tiles_of(int rows, int nb, int nw) {
  return square_mblocks(rows) * nb + wide_mblocks(rows) * nw;
}
// Relative cost of one tile of an expert with `rows` rows: the A blocks per wave of
// the body its tallest M block runs, plus 2 for the work of each K group that does not
// grow with them (barrier, row sums, load issue).  3..10 for an expert with rows.
constexpr int kMaxTileCost = 10;
__device__ __forceinline__ int tile_cost(int rows) {
  const int msq = square_mblocks(rows);
  const int nm = msq > 0 ? msq : wide_mblocks(rows);
  if (nm == 0) return 0;
  const int mb16 = ((rows + nm - 1) / nm + 15) >> 4;
  const int nact = min(kABlocks, msq > 0 ? (mb16 + 1) >> 1 : mb16);
  const int body = nact > 4 ? nact : (msq > 0 || nact > 2) ? 4 : nact;
  return body + 2;
}
// an entry of the tile list: the first tile of an expert above the expert's index
constexpr int kExpertBits = 10;                      // kMaxExperts = 1024
constexpr int kExpertMask = (1 << kExpertBits) - 1;
constexpr int kMaxTiles = 1 << (31 - kExpertBits);  // tile numbers that fit an entry

// kForm: kFormG128, the group-128 FP8 form; kFormChannel, the per-channel
// variant (INT8 activations with row code sums a_rowsum, one scale per weight
// row in w_scale [E][N]): int32 products accumulated by the matrix core over
// all of K, no group scales, no row-sum MFMAs; kFormMx, MXFP4 weights (w_scale
// holds the E8M0 bytes).
// kSwiglu: the fused gate/up form: tile column v multiplies weight row
// gate_up_row(v), so a wave's B blocks 2 jp and 2 jp + 1 are the gate and the
// up rows of the same 16 output columns; the epilogue writes
// act = silu(gate) * up [M][N/2] and the tile's max |act| of each row to
// pmax[p][s] for the slots s of 64 output columns the tile covers.
// kScatter (plain form only): row p of the result is stored as row
// out_rows[p] of out (the down GEMM writing token-major rows).
template <int kForm, bool kSwiglu, bool kScatter = false>
__global__ __launch_bounds__(kThreads, 1) void gg_tiled_kernel(const uint8_t* __restrict__ a,
                                                               const float* __restrict__ a_scale,
                                                               const int32_t* __restrict__ a_rowsum,
                                                               const int32_t* __restrict__ a_rows,
                                                               const int32_t* __restrict__ offsets, int E,
                                                               const int32_t* __restrict__ w_packed,
                                                               const float* __restrict__ w_scale, int64_t N,
                                                               int64_t K, float* __restrict__ out,
                                                               float* __restrict__ pmax, int sel_rows,
                                                               const int32_t* __restrict__ out_rows) {
  constexpr bool kInt8 = kForm == kFormChannel;
  constexpr bool kMx = kForm == kFormMx;
  __shared__ RingSlot ring0, ring1, ring2;
  __shared__ __attribute__((aligned(16))) float sc0[kWideCols], sc1[kWideCols], sc2[kWideCols];   // group scales (MX: E8M0 words)
  __shared__ __attribute__((aligned(16))) float bias_sm[2][kTM];   // -2^-6 * group code sums: [group parity][row]
  __shared__ __attribute__((aligned(16))) float ascale_sm[kTM];    // token scales of the tile's rows
  __shared__ int tile_start[kMaxExperts + 1];                      // the tile list: (first tile << 10) | expert
  __shared__ int wscan[2][2][kWaves], wmax[kWaves];
  __shared__ unsigned int rmax_sm[2][kTM];                         // fused form: row max |act| of the tile, by tile parity
  __shared__ __attribute__((aligned(16))) int dst_sm[kScatter ? kTM : 4];   // scatter form: the rows of out

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps wave-indexed values scalar
  const int lr = lane & 15, lq = lane >> 4;                    // 16x16x128 lane roles: row/column, K quarter
  const int NB = (int)((N + kTN - 1) / kTN);                   // 256-column blocks
  const int NW = (NB + 1) / 2;                                 // 512-column blocks
  const int G = (int)(K >> 7);
  const uint32_t row_bytes = (uint32_t)(K >> 1);
  const int half = (int)(N >> 1);                              // output columns of the fused form
  int* rowsum_sm = reinterpret_cast<int*>(&bias_sm[0][0]);   // the INT8 form has no group sums: row code sums

  // ---- tile numbering.  In the fused gate/up form the experts with rows go in
  // order of their tile cost, dearest first (ties by index), so that the last,
  // partial round of tiles holds the cheapest ones: with 20.1 rounds of 256
  // tiles at prefill T=8192, the workgroups that run one tile more end that
  // much later than the rest (measured 2.5-4% off that GEMM at prefill).  The
  // other forms keep the experts in index order: the same ordering made the
  // down GEMM 2-9% slower.  Entry i of tile_start is the i-th expert's first
  // tile number above its index; one block-wide scan per cost class numbers
  // the class's tiles and entries (a single class in index order).
  int n_list = 0;                                   // experts with rows (entries of the list)
  {
    constexpr int kPer = kMaxExperts / kThreads;   // experts per thread
    int cnt[kPer], cst[kPer];
    int most = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ex = tid * kPer + i;
      const int rows = ex < E ? offsets[ex + 1] - offsets[ex] : 0;
      cnt[i] = tiles_of(rows, NB, NW);
      cst[i] = tile_cost(rows);
      most = max(most, rows);
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) most = max(most, __shfl_xor(most, off, kWave));
    if (lane == 0) wmax[wave] = most;
    __syncthreads();
    // the choice on the device: nothing to do when the stream kernel takes the batch
    if (sel_rows >= 0) {
      int top = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) top = max(top, wmax[w]);
      if (top <= sel_rows) return;
    }
    int tile_base = 0;                              // tiles and entries of the dearer classes
    if constexpr (!kSwiglu) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) cst[i] = 1;
    }
    for (int c = kSwiglu ? kMaxTileCost : 1; c >= 1; --c) {
      int lt = 0, ln = 0;                           // this thread's tiles and experts of class c
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (cnt[i] > 0 && cst[i] == c) {
          lt += cnt[i];
          ++ln;
        }
      int it = lt, in = ln;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int ot = __shfl_up(it, off, kWave), on = __shfl_up(in, off, kWave);
        if (lane >= off) {
          it += ot;
          in += on;
        }
      }
      // two buffers by class parity: a wave writing one has passed the barrier
      // after which every wave read it last
      int (&buf)[2][kWaves] = wscan[c & 1];
      if (lane == kWave - 1) {
        buf[0][wave] = it;
        buf[1][wave] = in;
      }
      __syncthreads();
      int bt = 0, bn = 0, tt = 0, tn = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (w < wave) {
          bt += buf[0][w];
          bn += buf[1][w];
        }
        tt += buf[0][w];
        tn += buf[1][w];
      }
      int t0 = tile_base + bt + it - lt, s0 = n_list + bn + in - ln;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (cnt[i] > 0 && cst[i] == c) {
          tile_start[s0++] = (t0 << kExpertBits) | (tid * kPer + i);
          t0 += cnt[i];
        }
      tile_base += tt;
      n_list += tn;
    }
    if (tid == 0) tile_start[n_list] = tile_base << kExpertBits;   // the grand total
    __syncthreads();
  }
  const int total = tile_start[n_list] >> kExpertBits;

  // lane-constant parts of the swizzled LDS addresses (the row or column
  // bases of the blocks are multiples of 16, so the swizzle depends on lr only);
  // the A operand's two 16-byte chunks: 2 lq and 2 lq + 1 (K bytes 32 lq .. +31),
  // in the MX form lq and lq + 4
  const int fa = swz_a(lr);                       // activation swizzle of row 16 b + lr
  const int ca0 = kMx ? lq : 2 * lq, ca1 = kMx ? lq + 4 : 2 * lq + 1;
  const uint32_t a_rd0 = (uint32_t)lr * kGroup + 16u * (uint32_t)(ca0 ^ fa);
  const uint32_t a_rd1 = (uint32_t)lr * kGroup + 16u * (uint32_t)(ca1 ^ fa);
  const uint32_t w_rd_lane = (uint32_t)lr * 64u + 16u * (uint32_t)(lq ^ swz_w(lr));

  // Tile t runs on the XCD and in the round that keep data sharing local:
  // workgroups are dispatched round-robin over the XCDs, so workgroup w sits
  // on XCD w % X.  Each round hands the X XCDs consecutive windows of grid/X
  // tiles.
  const int grid = gridDim.x;
  const bool xcd_windows = (grid % kXcds) == 0;
  const int window = grid / kXcds;
  const int my_slot = xcd_windows ? (int)(blockIdx.x % kXcds) * window + (int)(blockIdx.x / kXcds) : (int)blockIdx.x;
  int tpar = 0;                                                    // parity of this workgroup's tile count
  for (int t = my_slot; t < total; t += grid, tpar ^= 1) {
    // ---- which expert, and which tile of it
    int lo_e = 0, hi_e = n_list;               // entry lo_e: first tile <= t < the next entry's
    while (hi_e - lo_e > 1) {
      const int mid = (lo_e + hi_e) >> 1;
      if ((tile_start[mid] >> kExpertBits) <= t) lo_e = mid; else hi_e = mid;
    }
    const int entry = __builtin_amdgcn_readfirstlane(tile_start[lo_e]);
    const int e = entry & kExpertMask;
    const int r_e = offsets[e], rows_e = offsets[e + 1] - r_e;
    const int msq = square_mblocks(rows_e);    // 0: the expert has wide tiles only
    const int local = t - (entry >> kExpertBits);
    // tile (mb, nb) of the expert's M blocks and column blocks (square: 256 columns,
    // wide: 512): the M blocks in groups of kGroupM, each group walking the column
    // blocks with its M blocks adjacent
    const bool is_wide = msq == 0;
    const int nm = is_wide ? wide_mblocks(rows_e) : msq;
    const int ncb = is_wide ? NW : NB;
    const int mg = local / (kGroupM * ncb);
    const int gm0 = mg * kGroupM, gsz = min(kGroupM, nm - gm0);
    const int rr = local - mg * kGroupM * ncb;
    const int nb = rr / gsz, mb = gm0 + (rr - nb * gsz);
    // M block mb of nm: rows_e / nm rows, the first rows_e % nm blocks one more
    const int base = rows_e / nm, extra = rows_e - base * nm;
    const int r0 = r_e + mb * base + min(mb, extra);
    const int mlen = base + (mb < extra ? 1 : 0);
    const int n0 = nb * (is_wide ? kWideCols : kTN);

    // The rest of the tile (K loop and epilogue) is compiled per tile shape
    // and per number kNB of A blocks of the wave (0, 1, 2, 4, 5, 6, 7 or 8), without
    // branches between the blocks; a wave with nact blocks holding rows runs
    // the smallest kNB >= nact (the blocks past nact multiply clamped rows,
    // which the epilogue drops).
    auto run_tile = [=](auto W_, auto NB_) mutable {
      constexpr bool kWide = decltype(W_)::value;
      constexpr int kNB = decltype(NB_)::value;
      constexpr int kRows = kWide ? kWideRows : kTM;       // rows of the tile
      constexpr int kCols = kWide ? kWideCols : kTN;       // columns of the tile
      constexpr int kARows = kRows / kWaves;               // activation rows each wave loads (and sums)
      constexpr int kWCols = kCols / kWaves;               // weight columns each wave loads
      constexpr int kALoads = kARows / 8, kWLoads = kWCols / 16;
      constexpr uint32_t kWBase = kRows * kGroup;          // weight columns' offset in a slot
      constexpr int kBlockStride = kWide ? 16 : 32;        // rows between a wave's A blocks
      const int rg = kWide ? 0 : wave >> 2;                // row group (its first A block)
      const int cg = kWide ? wave : wave & 3;              // column group (64 columns)
      // this wave's group scales: columns 64 sw + lane (the per-group forms).  Square
      // tiles have 256 columns: waves 4..7 repeat the loads of waves 0..3 (the same
      // bytes to the same LDS words), so that every wave issues the same loads per
      // stage and the K loop waits with one constant count, without branches.
      constexpr bool kScales = !kInt8;
      const int sw = kWide ? wave : (wave & 3);

      // ---- direct-load roles of this lane
      // activations: rows kARows wave + 8 q + lane / 8, chunk position lane % 8
      const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a, 0xffffffffu);
      uint32_t aoff[kALoads];
#pragma unroll
      for (int q = 0; q < kALoads; ++q) {
        const int r = kARows * wave + 8 * q + (lane >> 3);
        const int p = r0 + min(r, mlen - 1);
        const int c = (lane & 7) ^ swz_a(r);
        aoff[q] = (uint32_t)(a_rows ? a_rows[p] : p) * (uint32_t)K + 16u * (uint32_t)c;
      }
      // weights: columns kWCols wave + 16 q + lane / 4 of the tile, chunk position lane % 4:
      // load q reads the 1 KB piece of its 16 weight rows and the group (the piece's base
      // goes into the scalar offset; fused form: rows gate_up_row(vb + 16 q) .. +15).
      // Columns n and n + 16 q have the same swizzle, so one lane offset serves every q.
      // N % 64 == 0, so a wave's columns are either all below N or all past it; a wave
      // past N reads rows from 0, unused.
      const __amdgpu_buffer_rsrc_t rw =
          buffer_rsrc(reinterpret_cast<const uint8_t*>(w_packed) + (int64_t)e * N * row_bytes, (uint32_t)N * row_bytes);
      const int vb = n0 + kWCols * wave < N ? n0 + kWCols * wave : 0;
      const uint32_t woff = (uint32_t)(lane >> 2) * 64u + 16u * (uint32_t)((lane & 3) ^ swz_w(lane >> 2));
      // group scales: the words of group g of all N columns are contiguous
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w_scale + (int64_t)e * N * G, (uint32_t)(N * G * 4));
      const int scol = min(n0 + 64 * sw + lane, (int)N - 1);
      const uint32_t soff = (uint32_t)(kSwiglu ? gate_up_row(scol, half) : scol) * 4u;
      const uint32_t sstep = (uint32_t)N * 4u;    // scale offset step per group

      // The K loop issues a stage in two parts: the group scales and weight columns at the start of
      // the step, the activation rows after the products of its first A block (or two).  Issuing
      // everything right after the barrier, as every CU does at about the same moment, made the
      // loads wait longer: the split took 2-4% off the MX and INT8 GEMMs at prefill (the group-128
      // form, which waits later, was unchanged).
      auto stage_a = [&](auto S_, int g) {
        constexpr int S = decltype(S_)::value;
        RingSlot& sl = slot<S>(ring0, ring1, ring2);
#pragma unroll
        for (int q = 0; q < kALoads; ++q)
          dma16(ra, aoff[q], (uint32_t)g * kGroup, &sl.b[(kARows * wave + 8 * q) * kGroup]);
      };
      auto stage_w = [&](auto S_, int g) {
        constexpr int S = decltype(S_)::value;
        RingSlot& sl = slot<S>(ring0, ring1, ring2);
        if constexpr (kScales) dma4(rs, soff, (uint32_t)g * sstep, &slot<S>(sc0, sc1, sc2)[64 * sw]);
#pragma unroll
        for (int q = 0; q < kWLoads; ++q) {
          const int v = kSwiglu ? gate_up_row(vb + 16 * q, half) : vb + 16 * q;   // first weight row of load q
          dma16(rw, woff, ((uint32_t)(v >> 4) * (uint32_t)G + (uint32_t)g) * 1024u,
                &sl.b[kWBase + (kWCols * wave + 16 * q) * 64]);
        }
      };
      // all loads of group g into slot S (the prologue)
      auto stage = [&](auto S_, int g) {
        stage_w(S_, g);
        stage_a(S_, g);
      };
      // wait until only the loads of the group issued last are in flight
      auto wait_last_stage = [&]() {
        constexpr int kStage = kALoads + kWLoads + (kScales ? 1 : 0);   // loads per stage
        static_assert(kStage <= 15, "vmcnt field");
        __builtin_amdgcn_s_waitcnt(0x0F70 | kStage);
      };
      // -2^-6 * (sum of the activation codes) of this wave's rows for the group in slot S
      auto row_sums = [&](auto S_, int g) {
        const RingSlot& sl = slot<decltype(S_)::value>(ring0, ring1, ring2);
#pragma unroll
        for (int q = 0; q < kARows / 16; ++q) {
          const i32x4 x0 = lds_load<i32x4>(&sl.b[(kARows * wave + 16 * q) * kGroup + a_rd0]);
          const i32x4 x1 = lds_load<i32x4>(&sl.b[(kARows * wave + 16 * q) * kGroup + a_rd1]);
          const v8i av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          const v4f c = mfma16x16x128(av, bias_operand(), v4f{0.f, 0.f, 0.f, 0.f});
          if (lr == 0) *reinterpret_cast<v4f*>(&bias_sm[g & 1][kARows * wave + 16 * q + 4 * lq]) = c;
        }
      };

      // where the wait for group g+1 goes: the group-128 form after the last A block
      // (7% faster gate/up at prefill than halfway); the MX and INT8 forms halfway,
      // where they were 2-5% faster (the later wait made the MX form spill)
      constexpr int kWaitRegion = (kInt8 || kMx) ? (kNB - 1) / 2 : kNB - 1;
      using Acc = std::conditional_t<kInt8, i32x4, v4f>;
      Acc acc[kNB > 0 ? kNB : 1][kBBlocks];
#pragma unroll
      for (int i = 0; i < (kNB > 0 ? kNB : 1); ++i)
#pragma unroll
        for (int j = 0; j < kBBlocks; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = 0;
      // group-128 form: the last A block's products of a group and their group scales, scaled
      // into acc at the start of the next group (after its barrier, while its first LDS reads are
      // in flight) rather than before the barrier; zero before the first group
      v4f c_pend[kBBlocks];
      float s_pend[kBBlocks];
#pragma unroll
      for (int j = 0; j < kBBlocks; ++j) {
        s_pend[j] = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) c_pend[j][v] = 0.0f;
      }
      auto apply_pending = [&]() {
        if constexpr (!kInt8 && !kMx && kNB > 0) {
#pragma unroll
          for (int j = 0; j < kBBlocks; ++j) {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[kNB - 1][j][v] = fmaf(s_pend[j], c_pend[j][v], acc[kNB - 1][j][v]);
            asm volatile("" : "+v"(acc[kNB - 1][j]));
          }
        }
      };
      const uint32_t a_blk0 = (uint32_t)(16 * rg) * kGroup;             // first A block of the wave
      const uint32_t w_rd = kWBase + (uint32_t)(64 * cg) * 64u + w_rd_lane;

      // One K group in slot S: prefetch group g+2; multiply group g; after the
      // last A block's products (MX and INT8 forms: halfway through them), once
      // this wave's loads of group g+1 have landed, publish that group's row sums;
      // then one barrier.  kMore: groups g+1 and g+2
      // exist (the main part of the K loop), so the step has no branches: with a
      // branch around the wait, the compiler moved earlier products below it.
      auto step = [&](auto S_, auto M_, int g) {
        constexpr int S = decltype(S_)::value;
        constexpr bool kMore = decltype(M_)::value;
        if (!kMore && g >= G) return;
        const bool more = kMore || g + 2 < G;
        // scales of group g (MX: the E8M0 byte of the lane's K quarter, in byte 0)
        float s[kBBlocks];
        int sb[kBBlocks];
        if constexpr (kMx) {
#pragma unroll
          for (int j = 0; j < kBBlocks; ++j)
            sb[j] = (int)(__float_as_uint(slot<S>(sc0, sc1, sc2)[64 * cg + 16 * j + lr]) >> (8 * lq));
        } else if constexpr (!kInt8) {
#pragma unroll
          for (int j = 0; j < kBBlocks; ++j) s[j] = slot<S>(sc0, sc1, sc2)[64 * cg + 16 * j + lr];
        }
        if (more) stage_w(std::integral_constant<int, (S + 2) % 3>{}, g + 2);
        const RingSlot& sl = slot<S>(ring0, ring1, ring2);
        // this wave's loads of group g+1 landed (only those of group g+2 may stay
        // in flight); then the row sums of group g+1
        auto mid = [&]() {
          if (more) wait_last_stage();
          else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
          if (!kInt8 && !kMx && (kMore || g + 1 < G)) row_sums(std::integral_constant<int, (S + 1) % 3>{}, g + 1);
        };
        // the products of this group: kNB A blocks x kBBlocks B blocks
        auto compute = [&]() {
          v8i b[kBBlocks];
          i32x4 bx[kBBlocks];   // the packed bytes (MX: the operand as it is)
#pragma unroll
          for (int j = 0; j < kBBlocks; ++j) bx[j] = lds_load<i32x4>(&sl.b[w_rd + j * 16 * 64]);
          if constexpr (!kInt8 && !kMx) {
            __builtin_amdgcn_sched_barrier(0);
            apply_pending();
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (!kMx) {
#pragma unroll
            for (int j = 0; j < kBBlocks; ++j) b[j] = nibbles_to_fp8(bx[j]);
          }
          const float* bsum = &bias_sm[g & 1][16 * rg + 4 * lq];
          // operands of A block i: two 16-byte halves of the lane's 32 K bytes
          auto load_a = [&](int i) {
            const uint8_t* ab = &sl.b[a_blk0 + (uint32_t)(kBlockStride * i) * kGroup];
            const i32x4 x0 = lds_load<i32x4>(ab + a_rd0);
            const i32x4 x1 = lds_load<i32x4>(ab + a_rd1);
            return v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          };
          v8i av[2];
          v4f bias[2];
          v4f c[kBBlocks];   // products of the block in flight; each is scaled into acc just before it is reused
          av[0] = load_a(0);
          if constexpr (!kInt8 && !kMx) bias[0] = lds_load<v4f>(bsum);
          auto scale_into = [&](auto I_, int j) {   // acc[i] += s * D for B block j
            constexpr int i = decltype(I_)::value;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(s[j], c[j][v], acc[i][j][v]);
            asm volatile("" : "+v"(acc[i][j]));   // the FMAs stay here: sunk later they would hold c live
          };
          // region i: the products of A block i, each right after the group
          // scale of block i - 1 has been applied to the same B block (the
          // matrix core runs block i while the VALU scales block i - 1); the LDS
          // reads of block i + 1 are issued first
          auto region = [&](auto I_) {
            constexpr int i = decltype(I_)::value;
            if constexpr (i < kNB) {
              if constexpr (i + 1 < kNB) {
                av[(i + 1) & 1] = load_a(i + 1);
                if constexpr (!kInt8 && !kMx) bias[(i + 1) & 1] = lds_load<v4f>(bsum + kBlockStride * (i + 1));
              }
#pragma unroll
              for (int j = 0; j < kBBlocks; ++j) {
                if constexpr (kMx) {
                  acc[i][j] = mfma_mx(av[i & 1], bx[j], acc[i][j], sb[j]);
                } else if constexpr (kInt8) {
                  const v8i x = av[i & 1];
                  const i32x4 a_lo = {x[0], x[1], x[2], x[3]}, a_hi = {x[4], x[5], x[6], x[7]};
                  const i32x4 b_lo = {b[j][0], b[j][1], b[j][2], b[j][3]}, b_hi = {b[j][4], b[j][5], b[j][6], b[j][7]};
                  acc[i][j] = mfma_i8_16x16x64(a_lo, b_lo, acc[i][j]);
                  acc[i][j] = mfma_i8_16x16x64(a_hi, b_hi, acc[i][j]);
                } else {
                  if constexpr (i >= 1) scale_into(std::integral_constant<int, i - 1>{}, j);
                  c[j] = mfma16x16x128(av[i & 1], b[j], bias[i & 1]);
                }
              }
            } else if constexpr (!kInt8 && !kMx && i == kNB && i >= 1) {
#pragma unroll
              for (int j = 0; j < kBBlocks; ++j) {
                c_pend[j] = c[j];
                s_pend[j] = s[j];
              }
            }
            __builtin_amdgcn_sched_barrier(0);   // regions stay in order: no hoisting of later reads
            if constexpr (i == ((kNB >= 2 && kWaitRegion >= 1) ? 1 : 0)) {   // before the wait, which counts them
              if (more) stage_a(std::integral_constant<int, (S + 2) % 3>{}, g + 2);
            }
            if constexpr (i == kWaitRegion) mid();
          };
          region(std::integral_constant<int, 0>{});
          region(std::integral_constant<int, 1>{});
          region(std::integral_constant<int, 2>{});
          region(std::integral_constant<int, 3>{});
          region(std::integral_constant<int, 4>{});
          region(std::integral_constant<int, 5>{});
          region(std::integral_constant<int, 6>{});
          region(std::integral_constant<int, 7>{});
          region(std::integral_constant<int, 8>{});
        };
        if constexpr (kNB > 0) compute();
        else { if (more) stage_a(std::integral_constant<int, (S + 2) % 3>{}, g + 2); mid(); }
        __builtin_amdgcn_s_waitcnt(0xC07F);                      // lgkmcnt(0): LDS writes done
        barrier_loads_in_flight();
      };

      // byte offsets of the token scales (and row code sums) of the tile's rows, read
      // here: a wait for them after the stages below would wait for those as well
      uint32_t asrc = 0;
      if (wave < kRows / 64) {
        const int p = r0 + min(64 * wave + lane, mlen - 1);
        asrc = (uint32_t)(a_rows ? a_rows[p] : p) * 4u;
      }
      asm volatile("" :: "v"(asrc));
      // prologue: groups 0 and 1 in flight, this wave's rows of group 0 landed, their sums published
      stage(std::integral_constant<int, 0>{}, 0);
      if (G > 1) {
        stage(std::integral_constant<int, 1>{}, 1);
        wait_last_stage();
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);
      }
      if (!kInt8 && !kMx) row_sums(std::integral_constant<int, 0>{}, 0);
      // the fused form's row maxima of this tile start at 0 (the previous use of this
      // parity's array, two tiles back, ended before the last tile's first barrier)
      if (kSwiglu && tid < kTM) rmax_sm[tpar][tid] = 0u;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      barrier_loads_in_flight();
      // the token scales (and in the INT8 form the row code sums) of the tile's
      // rows, read in the epilogue (every wave is past the previous epilogue); the
      // K loop's last step waits for every load, so they have landed by then
      if (wave < kRows / 64) {
        dma4(buffer_rsrc(a_scale, 0xffffffffu), asrc, 0, &ascale_sm[64 * wave]);
        if constexpr (kInt8) dma4(buffer_rsrc(a_rowsum, 0xffffffffu), asrc, 0, &rowsum_sm[64 * wave]);
        if constexpr (kScatter)   // the rows of out: p itself indexes out_rows (no load to wait for)
          dma4(buffer_rsrc(out_rows, 0xffffffffu), (uint32_t)(r0 + min(64 * wave + lane, mlen - 1)) * 4u, 0,
               &dst_sm[64 * wave]);
      }

      // MX and INT8 forms: three steps at a time while every step has a next stage,
      // then the last 2..4 groups (all of them when G < 5), whose slots start again
      // at 0.  The group-128 form keeps checked steps throughout: with its products
      // held before the wait it spills inside the K loop.
      if constexpr (kInt8 || kMx) {
        int g = 0;
        for (; g + 5 <= G; g += 3) {
          step(std::integral_constant<int, 0>{}, std::true_type{}, g);
          step(std::integral_constant<int, 1>{}, std::true_type{}, g + 1);
          step(std::integral_constant<int, 2>{}, std::true_type{}, g + 2);
        }
        step(std::integral_constant<int, 0>{}, std::false_type{}, g);
        step(std::integral_constant<int, 1>{}, std::false_type{}, g + 1);
        step(std::integral_constant<int, 2>{}, std::false_type{}, g + 2);
        step(std::integral_constant<int, 0>{}, std::false_type{}, g + 3);
      } else {
        for (int g = 0; g < G; g += 3) {
          step(std::integral_constant<int, 0>{}, std::false_type{}, g);
          step(std::integral_constant<int, 1>{}, std::false_type{}, g + 1);
          step(std::integral_constant<int, 2>{}, std::false_type{}, g + 2);
        }
      }

      apply_pending();   // the last group's last A block
      // ---- epilogue: D lane holds column lr of its B block, rows 4 lq .. +3 of its A block
      if constexpr (kNB > 0) {
        // lane roles taken afresh: addresses built from them are not hoisted out of the tile
        // loop, where they would live (and spill) across every K loop
        int lr = lane & 15, lq = lane >> 4;
        asm volatile("" : "+v"(lr), "+v"(lq));
        float ws[kBBlocks];
        if constexpr (kInt8) {
#pragma unroll
          for (int j = 0; j < kBBlocks; ++j) {
            const int v = n0 + 64 * cg + 16 * j + lr;
            ws[j] = w_scale[(int64_t)e * N + (kSwiglu ? gate_up_row(v, half) : v)];
          }
        }
#pragma unroll
        for (int i = 0; i < kNB; ++i) {
          if (16 * rg + kBlockStride * i < mlen) {
            const int rt = 16 * rg + kBlockStride * i + 4 * lq;
            const v4f sc4 = lds_load<v4f>(&ascale_sm[rt]);
            i32x4 rs4 = {0, 0, 0, 0};
            if constexpr (kInt8) rs4 = lds_load<i32x4>(&rowsum_sm[rt]);
            i32x4 dst4 = {0, 0, 0, 0};
            if constexpr (kScatter) dst4 = lds_load<i32x4>(&dst_sm[rt]);
            // the GEMM output of B block j and row v (the value the unfused form stores)
            auto h = [&](int j, int v) {
              if constexpr (kInt8) return (float)(acc[i][j][v] - 8 * rs4[v]) * sc4[v] * ws[j];
              else if constexpr (kMx) return acc[i][j][v] * sc4[v];
              else return acc[i][j][v] * (sc4[v] * kUnitScale);
            };
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              if constexpr (kSwiglu) {
                const bool ok = rt + v < mlen;
                float* orow = out + (int64_t)(r0 + rt + v) * half + (n0 + 64 * cg) / 2 + lr;
                float m = 0.0f;
#pragma unroll
                for (int jp = 0; jp < kBBlocks / 2; ++jp) {
                  const float y = silu_mul(h(2 * jp, v), h(2 * jp + 1, v));
                  if (ok) __builtin_nontemporal_store(y, orow + 16 * jp);
                  m = fmaxf(m, fabsf(y));
                }
                m = max16(ok ? m : 0.0f);
                if (ok && lr == 0) atomicMax(&rmax_sm[tpar][rt + v], __float_as_uint(m));
              } else if (rt + v < mlen) {
                const int64_t dp = kScatter ? dst4[v] : r0 + rt + v;   // the row of out
                float* orow = out + dp * N + n0 + 64 * cg + lr;
#pragma unroll
                for (int j = 0; j < kBBlocks; ++j) __builtin_nontemporal_store(h(j, v), orow + 16 * j);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);   // one block at a time: its outputs' temporaries stay few
        }
      }
      if constexpr (kSwiglu) {
        // the tile's row maxima (reduced in LDS over the waves' column groups), stored once per
        // 64-column slot of the tile (plain stores: no atomics, no zeroing of the output)
        __builtin_amdgcn_s_waitcnt(0xC07F);
        barrier_loads_in_flight();
        if (tid < kRows && tid < mlen) {
          const int slots = (int)(N >> 7), s0 = n0 >> 7;
          const float m = __uint_as_float(rmax_sm[tpar][tid]);
#pragma unroll
          for (int q = 0; q < kCols / 128; ++q)
            if (s0 + q < slots) pmax[(int64_t)(r0 + tid) * slots + s0 + q] = m;
        }
      }
    };
    // A blocks of this wave holding rows: wide tiles ceil(mlen / 16) (every
    // wave), square tiles those of rg + 2 i < ceil(mlen / 16); none if the
    // wave's 64 columns are past N (N % 64 == 0: a column group is wholly in
    // or out).  A square tile has at least 128 rows, so each of its waves
    // with columns has 4 to 8 blocks; a wide tile of an expert with more than
    // 128 rows has at least 85, so 6 to 8 (a variant for each count).
    const int mb16 = (mlen + 15) >> 4;
    if (is_wide) {
      const int nact = __builtin_amdgcn_readfirstlane(n0 + 64 * wave < N ? min(kABlocks, mb16) : 0);
      if (nact > 7) run_tile(std::true_type{}, std::integral_constant<int, 8>{});
      else if (nact == 7) run_tile(std::true_type{}, std::integral_constant<int, 7>{});
      else if (nact == 6) run_tile(std::true_type{}, std::integral_constant<int, 6>{});
      else if (nact == 5) run_tile(std::true_type{}, std::integral_constant<int, 5>{});
      else if (nact > 2) run_tile(std::true_type{}, std::integral_constant<int, 4>{});
      else if (nact == 2) run_tile(std::true_type{}, std::integral_constant<int, 2>{});
      else if (nact == 1) run_tile(std::true_type{}, std::integral_constant<int, 1>{});
      else run_tile(std::true_type{}, std::integral_constant<int, 0>{});
    } else {
      const int rg = wave >> 2, cg = wave & 3;
      const int nact = __builtin_amdgcn_readfirstlane(n0 + 64 * cg < N ? min(kABlocks, (mb16 - rg + 1) >> 1) : 0);
      if (nact > 7) run_tile(std::false_type{}, std::integral_constant<int, 8>{});
      else if (nact == 7) run_tile(std::false_type{}, std::integral_constant<int, 7>{});
      else if (nact == 6) run_tile(std::false_type{}, std::integral_constant<int, 6>{});
      else if (nact == 5) run_tile(std::false_type{}, std::integral_constant<int, 5>{});
      else if (nact > 0) run_tile(std::false_type{}, std::integral_constant<int, 4>{});
      else run_tile(std::false_type{}, std::integral_constant<int, 0>{});
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

bool tiled_fits(const GemmArgs& g) {
  // the tiled kernel addresses its operands with 32-bit byte offsets
  constexpr int64_t k4G = (int64_t)1 << 32;
  // and the tile numbers fit an entry of the tile list: at most M_total / 128 + E M blocks
  const int64_t tiles = (g.M_total / kWideRows + g.E + 1) * ((g.N + kTN - 1) / kTN);
  return g.M_total * g.K < k4G && g.M_total * 4 < k4G && g.N * (g.K / 2) < k4G && g.N * (g.K / 128) * 4 < k4G &&
         tiles < kMaxTiles;
}

hipError_t launch_gg_tiled(const GemmArgs& g, hipStream_t stream) {
  if (!tiled_fits(g)) {
    GemmArgs all = g;
    all.sel_rows = -1;
    return launch_gg_stream(all, stream);
  }
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(cu_count()), dim3(kThreads), 0, stream, g.a, g.a_scale, g.a_rowsum, g.a_rows,
                       g.offsets, g.E, g.w_packed, g.w_scale, g.N, g.K, g.out, g.pmax, (int)g.sel_rows,
                       g.out_rows);
  };
  if (g.pmax) {
    if (g.a_rowsum) go(gg_tiled_kernel<kFormChannel, true>);
    else if (g.mx) go(gg_tiled_kernel<kFormMx, true>);
    else go(gg_tiled_kernel<kFormG128, true>);
  } else if (g.out_rows) {
    if (g.a_rowsum) go(gg_tiled_kernel<kFormChannel, false, true>);
    else if (g.mx) go(gg_tiled_kernel<kFormMx, false, true>);
    else go(gg_tiled_kernel<kFormG128, false, true>);
  } else {
    if (g.a_rowsum) go(gg_tiled_kernel<kFormChannel, false>);
    else if (g.mx) go(gg_tiled_kernel<kFormMx, false>);
    else go(gg_tiled_kernel<kFormG128, false>);
  }
  return hipGetLastError();
}

}  // namespace w4a8
