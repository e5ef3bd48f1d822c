/*
 * w4a8_moe.h -- C ABI of the W4A8 mixture-of-experts routed-expert layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer, as the "GLM-5.3-W4A8" model card (gpustack) describes its
 * format in section 量化方式 (quantization method) and in its intro:
 *   - routed-expert weights are symmetric INT4, one scale per group of 128
 *     along the contraction axis K, stored compressed-tensors
 *     "pack-quantized": uint4b8 nibbles (u = q + 8), eight per int32 word;
 *   - activations are quantized to FP8 per token, dynamically, at run time;
 *   - the grouped GEMM turns the INT4 weights into FP8 inside the kernel and
 *     never dequantizes them to BF16.
 * Each expert has three projections (gate, up, down: "从 755GB 到 395GB",
 * Bitdeer AI blog, section 难点在于显存限制).  The layer's seven steps are the
 * six calls below, chained in this order:
 *   quant_act -> route -> permute -> grouped_gemm (gate/up) -> swiglu ->
 *   grouped_gemm (down) -> unpermute.
 *
 * Conventions shared by every call
 *   - Array pointers are DEVICE pointers; arrays are row-major, contiguous
 *     unless a leading dimension is given.  "u8 E4M3" arrays hold OCP
 *     E4M3FN codes (bias 7, max 448, no infinities).
 *   - Expert weights come in one of two formats, and each GEMM call names
 *     the one it takes:
 *       stored (the calls without "_prepacked"): the format the pages
 *         store, INT4 int32 [E][N][K/8] words whose nibble for k sits at
 *         bits 4*(k mod 8) of word k/8 and holds q + 8 (q in -8..7), with
 *         group scales fp32 [E][N][K/128]; MXFP4 u8 [E][N][K/2] codes and
 *         u8 [E][N][K/32] E8M0 scales;
 *       GEMM storage (the "_prepacked" calls): the same bytes permuted once
 *         by w4a8_moe_prepack_int4 / w4a8_moe_prepack_mxfp4, which the fast
 *         kernels read (described before w4a8_moe_prepack_int4).
 *     The two formats have the same size and the library cannot tell them
 *     apart from a pointer: weights in the wrong format give wrong numbers
 *     with status W4A8_OK.  The stored-format calls run the streaming kernel
 *     only (correct at any size, slower for many rows per expert).
 *   - The caller owns every buffer, including workspaces.  The library does
 *     not allocate, free, or keep any pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     only enqueues work on it and never synchronizes; ragged sizes (expert
 *     row offsets) stay on the device, so a chained layer is capturable.
 *   - Return value: W4A8_OK (0) or a w4a8_status code.  All argument checks
 *     run on the host before anything is launched: an argument error means
 *     nothing was enqueued.  W4A8_ERR_HIP reports a failed launch; where a
 *     call makes several launches (the layer's steps, or both GEMM kernels
 *     under W4A8_GG_AUTO), the ones before it may already be enqueued, and
 *     the outputs are then undefined.  w4a8_moe_last_error() gives the
 *     calling thread's last error detail.  Sizes of zero tokens/rows are
 *     valid no-ops.
 *   - The "not allocate" rule has one exception, for callers that cannot
 *     allocate: w4a8_moe_permute_noalloc uses a 1 MiB device array that the
 *     library holds per GPU.
 *   - Data preconditions that are NOT checked (undefined if violated):
 *     expert ids in [0, E); offsets monotone with offsets[E] == M_total;
 *     gather rows in range; no NaN/Inf in activations, logits or scales.
 *   - Every result is deterministic: the same inputs give bit-identical
 *     outputs from run to run.
 */
#ifndef W4A8_MOE_H
#define W4A8_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w4a8_status {
  W4A8_OK = 0,
  W4A8_ERR_NULL = 1,      /* a required pointer is NULL                        */
  W4A8_ERR_SHAPE = 2,     /* a size breaks the shape rules of the call         */
  W4A8_ERR_ALIGN = 3,     /* a pointer or leading dimension is misaligned      */
  W4A8_ERR_DEVICE = 4,    /* no HIP device, or the current device is not gfx950 */
  W4A8_ERR_HIP = 5,       /* a HIP runtime call or a kernel launch failed      */
  W4A8_ERR_WORKSPACE = 6  /* the workspace is smaller than required            */
} w4a8_status;

/* y_dtype values of w4a8_moe_unpermute */
#define W4A8_Y_F32 0
#define W4A8_Y_BF16 1

/* algo values of the _prepacked grouped GEMM calls.  W4A8_GG_AUTO takes the
 * streaming kernel while no expert has more than 20 rows and the average expert
 * at most 10 (M_total <= 10 E), else the tiled one.  Where M_total does not
 * settle it, both kernels are enqueued and the one the largest expert (known on
 * the device only) does not call for returns at once.  The calls without
 * _prepacked always take the streaming kernel. */
#define W4A8_GG_AUTO 0     /* choose from the rows per expert                     */
#define W4A8_GG_STREAM 1   /* weight-streaming kernel for few rows per expert     */
#define W4A8_GG_TILED 2    /* LDS-tiled persistent kernel for many rows per expert */

/*
 * Step 1 -- per-token dynamic FP8 quantization of the activations.
 * ("GLM-5.3-W4A8" card, section 量化方式 and the comparison table of section
 * 与其他 4-bit 版本的差异: FP8, per token, dynamic.)
 *   For each token t: amax = max_k |x[t,k]|, sx[t] = fl32(amax / 448)
 *   (1.0 if the row is all zero), qx[t,k] = E4M3(fl32(x[t,k] / sx[t])),
 *   rounded to nearest, ties to even, saturating at +-448, sign kept on 0.
 *   x_bf16 : bf16 bit patterns [T][ld_x] (first H columns used); 16-byte
 *            aligned, ld_x % 8 == 0, ld_x >= H.
 *   qx     : u8 E4M3 [T][H], 8-byte aligned.     sx : fp32 [T].
 *   Rules  : T >= 0, H > 0, H % 128 == 0.
 */
int w4a8_moe_quant_act(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x,
                       uint8_t* qx, float* sx, void* stream);

/*
 * Step 2 -- top-k softmax routing of each token to the routed experts.
 * (256 routed experts per MoE layer: "从 755GB 到 395GB", section
 * 我们量化了什么; the router itself stays BF16 per the "GLM-5.3-W4A8" card,
 * section 量化方式, so its logits are an input here.)
 *   ids[t, 0..k-1] = the k largest logits[t, :] in descending order, equal
 *   logits ordered by the lower expert index; p = softmax(logits[t, :]);
 *   w[t, j] = p[ids_j] / sum_j' p[ids_j'] if renormalize, else p[ids_j].
 *   logits : fp32 [T][E].   ids : int32 [T][k].   w : fp32 [T][k].
 *   Rules  : T >= 0, 1 <= k <= E <= 1024, T * k < 2^31.
 */
int w4a8_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renormalize,
                   int32_t* ids, float* w, void* stream);

/* Bytes of device workspace w4a8_moe_permute needs (>= 0), or -1 on bad sizes. */
int64_t w4a8_moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E);

/*
 * Step 3 -- group the T*k routed rows by expert (a stable counting sort).
 * (The expert-parallel dispatch of the pages' engines, "GLM-5.3-W4A8" card,
 * sections 性能 and 部署, done here inside one GPU.)
 *   f = t*k + j indexes ids.  counts[e] = #{f : ids[f] == e};
 *   offsets = exclusive prefix sum of counts (E + 1 entries, offsets[E] = T*k);
 *   rows of expert e are offsets[e] .. offsets[e+1]-1, ordered by f;
 *   row_token[p] = token of routed row p;  inv_pos[f] = row of index f.
 *   An id outside [0, E) is not routed: it is not counted (offsets[E] is then
 *   the number of routed ids, and row_token past it is not written) and its
 *   inv_pos is -1, which w4a8_moe_unpermute skips.
 *   ids : int32 [T*k].  offsets : int32 [E+1].  row_token, inv_pos : int32 [T*k].
 *   workspace : device memory of w4a8_moe_permute_workspace_bytes(T, k, E)
 *   bytes, 4-byte aligned (contents need no initialisation).
 *   Rules : T >= 0, 1 <= k <= E <= 1024, T * k < 2^31.  T == 0 still writes
 *   offsets (all zero).
 */
int w4a8_moe_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E,
                     int32_t* offsets, int32_t* row_token, int32_t* inv_pos,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * w4a8_moe_permute without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * hipMalloc): the sort's per-(expert, block) counts go to a buffer of 1 MiB
 * that the library holds on each GPU until the process ends, and nothing is
 * allocated.  Same arguments (minus the workspace), results and rules as
 * w4a8_moe_permute, and:
 *   - sizes that need more than 1 MiB (w4a8_moe_permute_workspace_bytes(T, k,
 *     E) > 1048576, e.g. T*k above 1,048,576 routed rows at E = 256) return
 *     W4A8_ERR_WORKSPACE and launch nothing;
 *   - every call on one GPU shares that GPU's buffer: calls that overlap on
 *     one GPU (several streams or host threads) race and must not be made.
 */
int w4a8_moe_permute_noalloc(const int32_t* ids, int64_t T, int32_t k, int32_t E,
                             int32_t* offsets, int32_t* row_token, int32_t* inv_pos, void* stream);

/*
 * Steps 1, 2 and 3 in one call: w4a8_moe_quant_act, w4a8_moe_route and
 * w4a8_moe_permute on the same arguments, with the same results.  For decode
 * batches (T*k <= 4096 and H <= 8192) they run as one kernel: the quantizer
 * and the router side by side, and the router workgroup that finishes last
 * sorts the routed rows; otherwise as the three kernels.
 *   counter : one uint32 on the device, 4-byte aligned, zero before the
 *             first call; every call leaves it zero.  Calls that share a
 *             counter must not overlap (use one per stream).
 *   Every other argument and rule: as in the three calls.
 */
int w4a8_moe_front(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x, uint8_t* qx, float* sx,
                   const float* logits, int32_t E, int32_t k, int32_t renormalize, int32_t* ids, float* w,
                   int32_t* offsets, int32_t* row_token, int32_t* inv_pos, void* workspace, int64_t workspace_bytes,
                   uint32_t* counter, void* stream);

/* The same with the INT8 quantizer of w4a8_moe_quant_act_i8 (codes plus row sums). */
int w4a8_moe_front_i8(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x, int8_t* qx, float* sx,
                      int32_t* rowsum, const float* logits, int32_t E, int32_t k, int32_t renormalize, int32_t* ids,
                      float* w, int32_t* offsets, int32_t* row_token, int32_t* inv_pos, void* workspace,
                      int64_t workspace_bytes, uint32_t* counter, void* stream);

/*
 * ---- GEMM storage of the expert weights ------------------------------------
 * The "_prepacked" grouped GEMMs read the 4-bit weights in a permuted order,
 * written once by a prepack call: the 64 packed bytes of one 128-wide K group of 16
 * consecutive weight rows are one contiguous 1 KB piece, and the per-group
 * scales are group-major.  (The INT4 form the pages store, int32 uint4b8
 * words row by row, is the input of w4a8_moe_prepack_int4.)  G = K/128:
 *   weights : int32 [E][N/16][G][16][16] (INT4) or u8 [E][N/16][G][16][64]
 *             (MXFP4): row n, group g (row-major words 16g .. 16g+15, bytes
 *             64g .. 64g+63) at byte ((e (N/16) + n/16) G + g) 1024 + 64 (n % 16).
 *             An INT4 word keeps its eight K elements but holds their nibbles
 *             in the order k0 k4 k1 k5 k2 k6 k3 k7 (bits 0..31), so that one
 *             mask yields k0..k3 and one shift and mask k4..k7, a byte each;
 *   scales  : fp32 [E][G][N] (INT4 group 128) or u8 [E][G][N][4] (MXFP4):
 *             row n, group g at ((e G + g) N + n) 4.  Per-channel scales
 *             ([E][N]) need no change.
 * Reading whole 1 KB pieces and group-major scales, every weight and scale
 * load fills whole cache lines.
 */

/*
 * Offline layout step, INT4: row-major uint4b8 words w_packed int32 [E][N][K/8]
 * (and, for the group-128 form, w_scale fp32 [E][N][K/128]) -> GEMM storage
 * w_blk int32 [E][N/16][K/128][16][16] (and s_blk fp32 [E][K/128][N]).  A
 * permutation of the words, and of the nibbles inside each word (see above).
 * Pass w_scale = s_blk = NULL for per-channel scales,
 * which the GEMMs read as they are.
 *   Rules : 0 <= E <= 1024, N % 16 == 0, K % 128 == 0; weights 16-byte
 *   aligned, scales 4-byte aligned; no overlap of inputs and outputs.
 */
int w4a8_moe_prepack_int4(const int32_t* w_packed, const float* w_scale, int32_t E, int64_t N, int64_t K,
                          int32_t* w_blk, float* s_blk, void* stream);

/*
 * Steps 4 and 6 -- grouped W4A8 GEMM over the experts' row ranges, on the
 * weights as stored.
 * ("GLM-5.3-W4A8" card, section 量化方式: INT4 weights become FP8 inside
 * the kernel, FP8 matrix multiply, no BF16 dequantization; the weights are
 * compressed-tensors pack-quantized uint4b8 in int32 with group size 128.)
 *   For expert e and each row p in [offsets[e], offsets[e+1]), with
 *   r = a_rows ? a_rows[p] : p:
 *     out[p, n] = a_scale[r] * sum_g w_scale[e, n, g] *
 *                 sum_{k in group g} E4M3(a[r, k]) * q[e, n, k]
 *   a        : u8 E4M3 [*][K], 16-byte aligned (source rows; gathered by
 *              a_rows when it is not NULL).   a_scale : fp32 [*].
 *   a_rows   : int32 [M_total] or NULL.
 *   offsets  : int32 [E+1] on the device, offsets[E] == M_total.
 *   w_packed : int32 [E][N][K/8]: nibble k of row n at bits 4 (k mod 8) of
 *              word k/8, holding q + 8; 16-byte aligned.
 *   w_scale  : fp32 [E][N][K/128].
 *   out      : fp32 [M_total][N], 16-byte aligned.
 *   Rules    : M_total >= 0, 1 <= E <= 1024, N > 0, N % 16 == 0, K > 0,
 *              K % 128 == 0.  Unchecked: with a_rows, a_rows[p] * K < 2^32.
 *   Accumulation is fp32 per 128-wide group, then the group scale is
 *   applied in fp32.  The matrix cores' FP8 dot products round within about
 *   1e-5 of the group's sum of |products|, so results agree with the exact
 *   sum to about 1e-5 relative (Frobenius norm over a matrix).
 *   Runs the weight-streaming kernel, which reads each expert's weights once
 *   per 16 of its rows (once per 64 when M_total > 8 E): right for decode;
 *   for many rows per expert, prepack the weights and call
 *   w4a8_moe_grouped_gemm_prepacked.
 */
int w4a8_moe_grouped_gemm(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                          int64_t M_total, const int32_t* offsets, int32_t E,
                          const int32_t* w_packed, const float* w_scale,
                          int64_t N, int64_t K, float* out, void* stream);

/*
 * The same on weights in the GEMM storage (w4a8_moe_prepack_int4):
 *   w_blk : int32 [E][N/16][K/128][16][16], 16-byte aligned.
 *   s_blk : fp32 [E][K/128][N].
 *   algo  : W4A8_GG_AUTO, W4A8_GG_STREAM or W4A8_GG_TILED; every algo
 *           computes the same bits, the choice only affects speed.
 *   Rules : as w4a8_moe_grouped_gemm, with N % 64 == 0.
 */
int w4a8_moe_grouped_gemm_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                    int64_t M_total, const int32_t* offsets, int32_t E,
                                    const int32_t* w_blk, const float* s_blk,
                                    int64_t N, int64_t K, float* out, int32_t algo, void* stream);

/*
 * Step 5 -- SwiGLU of the gate/up output and per-row FP8 re-quantization.
 * (Three projections per expert: Bitdeer AI blog, section 难点在于显存限制;
 * per-token FP8 activations: "GLM-5.3-W4A8" card, section 量化方式.)
 *   gate = h[p, 0:I], up = h[p, I:2I]; act = silu(gate) * up in fp32,
 *   silu(z) = z / (1 + exp(-z)); then the step-1 rule per routed row:
 *   sa[p] = fl32(amax / 448), qa[p, i] = E4M3(fl32(act / sa[p])).
 *   h : fp32 [M][2I], 16-byte aligned.  qa : u8 E4M3 [M][I], 4-byte aligned.
 *   sa : fp32 [M].   Rules : M >= 0, I > 0, I % 128 == 0.
 */
int w4a8_moe_swiglu(const float* h, int64_t M, int64_t I, uint8_t* qa, float* sa, void* stream);

/*
 * Step 7 -- routing-weighted combine of the k expert outputs of each token.
 *   y[t, :] = sum_{j = 0..k-1} w[t, j] * o[inv_pos[t*k + j], :]  (fp32, j ascending)
 *   o : fp32 [T*k][H], 16-byte aligned.  inv_pos : int32 [T*k].  w : fp32 [T][k].
 *   y : [T][H], fp32 (y_dtype W4A8_Y_F32, 16-byte aligned) or bf16 bit
 *       patterns rounded to nearest even (W4A8_Y_BF16, 8-byte aligned).
 *   Rules : T >= 0, k >= 1, H > 0, H % 128 == 0, T * k < 2^31.
 */
int w4a8_moe_unpermute(const float* o, const int32_t* inv_pos, const float* w,
                       int64_t T, int32_t k, int64_t H, void* y, int32_t y_dtype, void* stream);

/*
 * Step 7 with the routing-weighted scatter done in the down GEMM's epilogue:
 * each expert output row is weighted and written to its token's slot, and the
 * combine sums each token's k slots.  (Each token's output is the sum of its
 * top-k experts' outputs weighted by the router's weights: "从 755GB 到
 * 395GB", section 我们量化了什么, 256 routed experts per layer, and the
 * "GLM-5.3-W4A8" card, section 量化方式.)  Three calls:
 *
 * w4a8_moe_row_sources -- for every routed index f = t*k + j (inv_pos[f] = p,
 *   0 <= p < M_total): row_src[p] = f and row_scale[p] = fl32(a_scale[p] * w[f]).
 *   inv_pos : int32 [T*k].  w : fp32 [T][k].  a_scale : fp32 [M_total] (the down
 *   GEMM's activation scales, sa of step 5).  row_src : int32 [M_total],
 *   row_scale : fp32 [M_total].  All 4-byte aligned.
 *   Rules : T >= 0, k >= 1, T * k < 2^31, 0 <= M_total <= T * k.  M_total = 0 is
 *   a no-op (pointers may then be null).  inv_pos must map the routed indices
 *   one to one onto [0, M_total), as w4a8_moe_permute writes it; values outside
 *   that range are skipped.
 *
 * w4a8_moe_grouped_gemm_scatter_prepacked (and _i8_, _mxfp4_) -- the grouped
 *   GEMM of the matching _prepacked call, with row p of the result stored as
 *   row row_dst[p] of out.  Called with a_scale = row_scale and row_dst = row_src
 *   it writes o_tok[f, :] = w[f] * o[p, :] (the weight enters through the row's
 *   scale).  row_dst : int32 [M_total], 4-byte aligned, each value a distinct
 *   row of out (not checked).  out : fp32 [rows][N], 16-byte aligned; rows of
 *   out that no row_dst names are left as they were.  Other arguments and rules
 *   as in the _prepacked call.
 *
 * w4a8_moe_combine -- y[t, :] = sum over j = 0..k-1 with inv_pos[t*k + j] >= 0,
 *   j ascending, of o_tok[t*k + j, :] (fp32 adds).  o_tok : fp32 [T*k][H],
 *   16-byte aligned.  y and y_dtype as in w4a8_moe_unpermute.
 *   Rules : as w4a8_moe_unpermute.
 *
 * The chain gives step 7's y up to the rounding of w * o before the sum (one
 * fp32 rounding more per term); its reads of the expert outputs are contiguous
 * k-row blocks instead of gathered rows.
 */
int w4a8_moe_row_sources(const int32_t* inv_pos, const float* w, const float* a_scale, int64_t T, int32_t k,
                         int64_t M_total, int32_t* row_src, float* row_scale, void* stream);
int w4a8_moe_grouped_gemm_scatter_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                            int64_t M_total, const int32_t* offsets, int32_t E,
                                            const int32_t* w_blk, const float* s_blk, int64_t N, int64_t K,
                                            const int32_t* row_dst, float* out, int32_t algo, void* stream);
int w4a8_moe_grouped_gemm_scatter_i8_prepacked(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                               const int32_t* a_rows, int64_t M_total, const int32_t* offsets,
                                               int32_t E, const int32_t* w_blk, const float* w_scale, int64_t N,
                                               int64_t K, const int32_t* row_dst, float* out, int32_t algo,
                                               void* stream);
int w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                                  int64_t M_total, const int32_t* offsets, int32_t E,
                                                  const uint8_t* w_blk, const uint8_t* s_blk, int64_t N, int64_t K,
                                                  const int32_t* row_dst, float* out, int32_t algo, void* stream);
int w4a8_moe_combine(const float* o_tok, const int32_t* inv_pos, int64_t T, int32_t k, int64_t H, void* y,
                     int32_t y_dtype, void* stream);

/*
 * Offline step before the layer -- quantize expert weights to the layer's
 * INT4 format.  ("GLM-5.3-W4A8" card, section 量化方式: float32 weights,
 * symmetric INT4 with group size 128 along K, each group's scale chosen by the
 * smallest squared error over 11 shrink ratios 1.00, 0.97, ..., 0.70, packed
 * as compressed-tensors uint4b8 in int32.)
 *   For every row n and group g of 128 weights:
 *     amax = max |w| over the group (1 if it is all zero);
 *     s_r = fl32(r * amax / 7);  q_r = clamp(round-half-even(w / s_r), -8, 7)
 *     (the exact quotient rounded);  with mse_clip the group keeps the r of
 *     smallest sum (w - q_r s_r)^2 (fp64 sums; the larger r on ties), without
 *     it r = 1 (plain round-to-nearest).
 *   w        : fp32 [rows][K] (rows = experts x output channels), 8-byte aligned.
 *   w_packed : int32 [rows][K/8]: nibble k at bits 4 (k mod 8) of word k/8, holding q + 8.
 *   w_scale  : fp32 [rows][K/128].
 *   Rules    : rows >= 0, K > 0, K % 128 == 0.  Inputs must be finite.
 */
int w4a8_moe_quantize_weights(const float* w, int64_t rows, int64_t K, int32_t mse_clip,
                              int32_t* w_packed, float* w_scale, void* stream);

/*
 * ---- The per-channel INT4 x per-token INT8 variant ---------------------
 * ("GLM-5.3-Channel-INT4-w4a8" card, section 1: routed experts INT4 W4A8
 * with weights quantized RTN, static, per channel; activations INT8,
 * dynamic, per token.)  Routing, permutation and the combine are shared with
 * the group-128 FP8 form above; these calls replace steps 1, 4, 5 and 6.
 */

/*
 * Step 1, INT8 -- per-token quantization of bf16 activations.
 *   scale sx[t] = fl32(amax / 127) (1.0 for an all-zero row);
 *   qx[t, k] = clamp(round-half-even(fl32(x[t, k] / sx[t])), -127, 127);
 *   rowsum[t] = sum_k qx[t, k] (the INT8 GEMM uses it to undo the +8
 *   offset of the stored weight nibbles).
 *   x : bf16 [T][ld_x] (H used), 16-byte aligned.  qx : int8 [T][H], 8-byte
 *   aligned.  sx : fp32 [T].  rowsum : int32 [T].
 *   Rules : T >= 0, H > 0, H % 128 == 0, ld_x >= H, ld_x % 8 == 0.
 */
int w4a8_moe_quant_act_i8(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x,
                          int8_t* qx, float* sx, int32_t* rowsum, void* stream);

/*
 * Steps 4 and 6, INT8 -- grouped GEMM with per-channel INT4 weights, as stored.
 *   For expert e and each row p in [offsets[e], offsets[e+1]), with
 *   r = a_rows ? a_rows[p] : p:
 *     out[p, n] = a_scale[r] * w_scale[e, n] * sum_k a[r, k] * q[e, n, k]
 *   computed as (sum_k a u - 8 rowsum[r]) with u = q + 8, exact in int32
 *   (K <= 2^20), then the two scales in fp32.
 *   a : int8 [*][K], 16-byte aligned.  a_scale : fp32 [*].  a_rowsum : int32 [*].
 *   a_rows, offsets : as in w4a8_moe_grouped_gemm.
 *   w_packed : int32 [E][N][K/8] uint4b8 words as stored, 16-byte aligned.
 *   w_scale : fp32 [E][N].  out : fp32 [M_total][N], 16-byte aligned.
 *   Rules : as in w4a8_moe_grouped_gemm, and K <= 2^20.
 */
int w4a8_moe_grouped_gemm_i8(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                             const int32_t* a_rows, int64_t M_total, const int32_t* offsets, int32_t E,
                             const int32_t* w_packed, const float* w_scale, int64_t N, int64_t K,
                             float* out, void* stream);

/* The same on weights in the GEMM storage (w_blk int32 [E][N/16][K/128][16][16],
 * w4a8_moe_prepack_int4 with no scales); per-channel scales w_scale [E][N] as
 * they are.  algo : W4A8_GG_*.  Rules : N % 64 == 0, otherwise as above. */
int w4a8_moe_grouped_gemm_i8_prepacked(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                       const int32_t* a_rows, int64_t M_total, const int32_t* offsets, int32_t E,
                                       const int32_t* w_blk, const float* w_scale, int64_t N, int64_t K,
                                       float* out, int32_t algo, void* stream);

/*
 * Step 5, INT8 -- SwiGLU of the gate/up output, then the step-1 INT8 rule
 * per routed row (with row sums).
 *   h : fp32 [M][2I], 16-byte aligned.  qa : int8 [M][I], 4-byte aligned.
 *   sa : fp32 [M].  rowsum : int32 [M].  Rules : M >= 0, I > 0, I % 128 == 0.
 */
int w4a8_moe_swiglu_i8(const float* h, int64_t M, int64_t I, int8_t* qa, float* sa, int32_t* rowsum,
                       void* stream);

/*
 * Offline, INT8 variant -- per-channel RTN INT4 weights.
 *   s[n] = fl32(amax_n / 7) (1/7 for an all-zero row);
 *   q = clamp(round-half-even(w / s[n]), -8, 7) (the exact quotient rounded).
 *   w : fp32 [rows][K], 8-byte aligned.  w_packed : int32 [rows][K/8] uint4b8.
 *   w_scale : fp32 [rows].  Rules : rows >= 0, K > 0, K % 128 == 0.
 */
int w4a8_moe_quantize_weights_channel(const float* w, int64_t rows, int64_t K, int32_t* w_packed,
                                      float* w_scale, void* stream);

/*
 * ---- Fused epilogues ------------------------------------------------------
 * Steps 4 and 5 of the layer split differently: the gate/up GEMM applies
 * SwiGLU in its epilogue and writes act = silu(gate) * up instead of the
 * [M][2I] gate/up output, plus partial row maxima of |act|; the requant call
 * then turns act into the step-5 codes.  The results are those of step 4
 * followed by step 5 (the same fp32 values, the same scale and code rule)
 * with half the intermediate bytes.  (The SwiGLU after the gate/up
 * projection and the per-token re-quantization: "GLM-5.3-W4A8" card,
 * sections 量化方式 and 与其他 4-bit 版本的差异.)
 */

/*
 * Steps 4 + 5a, group-128 FP8 form, weights as stored.
 *   For expert e and row p in [offsets[e], offsets[e+1]) (r = a_rows ? a_rows[p] : p):
 *     gate[n] = h[p, n], up[n] = h[p, I + n] of w4a8_moe_grouped_gemm with N = 2I;
 *     act[p, n] = silu(gate[n]) * up[n], silu(z) = z / (1 + e^-z), fp32 (hardware
 *     exponential and reciprocal: within a few ulp of the exact value);
 *     act_pmax[p, s], s < I/64: maxima of |act[p, :]| over parts of the row, whose
 *     maximum is max_n |act[p, n]| (every entry is written; no zeroing needed).
 *   a, a_scale, a_rows, offsets : as in w4a8_moe_grouped_gemm.
 *   w13 : int32 [E][2I][K/8] as stored (gate rows 0..I-1, up rows I..2I-1),
 *         16-byte aligned.   s13 : fp32 [E][2I][K/128].
 *   act : fp32 [M_total][I], 16-byte aligned.  act_pmax : fp32 [M_total][I/64], 4-byte aligned.
 *   Rules : I > 0, I % 128 == 0, K % 128 == 0, 1 <= E <= 1024; otherwise as in w4a8_moe_grouped_gemm.
 */
int w4a8_moe_grouped_gemm_swiglu(const uint8_t* a, const float* a_scale, const int32_t* a_rows, int64_t M_total,
                                 const int32_t* offsets, int32_t E, const int32_t* w13, const float* s13, int64_t I,
                                 int64_t K, float* act, float* act_pmax, void* stream);

/* The same on the GEMM storage of w13 (int32 [E][2I/16][K/128][16][16]) and
 * s13 (fp32 [E][K/128][2I]); algo : W4A8_GG_*. */
int w4a8_moe_grouped_gemm_swiglu_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                           int64_t M_total, const int32_t* offsets, int32_t E, const int32_t* w13,
                                           const float* s13, int64_t I, int64_t K, float* act, float* act_pmax,
                                           int32_t algo, void* stream);

/*
 * Steps 4 + 5a, per-channel INT8 form: as w4a8_moe_grouped_gemm_swiglu with
 * the products of w4a8_moe_grouped_gemm_i8 (a : int8 codes with row sums
 * a_rowsum; w13 : int32 [E][2I][K/8] as stored; s13 : fp32 [E][2I]; K <= 2^20).
 */
int w4a8_moe_grouped_gemm_swiglu_i8(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                    const int32_t* a_rows, int64_t M_total, const int32_t* offsets, int32_t E,
                                    const int32_t* w13, const float* s13, int64_t I, int64_t K, float* act,
                                    float* act_pmax, void* stream);

/* The same on the GEMM storage of w13; algo : W4A8_GG_*. */
int w4a8_moe_grouped_gemm_swiglu_i8_prepacked(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                              const int32_t* a_rows, int64_t M_total, const int32_t* offsets,
                                              int32_t E, const int32_t* w13, const float* s13, int64_t I, int64_t K,
                                              float* act, float* act_pmax, int32_t algo, void* stream);

/*
 * Step 5b, FP8 -- the step-1 rule per row, from the row maxima of the fused GEMM:
 *   m = max_s act_pmax[p, s]; sa[p] = fl32(m / 448) (1.0 if 0); qa[p, n] = E4M3(fl32(act[p, n] / sa[p])).
 *   act : fp32 [M][I], 16-byte aligned.  act_pmax : fp32 [M][I/64] (partial maxima of |act|).
 *   qa : u8 [M][I], 4-byte aligned.  sa : fp32 [M].  Rules : M >= 0, I > 0, I % 128 == 0.
 */
int w4a8_moe_requant(const float* act, const float* act_pmax, int64_t M, int64_t I, uint8_t* qa, float* sa,
                     void* stream);

/*
 * Step 5b, INT8: sa[p] = fl32(m / 127) (1.0 if 0);
 *   qa[p, n] = clamp(round-half-even(fl32(act[p, n] / sa[p])), -127, 127); rowsum[p] = sum_n qa[p, n].
 *   qa : int8 [M][I], 4-byte aligned.  rowsum : int32 [M].  Otherwise as w4a8_moe_requant.
 */
int w4a8_moe_requant_i8(const float* act, const float* act_pmax, int64_t M, int64_t I, int8_t* qa, float* sa,
                        int32_t* rowsum, void* stream);

/*
 * ---- MXFP4 group-32 weights ----------------------------------------------
 * The 4-bit alternative the "GLM-5.3-W4A8" card compares INT4 group 128
 * against (section 量化方式: MXFP4 with groups of 32, and the note that
 * Hopper has no FP4 matrix cores).  gfx950 multiplies FP4 by FP8 in its
 * matrix cores, so the same per-token FP8 activations (steps 1 and 5) meet
 * MXFP4 weights; routing, permutation, requant and combine are unchanged.
 * The format is the Open Compute Project microscaling one: E2M1 elements
 * (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 the sign) sharing one E8M0
 * scale (byte b = 2^(b - 127)) per 32 consecutive weights along K.
 * Row-major storage (what the quantizer writes):
 *   Weights : u8 [E][N][K/2], element k of a row in the low nibble of byte
 *             k/2 when k is even, the high nibble when odd.
 *   Scales  : u8 [E][N][K/32], the E8M0 byte of elements 32j .. 32j+31.
 * GEMM storage (what w4a8_moe_prepack_mxfp4 writes and the GEMMs read), the
 * same bytes permuted, G = K/128:
 *   Weights : u8 [E][N/16][G][16][64]: the 64 bytes of row n and K group g
 *             (row-major bytes 64g .. 64g+63) at ((e (N/16) + n/16) G + g) 1024 + 64 (n % 16).
 *   Scales  : u8 [E][G][N][4]: the 4 bytes of row n and group g (row-major
 *             bytes 4g .. 4g+3) at ((e G + g) N + n) 4.
 */

/*
 * Offline weight quantizer, MXFP4.  Per block of 32 (rows x K fp32, row-major):
 *   amax = max |w| (1 if the block is all zero); X = floor(log2 amax) - 2,
 *   clamped to [-127, 127]; w_scale byte = X + 127;
 *   code = E2M1 of w * 2^-X: the nearest magnitude, ties to the code with
 *   mantissa bit 0, saturating at 6, with the sign bit of w.
 *   w : fp32 [rows][K], 16-byte aligned.  w_packed : u8 [rows][K/2], 2-byte aligned.
 *   w_scale : u8 [rows][K/32].  Rules : rows >= 0, K > 0, K % 32 == 0.
 */
int w4a8_moe_quantize_weights_mxfp4(const float* w, int64_t rows, int64_t K, uint8_t* w_packed, uint8_t* w_scale,
                                    void* stream);

/*
 * Offline layout step, MXFP4: row-major weights and scales -> GEMM storage
 * (a permutation of bytes; see above).  Reads w_packed u8 [E][N][K/2] and
 * w_scale u8 [E][N][K/32]; writes w_blk u8 [E][N/16][K/128][16][64] and
 * s_blk u8 [E][K/128][N][4] (no overlap with the inputs).
 *   Rules : 0 <= E <= 1024, N % 16 == 0, K % 128 == 0; weights 16-byte
 *   aligned, scales 4-byte aligned.
 */
int w4a8_moe_prepack_mxfp4(const uint8_t* w_packed, const uint8_t* w_scale, int32_t E, int64_t N, int64_t K,
                           uint8_t* w_blk, uint8_t* s_blk, void* stream);

/*
 * Step 4, MXFP4 weights, as stored:
 *   out[p, n] = a_scale[r] * sum_k E4M3(a[r, k]) * E2M1(w[e, n, k]) * 2^(w_scale[e, n, k/32] - 127)
 *   (r = a_rows ? a_rows[p] : p; exact products, fp32 sums).
 *   a, a_scale, a_rows, offsets, out : as in w4a8_moe_grouped_gemm.
 *   w_packed : u8 [E][N][K/2] (row-major storage above), 16-byte aligned.
 *   w_scale : u8 [E][N][K/32], 4-byte aligned.
 *   Rules : N % 16 == 0, K % 128 == 0, 1 <= E <= 1024; errors as in w4a8_moe_grouped_gemm.
 */
int w4a8_moe_grouped_gemm_mxfp4(const uint8_t* a, const float* a_scale, const int32_t* a_rows, int64_t M_total,
                                const int32_t* offsets, int32_t E, const uint8_t* w_packed, const uint8_t* w_scale,
                                int64_t N, int64_t K, float* out, void* stream);

/* The same on the GEMM storage (w_blk u8 [E][N/16][K/128][16][64], s_blk u8
 * [E][K/128][N][4], from w4a8_moe_prepack_mxfp4); algo : W4A8_GG_*; N % 64 == 0. */
int w4a8_moe_grouped_gemm_mxfp4_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                          int64_t M_total, const int32_t* offsets, int32_t E, const uint8_t* w_blk,
                                          const uint8_t* s_blk, int64_t N, int64_t K, float* out, int32_t algo,
                                          void* stream);

/*
 * Steps 4 + 5a, MXFP4 weights: as w4a8_moe_grouped_gemm_swiglu with the
 * products of w4a8_moe_grouped_gemm_mxfp4 (w13 : u8 [E][2I][K/2] as stored,
 * 16-byte aligned; s13 : u8 [E][2I][K/32], 4-byte aligned).
 * Follow with w4a8_moe_requant.
 */
int w4a8_moe_grouped_gemm_swiglu_mxfp4(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                       int64_t M_total, const int32_t* offsets, int32_t E, const uint8_t* w13,
                                       const uint8_t* s13, int64_t I, int64_t K, float* act, float* act_pmax,
                                       void* stream);

/* The same on the GEMM storage of w13 and s13; algo : W4A8_GG_*. */
int w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                                 int64_t M_total, const int32_t* offsets, int32_t E,
                                                 const uint8_t* w13, const uint8_t* s13, int64_t I, int64_t K,
                                                 float* act, float* act_pmax, int32_t algo, void* stream);

/* Static name of a status code ("W4A8_OK", ...). */
const char* w4a8_moe_status_string(int status);

/* Detail of the calling thread's last error ("" if none).  Valid until the
 * thread's next call into the library. */
const char* w4a8_moe_last_error(void);

/* 1 if the current HIP device is a gfx950, 0 otherwise (including no device). */
int w4a8_moe_device_supported(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_MOE_H */
