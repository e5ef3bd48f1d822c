// Internal launchers of the W4A8 MoE kernels (called by the C ABI after it
// has validated every argument on the host).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

// One grouped GEMM on weights in the GEMM storage (launch_prepack): 1 KB per 16
// rows x 128 K ([E][N/16][K/128][16][64] bytes; INT4 words with their nibbles
// in the order k0 k4 k1 k5 k2 k6 k3 k7), per-group scales group-major
// ([E][K/128][N] 4-byte words).  a_rowsum == nullptr: the group-128 FP8 form
// (w_scale fp32 group scales), or with mx set the MXFP4 form; otherwise the
// per-channel INT8 form (INT8 activations with their row code sums, w_scale
// fp32 [E][N]).
struct GemmArgs {
  const uint8_t* a;
  const float* a_scale;
  const int32_t* a_rowsum;
  const int32_t* a_rows;
  int64_t M_total;
  const int32_t* offsets;
  int E;
  const int32_t* w_packed;
  const float* w_scale;
  int64_t N;
  int64_t K;
  float* out;
  // fused SwiGLU (gate/up GEMM only): when set, out is act [M_total][N/2] =
  // silu(gate) * up, gate and up being the weight rows n and N/2 + n, and
  // pmax [M_total][N/128] gets row maxima of |act| (each entry over some of
  // the row's columns; their max is the row's)
  float* pmax = nullptr;
  // MXFP4 weights: w_packed holds E2M1 codes (element k in the low nibble of
  // byte k/2 when k is even), w_scale the E8M0 block scales (the 4-byte word of
  // a row and group holds its four 32-element blocks)
  bool mx = false;
  // the weights in the row-major stored format (INT4 int32 [E][N][K/8] words,
  // nibble k at bits 4 (k mod 8); MXFP4 u8 [E][N][K/2]) with scales [E][N][K/128]
  // (fp32) or [E][N][K/32] (E8M0): the stream kernel only
  bool row_major = false;
  // the kernel choice taken on the device from the batch's largest expert: when
  // >= 0, both kernels are launched, the stream kernel returning at once if some
  // expert has more than sel_rows rows and the tiled kernel if none has
  int32_t sel_rows = -1;
  // plain form only: when set, GEMM row p is stored as row out_rows[p] of out
  // (the routing-weighted scatter: with a_scale holding sa[p] w[f], row p lands
  // weighted in its token-major slot f = t k + j)
  const int32_t* out_rows = nullptr;
};

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t H, int64_t ld, uint8_t* q, float* s,
                            hipStream_t stream);
hipError_t launch_route(const float* logits, int64_t T, int E, int k, int renormalize, int32_t* ids, float* w,
                        hipStream_t stream);
int64_t permute_workspace_bytes(int64_t R, int E);
// bytes of the buffer w4a8_moe_permute_noalloc uses in place of the workspace
constexpr int64_t kPermScratchBytes = (int64_t)1 << 20;
// the device address of that buffer on the current device (looked up once per device)
hipError_t permute_scratch(int32_t** ptr);
hipError_t launch_permute(const int32_t* ids, int64_t R, int k, int E, int32_t* offsets, int32_t* row_token,
                          int32_t* inv_pos, int32_t* counts, hipStream_t stream);
hipError_t launch_gg_stream(const GemmArgs& g, hipStream_t stream);
hipError_t launch_gg_tiled(const GemmArgs& g, hipStream_t stream);
// whether the tiled kernel's 32-bit byte offsets reach every operand (else
// launch_gg_tiled runs the stream kernel)
bool tiled_fits(const GemmArgs& g);
hipError_t launch_swiglu(const float* h, int64_t M, int64_t I, uint8_t* q, float* s, hipStream_t stream);
hipError_t launch_quant_act_i8(const uint16_t* x, int64_t T, int64_t H, int64_t ld, int8_t* q, float* s,
                               int32_t* rowsum, hipStream_t stream);
hipError_t launch_swiglu_i8(const float* h, int64_t M, int64_t I, int8_t* q, float* s, int32_t* rowsum,
                            hipStream_t stream);
hipError_t launch_wquant_channel(const float* w, int64_t rows, int64_t K, int32_t* packed, float* scales,
                                 hipStream_t stream);
hipError_t launch_wquant(const float* w, int64_t rows, int64_t K, int mse_clip, int32_t* packed, float* scales,
                         hipStream_t stream);
hipError_t launch_wquant_mxfp4(const float* w, int64_t rows, int64_t K, uint8_t* packed, uint8_t* scales,
                               hipStream_t stream);
hipError_t launch_prepack(const void* w, const void* s, int64_t E, int64_t N, int64_t K, int nibble_split,
                          void* wb, void* sb, hipStream_t stream);
hipError_t launch_requant(const float* act, const float* pmax, int64_t M, int64_t I, uint8_t* q, float* s,
                          hipStream_t stream);
hipError_t launch_requant_i8(const float* act, const float* pmax, int64_t M, int64_t I, int8_t* q, float* s,
                             int32_t* rowsum, hipStream_t stream);
// layer steps 1-3 in one launch (front.hip); front_fits tells whether a shape
// qualifies (T k <= 4096 routed rows, H <= 8192)
struct FrontArgs {
  const uint16_t* x;
  int64_t T, H, ld;
  uint8_t* q;
  float* s;
  int32_t* rowsum;        // INT8 form only
  const float* logits;
  int E, k, renormalize;
  int32_t* ids;
  float* w;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* inv_pos;
  uint32_t* counter;      // zero before the call; left zero
};
bool front_fits(int64_t T, int64_t H, int k);
hipError_t launch_front(const FrontArgs& f, bool int8, hipStream_t stream);
hipError_t launch_unpermute(const float* o, const int32_t* inv_pos, const float* w, int64_t T, int k, int64_t H,
                            void* y, int bf16_out, hipStream_t stream);
// row_src[p] = f and row_scale[p] = a_scale[p] * w[f] for every routed index f (inv_pos[f] = p >= 0)
hipError_t launch_row_sources(const int32_t* inv_pos, const float* w, const float* a_scale, int64_t R,
                              int64_t M_total, int32_t* row_src, float* row_scale, hipStream_t stream);
// y[t] = sum over j of o_tok[t k + j] for the routed j, j ascending
hipError_t launch_combine(const float* o_tok, const int32_t* inv_pos, int64_t T, int k, int64_t H, void* y,
                          int bf16_out, hipStream_t stream);

}  // namespace w4a8
