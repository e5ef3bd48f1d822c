// C ABI of the W4A8 MoE layer: host-side argument checks, then kernel
// launches on the caller's stream.  Every check runs before anything is
// enqueued, so an argument error means no work was launched (a failed launch,
// W4A8_ERR_HIP, may follow launches of the same call that were enqueued).
#include "w4a8_moe.h"

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return W4A8_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

// 1 if the current device is a gfx950; fills the error detail otherwise.
int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(W4A8_ERR_DEVICE, "no usable HIP device (%s)", hipGetErrorString(e));
  }
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_device_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return W4A8_OK;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(W4A8_ERR_DEVICE, "hipGetDeviceProperties(%d) failed (%s)", dev, hipGetErrorString(e));
  }
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < kMaxDevices) g_device_ok[dev].store(good ? 1 : 2, std::memory_order_relaxed);
  if (!good)
    return fail(W4A8_ERR_DEVICE, "device %d is %s; this library runs on gfx950 (MI355X) only", dev,
                prop.gcnArchName);
  return W4A8_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(W4A8_ERR_HIP, "%s: launch failed (%s)", what, hipGetErrorString(e));
  return ok();
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxRows = (int64_t)1 << 31;   // row indices are int32

}  // namespace

extern "C" {

const char* w4a8_moe_status_string(int status) {
  switch (status) {
    case W4A8_OK: return "W4A8_OK";
    case W4A8_ERR_NULL: return "W4A8_ERR_NULL";
    case W4A8_ERR_SHAPE: return "W4A8_ERR_SHAPE";
    case W4A8_ERR_ALIGN: return "W4A8_ERR_ALIGN";
    case W4A8_ERR_DEVICE: return "W4A8_ERR_DEVICE";
    case W4A8_ERR_HIP: return "W4A8_ERR_HIP";
    case W4A8_ERR_WORKSPACE: return "W4A8_ERR_WORKSPACE";
    default: return "W4A8_ERR_UNKNOWN";
  }
}

const char* w4a8_moe_last_error(void) { return g_last_error.c_str(); }

int w4a8_moe_device_supported(void) { return check_device() == W4A8_OK ? 1 : 0; }

int w4a8_moe_quant_act(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x, uint8_t* qx, float* sx,
                       void* stream) {
  if (T < 0 || T >= kMaxRows) return fail(W4A8_ERR_SHAPE, "quant_act: T=%lld out of range", (long long)T);
  if (H <= 0 || H % 128) return fail(W4A8_ERR_SHAPE, "quant_act: H=%lld must be a positive multiple of 128",
                                     (long long)H);
  if (ld_x < H || ld_x % 8)
    return fail(W4A8_ERR_SHAPE, "quant_act: ld_x=%lld must be >= H and a multiple of 8", (long long)ld_x);
  if (T == 0) return ok();
  if (!x_bf16 || !qx || !sx) return fail(W4A8_ERR_NULL, "quant_act: null pointer");
  if (!aligned(x_bf16, 16) || !aligned(qx, 8) || !aligned(sx, 4))
    return fail(W4A8_ERR_ALIGN, "quant_act: x must be 16-byte, qx 8-byte, sx 4-byte aligned");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_quant_act(x_bf16, T, H, ld_x, qx, sx, as_stream(stream)), "quant_act");
}

int w4a8_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renormalize, int32_t* ids,
                   float* w, void* stream) {
  if (T < 0) return fail(W4A8_ERR_SHAPE, "route: T=%lld < 0", (long long)T);
  if (E < 1 || E > 1024 || k < 1 || k > E)
    return fail(W4A8_ERR_SHAPE, "route: need 1 <= k <= E <= 1024 (k=%d, E=%d)", k, E);
  if (T * (int64_t)k >= kMaxRows) return fail(W4A8_ERR_SHAPE, "route: T*k must be < 2^31");
  if (T == 0) return ok();
  if (!logits || !ids || !w) return fail(W4A8_ERR_NULL, "route: null pointer");
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(w, 4))
    return fail(W4A8_ERR_ALIGN, "route: arrays must be 4-byte aligned");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_route(logits, T, E, k, renormalize ? 1 : 0, ids, w, as_stream(stream)), "route");
}

int64_t w4a8_moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || T * (int64_t)k >= kMaxRows) return -1;
  return w4a8::permute_workspace_bytes(T * (int64_t)k, E);
}

int w4a8_moe_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* offsets, int32_t* row_token,
                     int32_t* inv_pos, void* workspace, int64_t workspace_bytes, void* stream) {
  if (T < 0) return fail(W4A8_ERR_SHAPE, "permute: T=%lld < 0", (long long)T);
  if (E < 1 || E > 1024 || k < 1 || k > E)
    return fail(W4A8_ERR_SHAPE, "permute: need 1 <= k <= E <= 1024 (k=%d, E=%d)", k, E);
  if (T * (int64_t)k >= kMaxRows) return fail(W4A8_ERR_SHAPE, "permute: T*k must be < 2^31");
  if (!offsets || !workspace) return fail(W4A8_ERR_NULL, "permute: null offsets or workspace");
  if (T > 0 && (!ids || !row_token || !inv_pos)) return fail(W4A8_ERR_NULL, "permute: null pointer");
  const int64_t need = w4a8::permute_workspace_bytes(T * (int64_t)k, E);
  if (workspace_bytes < need)
    return fail(W4A8_ERR_WORKSPACE, "permute: workspace of %lld bytes, need %lld", (long long)workspace_bytes,
                (long long)need);
  if (!aligned(ids, 4) || !aligned(offsets, 4) || !aligned(row_token, 4) || !aligned(inv_pos, 4) ||
      !aligned(workspace, 4))
    return fail(W4A8_ERR_ALIGN, "permute: arrays must be 4-byte aligned");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_permute(ids, T * (int64_t)k, k, E, offsets, row_token, inv_pos,
                                       static_cast<int32_t*>(workspace), as_stream(stream)),
                  "permute");
}

int w4a8_moe_permute_noalloc(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* offsets,
                             int32_t* row_token, int32_t* inv_pos, void* stream) {
  if (T < 0) return fail(W4A8_ERR_SHAPE, "permute_noalloc: T=%lld < 0", (long long)T);
  if (E < 1 || E > 1024 || k < 1 || k > E)
    return fail(W4A8_ERR_SHAPE, "permute_noalloc: need 1 <= k <= E <= 1024 (k=%d, E=%d)", k, E);
  if (T * (int64_t)k >= kMaxRows) return fail(W4A8_ERR_SHAPE, "permute_noalloc: T*k must be < 2^31");
  const int64_t need = w4a8::permute_workspace_bytes(T * (int64_t)k, E);
  if (need > w4a8::kPermScratchBytes)
    return fail(W4A8_ERR_WORKSPACE, "permute_noalloc: T=%lld, k=%d, E=%d need %lld bytes of scratch; the library "
                "holds %lld (use w4a8_moe_permute with a workspace)", (long long)T, k, E, (long long)need,
                (long long)w4a8::kPermScratchBytes);
  if (!offsets) return fail(W4A8_ERR_NULL, "permute_noalloc: null offsets");
  if (T > 0 && (!ids || !row_token || !inv_pos)) return fail(W4A8_ERR_NULL, "permute_noalloc: null pointer");
  if (!aligned(ids, 4) || !aligned(offsets, 4) || !aligned(row_token, 4) || !aligned(inv_pos, 4))
    return fail(W4A8_ERR_ALIGN, "permute_noalloc: arrays must be 4-byte aligned");
  if (int st = check_device()) return st;
  int32_t* scratch = nullptr;
  if (hipError_t e = w4a8::permute_scratch(&scratch); e != hipSuccess)
    return fail(W4A8_ERR_HIP, "permute_noalloc: no address for the library's scratch buffer (%s)",
                hipGetErrorString(e));
  (void)hipGetLastError();
  return launched(w4a8::launch_permute(ids, T * (int64_t)k, k, E, offsets, row_token, inv_pos, scratch,
                                       as_stream(stream)),
                  "permute_noalloc");
}

// steps 1-3: the rules of w4a8_moe_quant_act[_i8], w4a8_moe_route and w4a8_moe_permute together
static int run_front(const char* name, const uint16_t* x, int64_t T, int64_t H, int64_t ld_x, void* qx, float* sx,
                     int32_t* rowsum, bool int8, const float* logits, int32_t E, int32_t k, int32_t renormalize,
                     int32_t* ids, float* w, int32_t* offsets, int32_t* row_token, int32_t* inv_pos,
                     void* workspace, int64_t workspace_bytes, uint32_t* counter, void* stream) {
  if (T < 0 || T >= kMaxRows) return fail(W4A8_ERR_SHAPE, "%s: T=%lld out of range", name, (long long)T);
  if (H <= 0 || H % 128)
    return fail(W4A8_ERR_SHAPE, "%s: H=%lld must be a positive multiple of 128", name, (long long)H);
  if (ld_x < H || ld_x % 8)
    return fail(W4A8_ERR_SHAPE, "%s: ld_x=%lld must be >= H and a multiple of 8", name, (long long)ld_x);
  if (E < 1 || E > 1024 || k < 1 || k > E)
    return fail(W4A8_ERR_SHAPE, "%s: need 1 <= k <= E <= 1024 (k=%d, E=%d)", name, k, E);
  if (T * (int64_t)k >= kMaxRows) return fail(W4A8_ERR_SHAPE, "%s: T*k must be < 2^31", name);
  if (!offsets || !workspace || !counter) return fail(W4A8_ERR_NULL, "%s: null offsets, workspace or counter", name);
  if (T > 0 && (!x || !qx || !sx || !logits || !ids || !w || !row_token || !inv_pos || (int8 && !rowsum)))
    return fail(W4A8_ERR_NULL, "%s: null pointer", name);
  const int64_t need = w4a8::permute_workspace_bytes(T * (int64_t)k, E);
  if (workspace_bytes < need)
    return fail(W4A8_ERR_WORKSPACE, "%s: workspace of %lld bytes, need %lld", name, (long long)workspace_bytes,
                (long long)need);
  if (!aligned(x, 16) || !aligned(qx, 8) || !aligned(sx, 4) || !aligned(rowsum, 4) || !aligned(logits, 4) ||
      !aligned(ids, 4) || !aligned(w, 4) || !aligned(offsets, 4) || !aligned(row_token, 4) ||
      !aligned(inv_pos, 4) || !aligned(workspace, 4) || !aligned(counter, 4))
    return fail(W4A8_ERR_ALIGN, "%s: x must be 16-byte, qx 8-byte, the other arrays 4-byte aligned", name);
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  hipStream_t st = as_stream(stream);
  if (w4a8::front_fits(T, H, k)) {
    const w4a8::FrontArgs f{x, T, H, ld_x, static_cast<uint8_t*>(qx), sx, rowsum, logits, E, k, renormalize ? 1 : 0,
                            ids, w, offsets, row_token, inv_pos, counter};
    return launched(w4a8::launch_front(f, int8, st), name);
  }
  // other shapes: the three kernels one after the other (the counter is not used)
  if (T > 0) {
    const hipError_t e = int8 ? w4a8::launch_quant_act_i8(x, T, H, ld_x, static_cast<int8_t*>(qx), sx, rowsum, st)
                              : w4a8::launch_quant_act(x, T, H, ld_x, static_cast<uint8_t*>(qx), sx, st);
    if (e != hipSuccess) return launched(e, name);
    if (hipError_t e2 = w4a8::launch_route(logits, T, E, k, renormalize ? 1 : 0, ids, w, st); e2 != hipSuccess)
      return launched(e2, name);
  }
  return launched(w4a8::launch_permute(ids, T * (int64_t)k, k, E, offsets, row_token, inv_pos,
                                       static_cast<int32_t*>(workspace), st),
                  name);
}

int w4a8_moe_front(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x, uint8_t* qx, float* sx,
                   const float* logits, int32_t E, int32_t k, int32_t renormalize, int32_t* ids, float* w,
                   int32_t* offsets, int32_t* row_token, int32_t* inv_pos, void* workspace, int64_t workspace_bytes,
                   uint32_t* counter, void* stream) {
  return run_front("front", x_bf16, T, H, ld_x, qx, sx, nullptr, false, logits, E, k, renormalize, ids, w, offsets,
                   row_token, inv_pos, workspace, workspace_bytes, counter, stream);
}

int w4a8_moe_front_i8(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x, int8_t* qx, float* sx,
                      int32_t* rowsum, const float* logits, int32_t E, int32_t k, int32_t renormalize, int32_t* ids,
                      float* w, int32_t* offsets, int32_t* row_token, int32_t* inv_pos, void* workspace,
                      int64_t workspace_bytes, uint32_t* counter, void* stream) {
  return run_front("front_i8", x_bf16, T, H, ld_x, qx, sx, rowsum, true, logits, E, k, renormalize, ids, w,
                   offsets, row_token, inv_pos, workspace, workspace_bytes, counter, stream);
}

// ---- grouped GEMMs: three weight forms, plain or with the fused SwiGLU
// epilogue, on the row-major stored weights or on the GEMM storage
enum class Form { kG128, kChannel, kMx };

// W4A8_GG_AUTO: the stream kernel while no expert has more than kAutoStreamRows
// rows and the average expert at most kAutoStreamAvg.  Measured gate/up GEMM times
// on the decode shape (H 6144, I 2048, 256 experts, top-8, uniform routing; stream
// against tiled): 256 tokens (8 rows on average, 18 at most) 0.544 against 0.561
// ms; 384 tokens (12, 24) 0.581 against 0.569; 512 (16, 33) 0.635 against 0.578;
// 1024 (32, 51) 0.854 against 0.625.  Zipf(1.1)-skewed routing at 128-384 tokens
// (126-376 rows in the hottest expert) favours the tiled kernel by 22-36%.
constexpr int32_t kAutoStreamRows = 20;
constexpr int32_t kAutoStreamAvg = 10;

// Checks every argument of one grouped GEMM, then launches it.  fused: N is
// 2I (gate and up rows) and out is act [M_total][I] with pmax [M_total][I/64].
// row_major: the weights as stored (N % 16), else the GEMM storage (N % 64).
static int run_gemm(const char* name, Form form, bool fused, bool row_major, const void* a, const float* a_scale,
                    const int32_t* a_rowsum, const int32_t* a_rows, int64_t M_total, const int32_t* offsets,
                    int32_t E, const void* w, const void* s, int64_t N, int64_t K, float* out, float* pmax,
                    int32_t algo, void* stream, const int32_t* out_rows = nullptr) {
  if (M_total < 0 || M_total >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "%s: M_total=%lld out of range", name, (long long)M_total);
  if (E < 1 || E > 1024) return fail(W4A8_ERR_SHAPE, "%s: E=%d must be in [1, 1024]", name, E);
  if (fused) {
    if (N <= 0 || (N / 2) % 128 || N >= kMaxRows)
      return fail(W4A8_ERR_SHAPE, "%s: I=%lld must be a positive multiple of 128", name, (long long)(N / 2));
  } else {
    const int64_t mult = row_major ? 16 : 64;
    if (N <= 0 || N % mult || N >= kMaxRows)
      return fail(W4A8_ERR_SHAPE, "%s: N=%lld must be a positive multiple of %lld", name, (long long)N,
                  (long long)mult);
  }
  if (K <= 0 || K % 128 || K >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 128", name, (long long)K);
  if (form == Form::kChannel && K > (int64_t)1 << 20)
    return fail(W4A8_ERR_SHAPE, "%s: K=%lld would overflow the int32 sums", name, (long long)K);
  if (algo < W4A8_GG_AUTO || algo > W4A8_GG_TILED) return fail(W4A8_ERR_SHAPE, "%s: unknown algo %d", name, algo);
  if (M_total == 0) return ok();
  if (!a || !a_scale || !offsets || !w || !s || !out || (fused && !pmax) || (form == Form::kChannel && !a_rowsum))
    return fail(W4A8_ERR_NULL, "%s: null pointer", name);
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(out, 16) || !aligned(a_scale, 4) || !aligned(s, 4) ||
      !aligned(offsets, 4) || !aligned(a_rows, 4) || !aligned(pmax, 4) || !aligned(a_rowsum, 4) ||
      !aligned(out_rows, 4))
    return fail(W4A8_ERR_ALIGN, "%s: a, the weights and the output must be 16-byte aligned, the rest 4-byte", name);
  if (int st = check_device()) return st;
  w4a8::GemmArgs g{static_cast<const uint8_t*>(a), a_scale, form == Form::kChannel ? a_rowsum : nullptr, a_rows,
                   M_total, offsets, E, static_cast<const int32_t*>(w), static_cast<const float*>(s), N, K, out};
  g.pmax = fused ? pmax : nullptr;
  g.mx = form == Form::kMx;
  g.row_major = row_major;
  g.out_rows = out_rows;
  if (row_major) algo = W4A8_GG_STREAM;   // the tiled kernel reads the GEMM storage only
  (void)hipGetLastError();
  if (algo == W4A8_GG_AUTO) {
    // Where M_total alone does not settle it, both kernels are launched and the one
    // the largest expert does not call for returns at once (the largest expert is
    // known on the device only; the two launches cost 1.5% of the layer time at
    // uniform decode, against 22-36% saved on skewed batches).
    if (M_total <= kAutoStreamRows || !w4a8::tiled_fits(g)) algo = W4A8_GG_STREAM;
    else if (M_total > kAutoStreamAvg * (int64_t)E) algo = W4A8_GG_TILED;
    else {
      g.sel_rows = kAutoStreamRows;
      if (int st = launched(w4a8::launch_gg_tiled(g, as_stream(stream)), name)) return st;
      return launched(w4a8::launch_gg_stream(g, as_stream(stream)), name);
    }
  }
  if (algo == W4A8_GG_STREAM) return launched(w4a8::launch_gg_stream(g, as_stream(stream)), name);
  return launched(w4a8::launch_gg_tiled(g, as_stream(stream)), name);
}

int w4a8_moe_grouped_gemm(const uint8_t* a, const float* a_scale, const int32_t* a_rows, int64_t M_total,
                          const int32_t* offsets, int32_t E, const int32_t* w_packed, const float* w_scale,
                          int64_t N, int64_t K, float* out, void* stream) {
  return run_gemm("grouped_gemm", Form::kG128, false, true, a, a_scale, nullptr, a_rows, M_total, offsets, E,
                  w_packed, w_scale, N, K, out, nullptr, W4A8_GG_AUTO, stream);
}

int w4a8_moe_grouped_gemm_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows, int64_t M_total,
                                    const int32_t* offsets, int32_t E, const int32_t* w_blk, const float* s_blk,
                                    int64_t N, int64_t K, float* out, int32_t algo, void* stream) {
  return run_gemm("grouped_gemm_prepacked", Form::kG128, false, false, a, a_scale, nullptr, a_rows, M_total,
                  offsets, E, w_blk, s_blk, N, K, out, nullptr, algo, stream);
}

int w4a8_moe_grouped_gemm_swiglu(const uint8_t* a, const float* a_scale, const int32_t* a_rows, int64_t M_total,
                                 const int32_t* offsets, int32_t E, const int32_t* w13, const float* s13, int64_t I,
                                 int64_t K, float* act, float* act_pmax, void* stream) {
  return run_gemm("grouped_gemm_swiglu", Form::kG128, true, true, a, a_scale, nullptr, a_rows, M_total, offsets, E,
                  w13, s13, 2 * I, K, act, act_pmax, W4A8_GG_AUTO, stream);
}

int w4a8_moe_grouped_gemm_swiglu_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                           int64_t M_total, const int32_t* offsets, int32_t E, const int32_t* w13,
                                           const float* s13, int64_t I, int64_t K, float* act, float* act_pmax,
                                           int32_t algo, void* stream) {
  return run_gemm("grouped_gemm_swiglu_prepacked", Form::kG128, true, false, a, a_scale, nullptr, a_rows, M_total,
                  offsets, E, w13, s13, 2 * I, K, act, act_pmax, algo, stream);
}

int w4a8_moe_grouped_gemm_i8(const int8_t* a, const float* a_scale, const int32_t* a_rowsum, const int32_t* a_rows,
                             int64_t M_total, const int32_t* offsets, int32_t E, const int32_t* w_packed,
                             const float* w_scale, int64_t N, int64_t K, float* out, void* stream) {
  return run_gemm("grouped_gemm_i8", Form::kChannel, false, true, a, a_scale, a_rowsum, a_rows, M_total, offsets, E,
                  w_packed, w_scale, N, K, out, nullptr, W4A8_GG_AUTO, stream);
}

int w4a8_moe_grouped_gemm_i8_prepacked(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                       const int32_t* a_rows, int64_t M_total, const int32_t* offsets, int32_t E,
                                       const int32_t* w_blk, const float* w_scale, int64_t N, int64_t K, float* out,
                                       int32_t algo, void* stream) {
  return run_gemm("grouped_gemm_i8_prepacked", Form::kChannel, false, false, a, a_scale, a_rowsum, a_rows, M_total,
                  offsets, E, w_blk, w_scale, N, K, out, nullptr, algo, stream);
}

int w4a8_moe_grouped_gemm_swiglu_i8(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                    const int32_t* a_rows, int64_t M_total, const int32_t* offsets, int32_t E,
                                    const int32_t* w13, const float* s13, int64_t I, int64_t K, float* act,
                                    float* act_pmax, void* stream) {
  return run_gemm("grouped_gemm_swiglu_i8", Form::kChannel, true, true, a, a_scale, a_rowsum, a_rows, M_total,
                  offsets, E, w13, s13, 2 * I, K, act, act_pmax, W4A8_GG_AUTO, stream);
}

int w4a8_moe_grouped_gemm_swiglu_i8_prepacked(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                              const int32_t* a_rows, int64_t M_total, const int32_t* offsets,
                                              int32_t E, const int32_t* w13, const float* s13, int64_t I, int64_t K,
                                              float* act, float* act_pmax, int32_t algo, void* stream) {
  return run_gemm("grouped_gemm_swiglu_i8_prepacked", Form::kChannel, true, false, a, a_scale, a_rowsum, a_rows,
                  M_total, offsets, E, w13, s13, 2 * I, K, act, act_pmax, algo, stream);
}

int w4a8_moe_grouped_gemm_mxfp4(const uint8_t* a, const float* a_scale, const int32_t* a_rows, int64_t M_total,
                                const int32_t* offsets, int32_t E, const uint8_t* w_packed, const uint8_t* w_scale,
                                int64_t N, int64_t K, float* out, void* stream) {
  return run_gemm("grouped_gemm_mxfp4", Form::kMx, false, true, a, a_scale, nullptr, a_rows, M_total, offsets, E,
                  w_packed, w_scale, N, K, out, nullptr, W4A8_GG_AUTO, stream);
}

int w4a8_moe_grouped_gemm_mxfp4_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                          int64_t M_total, const int32_t* offsets, int32_t E, const uint8_t* w_blk,
                                          const uint8_t* s_blk, int64_t N, int64_t K, float* out, int32_t algo,
                                          void* stream) {
  return run_gemm("grouped_gemm_mxfp4_prepacked", Form::kMx, false, false, a, a_scale, nullptr, a_rows, M_total,
                  offsets, E, w_blk, s_blk, N, K, out, nullptr, algo, stream);
}

// the scatter forms: GEMM row p stored as row row_dst[p] of out
int w4a8_moe_grouped_gemm_scatter_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                            int64_t M_total, const int32_t* offsets, int32_t E, const int32_t* w_blk,
                                            const float* s_blk, int64_t N, int64_t K, const int32_t* row_dst,
                                            float* out, int32_t algo, void* stream) {
  if (M_total > 0 && !row_dst) return fail(W4A8_ERR_NULL, "grouped_gemm_scatter_prepacked: null row_dst");
  return run_gemm("grouped_gemm_scatter_prepacked", Form::kG128, false, false, a, a_scale, nullptr, a_rows,
                  M_total, offsets, E, w_blk, s_blk, N, K, out, nullptr, algo, stream, row_dst);
}

int w4a8_moe_grouped_gemm_scatter_i8_prepacked(const int8_t* a, const float* a_scale, const int32_t* a_rowsum,
                                               const int32_t* a_rows, int64_t M_total, const int32_t* offsets,
                                               int32_t E, const int32_t* w_blk, const float* w_scale, int64_t N,
                                               int64_t K, const int32_t* row_dst, float* out, int32_t algo,
                                               void* stream) {
  if (M_total > 0 && !row_dst) return fail(W4A8_ERR_NULL, "grouped_gemm_scatter_i8_prepacked: null row_dst");
  return run_gemm("grouped_gemm_scatter_i8_prepacked", Form::kChannel, false, false, a, a_scale, a_rowsum, a_rows,
                  M_total, offsets, E, w_blk, w_scale, N, K, out, nullptr, algo, stream, row_dst);
}

int w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                                  int64_t M_total, const int32_t* offsets, int32_t E,
                                                  const uint8_t* w_blk, const uint8_t* s_blk, int64_t N, int64_t K,
                                                  const int32_t* row_dst, float* out, int32_t algo, void* stream) {
  if (M_total > 0 && !row_dst) return fail(W4A8_ERR_NULL, "grouped_gemm_scatter_mxfp4_prepacked: null row_dst");
  return run_gemm("grouped_gemm_scatter_mxfp4_prepacked", Form::kMx, false, false, a, a_scale, nullptr, a_rows,
                  M_total, offsets, E, w_blk, s_blk, N, K, out, nullptr, algo, stream, row_dst);
}

int w4a8_moe_grouped_gemm_swiglu_mxfp4(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                       int64_t M_total, const int32_t* offsets, int32_t E, const uint8_t* w13,
                                       const uint8_t* s13, int64_t I, int64_t K, float* act, float* act_pmax,
                                       void* stream) {
  return run_gemm("grouped_gemm_swiglu_mxfp4", Form::kMx, true, true, a, a_scale, nullptr, a_rows, M_total, offsets,
                  E, w13, s13, 2 * I, K, act, act_pmax, W4A8_GG_AUTO, stream);
}

int w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked(const uint8_t* a, const float* a_scale, const int32_t* a_rows,
                                                 int64_t M_total, const int32_t* offsets, int32_t E,
                                                 const uint8_t* w13, const uint8_t* s13, int64_t I, int64_t K,
                                                 float* act, float* act_pmax, int32_t algo, void* stream) {
  return run_gemm("grouped_gemm_swiglu_mxfp4_prepacked", Form::kMx, true, false, a, a_scale, nullptr, a_rows,
                  M_total, offsets, E, w13, s13, 2 * I, K, act, act_pmax, algo, stream);
}

int w4a8_moe_swiglu(const float* h, int64_t M, int64_t I, uint8_t* qa, float* sa, void* stream) {
  if (M < 0 || M >= kMaxRows) return fail(W4A8_ERR_SHAPE, "swiglu: M=%lld out of range", (long long)M);
  if (I <= 0 || I % 128) return fail(W4A8_ERR_SHAPE, "swiglu: I=%lld must be a positive multiple of 128",
                                     (long long)I);
  if (M == 0) return ok();
  if (!h || !qa || !sa) return fail(W4A8_ERR_NULL, "swiglu: null pointer");
  if (!aligned(h, 16) || !aligned(qa, 4) || !aligned(sa, 4))
    return fail(W4A8_ERR_ALIGN, "swiglu: h must be 16-byte, qa and sa 4-byte aligned");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_swiglu(h, M, I, qa, sa, as_stream(stream)), "swiglu");
}

int w4a8_moe_quantize_weights(const float* w, int64_t rows, int64_t K, int32_t mse_clip, int32_t* w_packed,
                              float* w_scale, void* stream) {
  if (rows < 0 || rows >= kMaxRows) return fail(W4A8_ERR_SHAPE, "quantize_weights: rows=%lld out of range",
                                                (long long)rows);
  if (K <= 0 || K % 128) return fail(W4A8_ERR_SHAPE, "quantize_weights: K=%lld must be a positive multiple of 128",
                                     (long long)K);
  if (rows == 0) return ok();
  if (!w || !w_packed || !w_scale) return fail(W4A8_ERR_NULL, "quantize_weights: null pointer");
  if (!aligned(w, 8) || !aligned(w_packed, 4) || !aligned(w_scale, 4))
    return fail(W4A8_ERR_ALIGN, "quantize_weights: w must be 8-byte aligned, w_packed and w_scale 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_wquant(w, rows, K, mse_clip ? 1 : 0, w_packed, w_scale, as_stream(stream)),
                  "quantize_weights");
}

int w4a8_moe_quant_act_i8(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ld_x, int8_t* qx, float* sx,
                          int32_t* rowsum, void* stream) {
  if (T < 0 || T >= kMaxRows) return fail(W4A8_ERR_SHAPE, "quant_act_i8: T=%lld out of range", (long long)T);
  if (H <= 0 || H % 128) return fail(W4A8_ERR_SHAPE, "quant_act_i8: H=%lld must be a positive multiple of 128",
                                     (long long)H);
  if (ld_x < H || ld_x % 8) return fail(W4A8_ERR_SHAPE, "quant_act_i8: ld_x=%lld must be >= H and a multiple of 8",
                                        (long long)ld_x);
  if (T == 0) return ok();
  if (!x_bf16 || !qx || !sx || !rowsum) return fail(W4A8_ERR_NULL, "quant_act_i8: null pointer");
  if (!aligned(x_bf16, 16) || !aligned(qx, 8) || !aligned(sx, 4) || !aligned(rowsum, 4))
    return fail(W4A8_ERR_ALIGN, "quant_act_i8: x must be 16-byte aligned, qx 8-byte, sx and rowsum 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_quant_act_i8(x_bf16, T, H, ld_x, qx, sx, rowsum, as_stream(stream)),
                  "quant_act_i8");
}

int w4a8_moe_swiglu_i8(const float* h, int64_t M, int64_t I, int8_t* qa, float* sa, int32_t* rowsum,
                       void* stream) {
  if (M < 0 || M >= kMaxRows) return fail(W4A8_ERR_SHAPE, "swiglu_i8: M=%lld out of range", (long long)M);
  if (I <= 0 || I % 128) return fail(W4A8_ERR_SHAPE, "swiglu_i8: I=%lld must be a positive multiple of 128",
                                     (long long)I);
  if (M == 0) return ok();
  if (!h || !qa || !sa || !rowsum) return fail(W4A8_ERR_NULL, "swiglu_i8: null pointer");
  if (!aligned(h, 16) || !aligned(qa, 4) || !aligned(sa, 4) || !aligned(rowsum, 4))
    return fail(W4A8_ERR_ALIGN, "swiglu_i8: h must be 16-byte aligned, qa, sa and rowsum 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_swiglu_i8(h, M, I, qa, sa, rowsum, as_stream(stream)), "swiglu_i8");
}

int w4a8_moe_quantize_weights_channel(const float* w, int64_t rows, int64_t K, int32_t* w_packed, float* w_scale,
                                      void* stream) {
  if (rows < 0 || rows >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "quantize_weights_channel: rows=%lld out of range", (long long)rows);
  if (K <= 0 || K % 128)
    return fail(W4A8_ERR_SHAPE, "quantize_weights_channel: K=%lld must be a positive multiple of 128", (long long)K);
  if (rows == 0) return ok();
  if (!w || !w_packed || !w_scale) return fail(W4A8_ERR_NULL, "quantize_weights_channel: null pointer");
  if (!aligned(w, 8) || !aligned(w_packed, 4) || !aligned(w_scale, 4))
    return fail(W4A8_ERR_ALIGN, "quantize_weights_channel: w must be 8-byte aligned, w_packed and w_scale 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_wquant_channel(w, rows, K, w_packed, w_scale, as_stream(stream)),
                  "quantize_weights_channel");
}

int w4a8_moe_requant(const float* act, const float* act_pmax, int64_t M, int64_t I, uint8_t* qa, float* sa,
                     void* stream) {
  if (M < 0 || M >= kMaxRows) return fail(W4A8_ERR_SHAPE, "requant: M=%lld out of range", (long long)M);
  if (I <= 0 || I % 128) return fail(W4A8_ERR_SHAPE, "requant: I=%lld must be a positive multiple of 128",
                                     (long long)I);
  if (M == 0) return ok();
  if (!act || !act_pmax || !qa || !sa) return fail(W4A8_ERR_NULL, "requant: null pointer");
  if (!aligned(act, 16) || !aligned(act_pmax, 4) || !aligned(qa, 4) || !aligned(sa, 4))
    return fail(W4A8_ERR_ALIGN, "requant: act must be 16-byte aligned, act_pmax, qa and sa 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_requant(act, act_pmax, M, I, qa, sa, as_stream(stream)), "requant");
}

int w4a8_moe_requant_i8(const float* act, const float* act_pmax, int64_t M, int64_t I, int8_t* qa, float* sa,
                        int32_t* rowsum, void* stream) {
  if (M < 0 || M >= kMaxRows) return fail(W4A8_ERR_SHAPE, "requant_i8: M=%lld out of range", (long long)M);
  if (I <= 0 || I % 128) return fail(W4A8_ERR_SHAPE, "requant_i8: I=%lld must be a positive multiple of 128",
                                     (long long)I);
  if (M == 0) return ok();
  if (!act || !act_pmax || !qa || !sa || !rowsum) return fail(W4A8_ERR_NULL, "requant_i8: null pointer");
  if (!aligned(act, 16) || !aligned(act_pmax, 4) || !aligned(qa, 4) || !aligned(sa, 4) || !aligned(rowsum, 4))
    return fail(W4A8_ERR_ALIGN, "requant_i8: act must be 16-byte aligned, act_pmax, qa, sa and rowsum 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_requant_i8(act, act_pmax, M, I, qa, sa, rowsum, as_stream(stream)), "requant_i8");
}

int w4a8_moe_quantize_weights_mxfp4(const float* w, int64_t rows, int64_t K, uint8_t* w_packed, uint8_t* w_scale,
                                    void* stream) {
  if (rows < 0 || rows >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "quantize_weights_mxfp4: rows=%lld out of range", (long long)rows);
  if (K <= 0 || K % 32 || K >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "quantize_weights_mxfp4: K=%lld must be a positive multiple of 32 below 2^31",
                (long long)K);
  if (rows == 0) return ok();
  if (!w || !w_packed || !w_scale) return fail(W4A8_ERR_NULL, "quantize_weights_mxfp4: null pointer");
  if (!aligned(w, 16) || !aligned(w_packed, 2))
    return fail(W4A8_ERR_ALIGN, "quantize_weights_mxfp4: w must be 16-byte aligned, w_packed 2-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_wquant_mxfp4(w, rows, K, w_packed, w_scale, as_stream(stream)),
                  "quantize_weights_mxfp4");
}

int w4a8_moe_prepack_mxfp4(const uint8_t* w_packed, const uint8_t* w_scale, int32_t E, int64_t N, int64_t K,
                           uint8_t* w_blk, uint8_t* s_blk, void* stream) {
  if (E < 0 || E > 1024) return fail(W4A8_ERR_SHAPE, "prepack_mxfp4: E=%d must be in [0, 1024]", E);
  if (N <= 0 || N % 16 || N >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "prepack_mxfp4: N=%lld must be a positive multiple of 16", (long long)N);
  if (K <= 0 || K % 128 || K >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "prepack_mxfp4: K=%lld must be a positive multiple of 128", (long long)K);
  if (E == 0) return ok();
  if (!w_packed || !w_scale || !w_blk || !s_blk) return fail(W4A8_ERR_NULL, "prepack_mxfp4: null pointer");
  if (!aligned(w_packed, 16) || !aligned(w_blk, 16) || !aligned(w_scale, 4) || !aligned(s_blk, 4))
    return fail(W4A8_ERR_ALIGN, "prepack_mxfp4: weights must be 16-byte aligned, scales 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_prepack(w_packed, w_scale, E, N, K, 0, w_blk, s_blk, as_stream(stream)), "prepack_mxfp4");
}

int w4a8_moe_prepack_int4(const int32_t* w_packed, const float* w_scale, int32_t E, int64_t N, int64_t K,
                          int32_t* w_blk, float* s_blk, void* stream) {
  if (E < 0 || E > 1024) return fail(W4A8_ERR_SHAPE, "prepack_int4: E=%d must be in [0, 1024]", E);
  if (N <= 0 || N % 16 || N >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "prepack_int4: N=%lld must be a positive multiple of 16", (long long)N);
  if (K <= 0 || K % 128 || K >= kMaxRows)
    return fail(W4A8_ERR_SHAPE, "prepack_int4: K=%lld must be a positive multiple of 128", (long long)K);
  if (E == 0) return ok();
  if (!w_packed || !w_blk) return fail(W4A8_ERR_NULL, "prepack_int4: null weight pointer");
  if ((w_scale == nullptr) != (s_blk == nullptr))
    return fail(W4A8_ERR_NULL, "prepack_int4: w_scale and s_blk must both be given or both be null");
  if (!aligned(w_packed, 16) || !aligned(w_blk, 16) || !aligned(w_scale, 4) || !aligned(s_blk, 4))
    return fail(W4A8_ERR_ALIGN, "prepack_int4: weights must be 16-byte aligned, scales 4-byte");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_prepack(w_packed, w_scale, E, N, K, 1, w_blk, s_blk, as_stream(stream)), "prepack_int4");
}

int w4a8_moe_unpermute(const float* o, const int32_t* inv_pos, const float* w, int64_t T, int32_t k, int64_t H,
                       void* y, int32_t y_dtype, void* stream) {
  if (T < 0 || T >= kMaxRows) return fail(W4A8_ERR_SHAPE, "unpermute: T=%lld out of range", (long long)T);
  if (k < 1 || T * (int64_t)k >= kMaxRows) return fail(W4A8_ERR_SHAPE, "unpermute: bad k=%d", k);
  if (H <= 0 || H % 128) return fail(W4A8_ERR_SHAPE, "unpermute: H=%lld must be a positive multiple of 128",
                                     (long long)H);
  if (y_dtype != W4A8_Y_F32 && y_dtype != W4A8_Y_BF16)
    return fail(W4A8_ERR_SHAPE, "unpermute: y_dtype=%d must be W4A8_Y_F32 or W4A8_Y_BF16", y_dtype);
  if (T == 0) return ok();
  if (!o || !inv_pos || !w || !y) return fail(W4A8_ERR_NULL, "unpermute: null pointer");
  if (!aligned(o, 16) || !aligned(inv_pos, 4) || !aligned(w, 4) || !aligned(y, y_dtype == W4A8_Y_F32 ? 16 : 8))
    return fail(W4A8_ERR_ALIGN, "unpermute: o and f32 y must be 16-byte, bf16 y 8-byte aligned");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_unpermute(o, inv_pos, w, T, k, H, y, y_dtype == W4A8_Y_BF16, as_stream(stream)),
                  "unpermute");
}

int w4a8_moe_row_sources(const int32_t* inv_pos, const float* w, const float* a_scale, int64_t T, int32_t k,
                         int64_t M_total, int32_t* row_src, float* row_scale, void* stream) {
  if (T < 0 || T >= kMaxRows) return fail(W4A8_ERR_SHAPE, "row_sources: T=%lld out of range", (long long)T);
  if (k < 1 || T * (int64_t)k >= kMaxRows) return fail(W4A8_ERR_SHAPE, "row_sources: bad k=%d", k);
  if (M_total < 0 || M_total > T * (int64_t)k)
    return fail(W4A8_ERR_SHAPE, "row_sources: M_total=%lld must be in [0, T k]", (long long)M_total);
  if (M_total == 0) return ok();                  // nothing routed: no row to name
  if (!inv_pos || !w || !a_scale || !row_src || !row_scale) return fail(W4A8_ERR_NULL, "row_sources: null pointer");
  if (!aligned(inv_pos, 4) || !aligned(w, 4) || !aligned(a_scale, 4) || !aligned(row_src, 4) ||
      !aligned(row_scale, 4))
    return fail(W4A8_ERR_ALIGN, "row_sources: every array must be 4-byte aligned");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_row_sources(inv_pos, w, a_scale, T * (int64_t)k, M_total, row_src, row_scale,
                                           as_stream(stream)), "row_sources");
}

int w4a8_moe_combine(const float* o_tok, const int32_t* inv_pos, int64_t T, int32_t k, int64_t H, void* y,
                     int32_t y_dtype, void* stream) {
  if (T < 0 || T >= kMaxRows) return fail(W4A8_ERR_SHAPE, "combine: T=%lld out of range", (long long)T);
  if (k < 1 || T * (int64_t)k >= kMaxRows) return fail(W4A8_ERR_SHAPE, "combine: bad k=%d", k);
  if (H <= 0 || H % 128) return fail(W4A8_ERR_SHAPE, "combine: H=%lld must be a positive multiple of 128",
                                     (long long)H);
  if (y_dtype != W4A8_Y_F32 && y_dtype != W4A8_Y_BF16)
    return fail(W4A8_ERR_SHAPE, "combine: y_dtype=%d must be W4A8_Y_F32 or W4A8_Y_BF16", y_dtype);
  if (T == 0) return ok();
  if (!o_tok || !inv_pos || !y) return fail(W4A8_ERR_NULL, "combine: null pointer");
  if (!aligned(o_tok, 16) || !aligned(inv_pos, 4) || !aligned(y, y_dtype == W4A8_Y_F32 ? 16 : 8))
    return fail(W4A8_ERR_ALIGN, "combine: o_tok and f32 y must be 16-byte, bf16 y 8-byte aligned");
  if (int st = check_device()) return st;
  (void)hipGetLastError();
  return launched(w4a8::launch_combine(o_tok, inv_pos, T, k, H, y, y_dtype == W4A8_Y_BF16 ? 1 : 0,
                                       as_stream(stream)), "combine");
}

}  // extern "C"
