// A native caller of the W4A8 MoE C ABI: one layer step on device buffers it
// allocates itself (hipMalloc) and a HIP stream of its own, with no Python and
// no torch, the way a C or C++ serving engine would call the library.
//
//   moe_layer DIR T H I E k
//
// DIR holds the inputs as raw little-endian arrays:
//   x.bin       bf16 bits  uint16 [T][H]
//   logits.bin  fp32       [T][E]
//   w13.bin     int32      [E][2I][H/8]   uint4b8 words, gate rows then up rows
//   s13.bin     fp32       [E][2I][H/128]
//   w2.bin      int32      [E][H][I/8]
//   s2.bin      fp32       [E][H][I/128]
// and receives y.bin, fp32 [T][H].  The step is the layer's: prepack both
// weight sets to the GEMM storage, steps 1-3 in one call, the gate/up GEMM
// with SwiGLU in its epilogue, the re-quantization, the down GEMM and the
// routing-weighted combine, with the automatic kernel choice.
//
// Exit status: 0 on success, 2 when no gfx950 device is present, 1 on any
// other error (the failing call and the library's message are printed).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "w4a8_moe.h"

namespace {

int report(const char* what, int status) {
  std::fprintf(stderr, "%s: %s (%s)\n", what, w4a8_moe_status_string(status), w4a8_moe_last_error());
  return 1;
}

#define CALL(expr)                                  \
  do {                                              \
    const int st_ = (expr);                         \
    if (st_ != W4A8_OK) return report(#expr, st_);  \
  } while (0)

#define HIP_CHECK(expr)                                                              \
  do {                                                                               \
    const hipError_t e_ = (expr);                                                    \
    if (e_ != hipSuccess) {                                                          \
      std::fprintf(stderr, "%s: %s\n", #expr, hipGetErrorString(e_));               \
      return 1;                                                                      \
    }                                                                                \
  } while (0)

// Device allocations, freed when the caller returns.
struct DeviceBuffers {
  std::vector<void*> ptrs;
  bool failed = false;
  ~DeviceBuffers() {
    for (void* p : ptrs) (void)hipFree(p);
  }
  template <typename T>
  T* get(size_t count) {
    void* p = nullptr;
    if (hipMalloc(&p, std::max<size_t>(count, 1) * sizeof(T)) != hipSuccess) {
      failed = true;
      return nullptr;
    }
    ptrs.push_back(p);
    return static_cast<T*>(p);
  }
};

template <typename T>
bool read_array(const std::string& path, std::vector<T>& v) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  const size_t got = std::fread(v.data(), sizeof(T), v.size(), f);
  const bool at_end = std::fgetc(f) == EOF;
  std::fclose(f);
  return got == v.size() && at_end;
}

int run(const std::string& dir, int64_t T, int64_t H, int64_t I, int32_t E, int32_t k) {
  const int64_t R = T * k;
  std::vector<uint16_t> x((size_t)(T * H));
  std::vector<float> logits((size_t)(T * E));
  std::vector<int32_t> w13((size_t)(E * 2 * I * (H / 8))), w2((size_t)(E * H * (I / 8)));
  std::vector<float> s13((size_t)(E * 2 * I * (H / 128))), s2((size_t)(E * H * (I / 128)));
  if (!read_array(dir + "/x.bin", x) || !read_array(dir + "/logits.bin", logits) ||
      !read_array(dir + "/w13.bin", w13) || !read_array(dir + "/s13.bin", s13) ||
      !read_array(dir + "/w2.bin", w2) || !read_array(dir + "/s2.bin", s2)) {
    std::fprintf(stderr, "an input file in %s is missing or has the wrong size\n", dir.c_str());
    return 1;
  }

  DeviceBuffers d;
  uint16_t* x_d = d.get<uint16_t>(x.size());
  float* logits_d = d.get<float>(logits.size());
  int32_t* w13_d = d.get<int32_t>(w13.size());
  float* s13_d = d.get<float>(s13.size());
  int32_t* w2_d = d.get<int32_t>(w2.size());
  float* s2_d = d.get<float>(s2.size());
  int32_t* w13_blk = d.get<int32_t>(w13.size());
  float* s13_blk = d.get<float>(s13.size());
  int32_t* w2_blk = d.get<int32_t>(w2.size());
  float* s2_blk = d.get<float>(s2.size());
  uint8_t* qx = d.get<uint8_t>((size_t)(T * H));
  float* sx = d.get<float>((size_t)T);
  int32_t* ids = d.get<int32_t>((size_t)R);
  float* w = d.get<float>((size_t)R);
  int32_t* offsets = d.get<int32_t>((size_t)E + 1);
  int32_t* row_token = d.get<int32_t>((size_t)R);
  int32_t* inv_pos = d.get<int32_t>((size_t)R);
  const int64_t ws_bytes = w4a8_moe_permute_workspace_bytes(T, k, E);
  uint8_t* workspace = d.get<uint8_t>((size_t)std::max<int64_t>(ws_bytes, 4));
  uint32_t* counter = d.get<uint32_t>(1);
  float* act = d.get<float>((size_t)(R * I));
  float* pmax = d.get<float>((size_t)(R * (I / 64)));
  uint8_t* qa = d.get<uint8_t>((size_t)(R * I));
  float* sa = d.get<float>((size_t)R);
  float* o = d.get<float>((size_t)(R * H));
  float* y = d.get<float>((size_t)(T * H));
  if (d.failed) {
    std::fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }

  hipStream_t stream = nullptr;
  HIP_CHECK(hipStreamCreate(&stream));
  HIP_CHECK(hipMemcpy(x_d, x.data(), x.size() * sizeof(uint16_t), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(logits_d, logits.data(), logits.size() * sizeof(float), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(w13_d, w13.data(), w13.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(s13_d, s13.data(), s13.size() * sizeof(float), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(w2_d, w2.data(), w2.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(s2_d, s2.data(), s2.size() * sizeof(float), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemset(counter, 0, sizeof(uint32_t)));   // the front call's counter starts at zero

  // offline: the experts in the GEMM storage
  CALL(w4a8_moe_prepack_int4(w13_d, s13_d, E, 2 * I, H, w13_blk, s13_blk, stream));
  CALL(w4a8_moe_prepack_int4(w2_d, s2_d, E, H, I, w2_blk, s2_blk, stream));
  // the layer step
  CALL(w4a8_moe_front(x_d, T, H, H, qx, sx, logits_d, E, k, 1, ids, w, offsets, row_token, inv_pos, workspace,
                      ws_bytes, counter, stream));
  CALL(w4a8_moe_grouped_gemm_swiglu_prepacked(qx, sx, row_token, R, offsets, E, w13_blk, s13_blk, I, H, act, pmax,
                                              W4A8_GG_AUTO, stream));
  CALL(w4a8_moe_requant(act, pmax, R, I, qa, sa, stream));
  CALL(w4a8_moe_grouped_gemm_prepacked(qa, sa, nullptr, R, offsets, E, w2_blk, s2_blk, H, I, o, W4A8_GG_AUTO,
                                       stream));
  CALL(w4a8_moe_unpermute(o, inv_pos, w, T, k, H, y, W4A8_Y_F32, stream));
  HIP_CHECK(hipStreamSynchronize(stream));

  std::vector<float> y_h((size_t)(T * H));
  HIP_CHECK(hipMemcpy(y_h.data(), y, y_h.size() * sizeof(float), hipMemcpyDeviceToHost));
  HIP_CHECK(hipStreamDestroy(stream));
  FILE* f = std::fopen((dir + "/y.bin").c_str(), "wb");
  if (!f || std::fwrite(y_h.data(), sizeof(float), y_h.size(), f) != y_h.size()) {
    if (f) std::fclose(f);
    std::fprintf(stderr, "cannot write %s/y.bin\n", dir.c_str());
    return 1;
  }
  std::fclose(f);
  std::printf("moe_layer: T=%lld H=%lld I=%lld E=%d k=%d done\n", (long long)T, (long long)H, (long long)I, E, k);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr, "usage: %s DIR T H I E k\n", argv[0]);
    return 1;
  }
  const int64_t T = std::atoll(argv[2]), H = std::atoll(argv[3]), I = std::atoll(argv[4]);
  const int32_t E = std::atoi(argv[5]), k = std::atoi(argv[6]);
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || H % 128 || I % 128) {
    std::fprintf(stderr, "bad sizes\n");
    return 1;
  }
  if (!w4a8_moe_device_supported()) {
    std::fprintf(stderr, "no gfx950 device: %s\n", w4a8_moe_last_error());
    return 2;
  }
  return run(argv[1], T, H, I, E, k);
}
