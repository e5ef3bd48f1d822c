// Host-only stand-ins for the kernel launchers of the W4A8 MoE library, for the
// sanitizer build of its C ABI (abi.cpp) on a machine without a GPU.
//
// abi.cpp checks every argument on the host, then asks the HIP runtime for
// the device; with no gfx950 present that check fails and no launcher is
// reached.  These definitions only satisfy the linker (and report
// hipErrorNoDevice if one were reached).  permute_workspace_bytes, which the
// argument checks use, restates the library's size rule: one int32 count per
// expert and per block of 1024 routed rows.
#include "kernels.hpp"

namespace w4a8 {

namespace {
hipError_t absent() { return hipErrorNoDevice; }
}  // namespace

int64_t permute_workspace_bytes(int64_t R, int E) {
  const int64_t nblk = (R + 1023) / 1024;
  return (nblk > 0 ? nblk : 1) * (int64_t)E * (int64_t)sizeof(int32_t);
}
hipError_t permute_scratch(int32_t**) { return absent(); }
bool front_fits(int64_t, int64_t, int) { return false; }

hipError_t launch_quant_act(const uint16_t*, int64_t, int64_t, int64_t, uint8_t*, float*, hipStream_t) {
  return absent();
}
hipError_t launch_route(const float*, int64_t, int, int, int, int32_t*, float*, hipStream_t) { return absent(); }
hipError_t launch_permute(const int32_t*, int64_t, int, int, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  return absent();
}
hipError_t launch_gg_stream(const GemmArgs&, hipStream_t) { return absent(); }
hipError_t launch_gg_tiled(const GemmArgs&, hipStream_t) { return absent(); }
bool tiled_fits(const GemmArgs&) { return true; }
hipError_t launch_row_sources(const int32_t*, const float*, const float*, int64_t, int64_t, int32_t*, float*,
                              hipStream_t) {
  return absent();
}
hipError_t launch_combine(const float*, const int32_t*, int64_t, int, int64_t, void*, int, hipStream_t) {
  return absent();
}
hipError_t launch_swiglu(const float*, int64_t, int64_t, uint8_t*, float*, hipStream_t) { return absent(); }
hipError_t launch_quant_act_i8(const uint16_t*, int64_t, int64_t, int64_t, int8_t*, float*, int32_t*, hipStream_t) {
  return absent();
}
hipError_t launch_swiglu_i8(const float*, int64_t, int64_t, int8_t*, float*, int32_t*, hipStream_t) {
  return absent();
}
hipError_t launch_wquant_channel(const float*, int64_t, int64_t, int32_t*, float*, hipStream_t) { return absent(); }
hipError_t launch_wquant(const float*, int64_t, int64_t, int, int32_t*, float*, hipStream_t) { return absent(); }
hipError_t launch_wquant_mxfp4(const float*, int64_t, int64_t, uint8_t*, uint8_t*, hipStream_t) { return absent(); }
hipError_t launch_prepack(const void*, const void*, int64_t, int64_t, int64_t, int, void*, void*, hipStream_t) {
  return absent();
}
hipError_t launch_requant(const float*, const float*, int64_t, int64_t, uint8_t*, float*, hipStream_t) {
  return absent();
}
hipError_t launch_requant_i8(const float*, const float*, int64_t, int64_t, int8_t*, float*, int32_t*, hipStream_t) {
  return absent();
}
hipError_t launch_front(const FrontArgs&, bool, hipStream_t) { return absent(); }
hipError_t launch_unpermute(const float*, const int32_t*, const float*, int64_t, int, int64_t, void*, int,
                            hipStream_t) {
  return absent();
}

}  // namespace w4a8
