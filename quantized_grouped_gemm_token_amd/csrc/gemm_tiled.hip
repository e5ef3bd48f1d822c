// Grouped W4A8 GEMM, tiled form: for many rows per expert (prefill).
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace w4a8 {

hipError_t launch_gg_tiled(const GemmArgs& g, hipStream_t stream) { return launch_gg_stream(g, stream); }

}  // namespace w4a8
