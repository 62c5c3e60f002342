// fp32-weight instantiations of the GEMV and MFMA kernels (own compile unit).
#include "gemv_impl.h"
#include "mfma_impl.h"

namespace cps {
hipError_t launch_gemv_f32(int mode, int mt, const GemvArgs& a, int gx, int gy, hipStream_t s) {
  return launch_gemv_t<float>(mode, mt, a, gx, gy, s);
}
hipError_t launch_mfma_f32(int mode, int tile, const GemvArgs& a, dim3 grid, hipStream_t s) {
  return launch_mfma_t<float>(mode, tile, a, grid, s);
}
}  // namespace cps
