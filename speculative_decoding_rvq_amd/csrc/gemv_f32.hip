// fp32-weight instantiations of the skinny GEMV (compiled as its own unit).
#include "gemv_impl.h"

namespace cps {
hipError_t launch_gemv_f32(int mode, int mt, const GemvArgs& a, int gx, int gy, hipStream_t s) {
  return launch_gemv_t<float>(mode, mt, a, gx, gy, s);
}
}  // namespace cps
