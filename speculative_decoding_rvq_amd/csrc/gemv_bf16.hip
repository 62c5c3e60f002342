// bf16-weight instantiations of the skinny GEMV (compiled as its own unit).
#include "gemv_impl.h"

namespace cps {
hipError_t launch_gemv_bf16(int mode, int mt, const GemvArgs& a, int gx, int gy, hipStream_t s) {
  return launch_gemv_t<uint16_t>(mode, mt, a, gx, gy, s);
}
}  // namespace cps
