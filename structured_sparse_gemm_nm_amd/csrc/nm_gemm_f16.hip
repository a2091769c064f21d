// Instantiates the tiled matrix-core kernels for one element type (f16).
#include "nm_gemm_kernels.h"
#include "nm_vw_kernels.h"

namespace nm {

hipError_t launch_tiles_f16(const nm_plan& pl, int amode, const GemmArgs& A, hipStream_t s) {
  return launch_tiles_dt<DT_F16>(pl, amode, A, s);
}

hipError_t launch_vw_f16(const nm_plan& pl, const GemmArgs& A, hipStream_t s) { return launch_vw_dt<DT_F16>(pl, A, s); }

}  // namespace nm
