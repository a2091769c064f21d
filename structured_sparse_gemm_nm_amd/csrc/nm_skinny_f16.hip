// Instantiates the streamed small-n kernels for one element type (f16).
#include "nm_skinny_kernels.h"

namespace nm {

hipError_t launch_skinny2_f16(const nm_plan& pl, const GemmArgs& A, hipStream_t s, bool dense_a) {
  return launch_skinny2_dt<DT_F16>(pl, A, s, dense_a);
}

}  // namespace nm
