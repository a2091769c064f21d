// Instantiates the streamed small-n kernels for one element type (i8).
#include "nm_skinny_kernels.h"

namespace nm {

hipError_t launch_skinny2_i8(const nm_plan& pl, const GemmArgs& A, hipStream_t s, bool dense_a) {
  return launch_skinny2_dt<DT_I8>(pl, A, s, dense_a);
}

}  // namespace nm
