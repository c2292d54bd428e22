// gemm_rs_mixed.hip -- the direct-form GEMM-RS kernels that can run a
// workgroup holding owner rows beside published rows of other segments (those
// rows are stored and published before the workgroup's readiness wait; see
// gemm_rs_impl.h).  A translation unit of its own, so that these instantiations
// build in parallel with the others.
#include "gemm_rs_kernel.h"

namespace arepi {

bool launch_gemm_rs_mixed(int cfg, const void *params, hipStream_t s) {
    return launch_tile<true>(cfg, *static_cast<const GemmRsParams *>(params), s);
}

}  // namespace arepi
