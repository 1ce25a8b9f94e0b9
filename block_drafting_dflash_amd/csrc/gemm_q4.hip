// Instantiations of the weight-streaming GEMM for q4 weights (one translation unit per
// weight type so the kernels compile in parallel).
#include "gemm_impl.h"

namespace dflash {

hipError_t launch_gemm_q4(const GemmPlan& pl, int epi, int xsrc, const GemmParams& p, hipStream_t s) {
  return by_kind<WT_Q4>(pl, epi, xsrc, p, s);
}

}  // namespace dflash
