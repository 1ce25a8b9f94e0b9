// Instantiations of the weight-streaming GEMM for f32 weights (one translation unit per
// weight type so the kernels compile in parallel).
#include "gemm_impl.h"

namespace dflash {

hipError_t launch_gemm_f32(const GemmPlan& pl, int epi, int xsrc, const GemmParams& p, hipStream_t s) {
  return by_kind<WT_F32>(pl, epi, xsrc, p, s);
}

}  // namespace dflash
