// Launch-plan checks and weight-type dispatch of the weight-streaming GEMM (the kernel
// and its instantiation tables live in gemm_impl.h and gemm_{f32,bf16,q4}.hip).
#include "common.h"
#include "kernels.h"

namespace dflash {

hipError_t launch_gemm_f32(const GemmPlan& pl, int epi, int xsrc, const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmPlan& pl, int epi, int xsrc, const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_q4(const GemmPlan& pl, int epi, int xsrc, const GemmParams& p, hipStream_t s);

size_t gemm_lds_bytes(int wt, int xsrc, int split, int R, int waves, int nb, int K, int tiles_per_wg) {
  return gemm_lds_layout(wt, xsrc, split, R, waves, nb, K, tiles_per_wg).total;
}

bool gemm_plan_supported(const GemmPlan& pl, int epi, int xsrc) {
  if (epi == EPI_ARGMAX)
    return xsrc == XSRC_LDS && pl.ch == 8 && (pl.nch == 1 || pl.nch == 2) &&
           (pl.tiles_per_wg == 1 || pl.tiles_per_wg == 2 || pl.tiles_per_wg == 4 || pl.tiles_per_wg == 8 ||
            pl.tiles_per_wg == 16);
  if (xsrc != XSRC_GLOBAL)
    return pl.ch == 8 && (pl.tiles_per_wg == 1 || pl.tiles_per_wg == 2) && (pl.nch == 1 || pl.nch == 2);
  return pl.ch == 8 && pl.tiles_per_wg == 1 &&
         (pl.nch == 1 || pl.nch == 2 || pl.nch == 3 || pl.nch == 4 || pl.nch == 5 || pl.nch == 10);
}

hipError_t launch_gemm(int wt, int epi, int xsrc, const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  if (p.R < 1 || p.R > GEMM_MAX_ROWS || pl.grid < 1 || p.waves != pl.waves || !gemm_plan_supported(pl, epi, xsrc))
    return hipErrorInvalidValue;
  if (p.nseg < 1 || p.nseg > GEMM_MAXSEG || (epi == EPI_ARGMAX && (p.nseg != 1 || p.seg[0].col0 != 0)))
    return hipErrorInvalidValue;  // the argmax kernel reads one matrix
  if (p.z && (epi != EPI_RESID || p.zper < 0 || p.zper == 1 || p.zrow0 < 0 || !p.zgain || (p.split && !p.zlo)))
    return hipErrorInvalidValue;  // gained rows come from a residual launch: all, or runs of 2 or more
  if (wt == WT_F32) return launch_gemm_f32(pl, epi, xsrc, p, s);
  if (wt == WT_BF16) return launch_gemm_bf16(pl, epi, xsrc, p, s);
  if (wt == WT_Q4) return launch_gemm_q4(pl, epi, xsrc, p, s);
  return hipErrorInvalidValue;
}

}  // namespace dflash
