// Skinny weight-streaming GEMM for the DFlash block forward: Y[r, n] = sum_k X[r, k] W[n, k]
// with at most 48 activation rows against weight matrices of up to 202048 rows.
//
// The block forward multiplies B+1 (or B) rows by every drafter weight once, so each
// weight byte is read exactly once per pass and the kernel is bound by HBM bandwidth. The
// contraction uses MFMA tiles (A = 16 activation rows, B = 16 weight rows, 32 k per
// bf16 instruction, 4 k per f32 instruction); the weights go straight from global memory
// into the B operand with one 16-byte load per lane per step, and every wave prefetches
// the next chunk of weights while it multiplies the current one.
//
// Work decomposition: a work-group owns 16 output columns (32 for the SwiGLU pair) and
// all of K; its waves split K evenly and sum their partial tiles through LDS in a fixed
// order, so every output's reduction order is the same whatever R is (a row gives
// bit-identical results in a 4-row or a 16-row call). Activations come either straight
// from global memory (L2-resident) or staged once in LDS, optionally through the RMSNorm
// prologue y = x * rsqrt(mean(x^2) + eps) * g rounded to the operand dtype.
// Epilogues: store, residual add, SwiGLU, and the fused argmax of the lm_head, which
// reduces (value, index) keys with wavefront shuffles and one 64-bit atomicMax per row.
#include "common.h"
#include "kernels.h"

namespace dflash {

template <int WT> struct WTr;
template <> struct WTr<WT_F32> {
  static constexpr int KSTEP = 16;  // k covered by one 16-byte lane load across the wave
  static constexpr int EPL = 4;     // elements per lane per step
  static constexpr int ELT = 4;     // bytes per weight/activation element
  static constexpr bool BF = false;
};
template <> struct WTr<WT_BF16> {
  static constexpr int KSTEP = 32;
  static constexpr int EPL = 8;
  static constexpr int ELT = 2;
  static constexpr bool BF = true;
};

template <int WT>
__device__ __forceinline__ f32x4_t step_mfma(u32x4_t x, u32x4_t w, f32x4_t acc) {
  if constexpr (WT == WT_BF16) {
    return mfma_bf16(x, w, acc);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32(__uint_as_float(x[e]), __uint_as_float(w[e]), acc);
    return acc;
  }
}

__device__ __forceinline__ int find_seg(const GemmParams& p, int col) {
  int s = 0;
  for (int i = 1; i < p.nseg; ++i)
    if (col >= p.seg[i].col0) s = i;
  return s;
}

template <int WT, int RT, int NB, int EPI, int XSRC>
__global__ __launch_bounds__(512) void gemm_kernel(const GemmParams p) {
  using T = WTr<WT>;
  constexpr bool BF = T::BF;
  constexpr int CH = chunk_steps(RT);
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int nw = p.waves;
  const int K = p.K, R = p.R, nch = p.nchunks;
  const int kw = K / nw;  // k owned by this wave in every tile

  float* red = (float*)smem;  // [nw][RT][NB][64 lanes][4]
  unsigned char* xs = smem + (size_t)nw * RT * NB * 1024;
  float* rinv = (float*)(xs + (size_t)R * p.xstride * T::ELT);

  const int my_tiles = (p.ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int nit = my_tiles * nch;

  // byte pointers of this lane's weight rows for a tile
  auto wrows = [&](int j, const unsigned char* (&wr)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int s, row;
      if constexpr (NB == 1) {
        s = find_seg(p, 16 * j);
        row = 16 * j - p.seg[s].col0 + li;
      } else {
        s = nb;
        row = 16 * j + li;
      }
      wr[nb] = (const unsigned char*)p.seg[s].w + ((size_t)row * K + (size_t)w * kw + lg * T::EPL) * T::ELT;
    }
  };

  auto load = [&](u32x4_t (&wb)[NB][CH], u32x4_t (&xb)[RT][CH], int it) {
    const int ti = it / nch, c = it - ti * nch;
    const int j = (int)blockIdx.x + ti * (int)gridDim.x;
    const unsigned char* wr[NB];
    wrows(j, wr);
    const size_t kb = (size_t)c * CH * T::KSTEP * T::ELT;
#pragma unroll
    for (int s = 0; s < CH; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        wb[nb][s] = *(const u32x4_t*)(wr[nb] + kb + (size_t)s * T::KSTEP * T::ELT);
    if constexpr (XSRC == XSRC_GLOBAL) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = rt * 16 + li;
        const unsigned char* xr = (const unsigned char*)p.x +
            ((size_t)r * p.ldx + (size_t)w * kw + lg * T::EPL) * T::ELT + kb;
#pragma unroll
        for (int s = 0; s < CH; ++s) {
          u32x4_t v = {0u, 0u, 0u, 0u};
          if (r < R) v = *(const u32x4_t*)(xr + (size_t)s * T::KSTEP * T::ELT);
          xb[rt][s] = v;
        }
      }
    }
  };

  f32x4_t acc[RT][NB];
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rt][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](u32x4_t (&wb)[NB][CH], u32x4_t (&xb)[RT][CH], int it) {
    const int c = it % nch;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        u32x4_t xf;
        if constexpr (XSRC == XSRC_GLOBAL) {
          xf = xb[rt][s];
        } else {
          const int r = rt * 16 + li;
          xf = u32x4_t{0u, 0u, 0u, 0u};
          if (r < R) {
            const int k = w * kw + (c * CH + s) * T::KSTEP + lg * T::EPL;
            xf = *(const u32x4_t*)(xs + ((size_t)r * p.xstride + k) * T::ELT);
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rt][nb] = step_mfma<WT>(xf, wb[nb][s], acc[rt][nb]);
      }
    }
  };

  auto finalize = [&](int it) {
    const int ti = it / nch;
    const int j = (int)blockIdx.x + ti * (int)gridDim.x;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        *(f32x4_t*)&red[((size_t)((w * RT + rt) * NB + nb) * 64 + lane) * 4] = acc[rt][nb];
        acc[rt][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    __syncthreads();
    // wave w finishes row tiles w, w+nw, ... (the argmax launch guarantees nw >= RT)
    for (int rt = w; rt < RT; rt += nw) {
      f32x4_t v[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        v[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int ww = 0; ww < nw; ++ww) v[nb] += *(const f32x4_t*)&red[((size_t)((ww * RT + rt) * NB + nb) * 64 + lane) * 4];
      }
      const int col = 16 * j + li;
      if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rt * 16 + 4 * lg + q;
          unsigned long long key = (r < R) ? argmax_key(v[0][q], col) : 0ull;
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            unsigned long long other = shfl_xor_u64(key, o);
            key = other > key ? other : key;
          }
          best[q] = key > best[q] ? key : best[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rt * 16 + 4 * lg + q;
          if (r >= R) continue;
          const size_t o = (size_t)r * p.ldy + col;
          if constexpr (EPI == EPI_STORE) {
            ((float*)p.y)[o] = v[0][q];
          } else if constexpr (EPI == EPI_RESID) {
            ((float*)p.y)[o] += v[0][q];
          } else if constexpr (EPI == EPI_SWIGLU) {
            const float g = v[0][q], u = v[NB - 1][q];
            act_st<BF>(p.y, o, g / (1.0f + expf(-g)) * u);
          }
        }
      }
    }
    __syncthreads();
  };

  // ---- issue the first weight chunk before staging activations -------------------------
  u32x4_t wA[NB][CH], wB[NB][CH];
  u32x4_t xA[RT][CH], xB[RT][CH];
  if (nit > 0) load(wA, xA, 0);

  if constexpr (XSRC != XSRC_GLOBAL) {
    if constexpr (XSRC == XSRC_NORM) {
      const float* xf = (const float*)p.x;
      for (int r = w; r < R; r += nw) {
        float ss = 0.f;
        for (int k = lane * 4; k < K; k += 256) {
          const float4 v = *(const float4*)(xf + (size_t)r * p.ldx + k);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss = wave_sum(ss);
        if (lane == 0) rinv[r] = rsqrtf(ss / (float)K + p.eps);
      }
      __syncthreads();
    }
    for (int i = tid * 4; i < R * K; i += blockDim.x * 4) {
      const int r = i / K, k = i - r * K;
      float v[4];
      if constexpr (XSRC == XSRC_NORM) {
        const float4 t = *(const float4*)((const float*)p.x + (size_t)r * p.ldx + k);
        const float s = rinv[r];
        v[0] = t.x * s * act_ld<BF>(p.gain, k + 0);
        v[1] = t.y * s * act_ld<BF>(p.gain, k + 1);
        v[2] = t.z * s * act_ld<BF>(p.gain, k + 2);
        v[3] = t.w * s * act_ld<BF>(p.gain, k + 3);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = act_ld<BF>(p.x, (int64_t)r * p.ldx + k + e);
      }
      unsigned char* dst = xs + ((size_t)r * p.xstride + k) * T::ELT;
      if constexpr (BF) {
        uint2 pk;
        pk.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        pk.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *(uint2*)dst = pk;
      } else {
        *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
  }

  // ---- main loop over (tile, chunk), two chunks per trip (register double buffer) -------
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) load(wB, xB, it + 1);
    compute(wA, xA, it);
    if ((it + 1) % nch == 0) finalize(it);
    if (it + 1 >= nit) break;
    if (it + 2 < nit) load(wA, xA, it + 2);
    compute(wB, xB, it + 1);
    if ((it + 2) % nch == 0) finalize(it + 1);
  }

  if constexpr (EPI == EPI_ARGMAX) {
    if (w < RT && li == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = w * 16 + 4 * lg + q;
        if (r < R && best[q] != 0ull) atomicMax(&p.keys[r], best[q]);
      }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(p.ticket, 1u) == gridDim.x - 1);
    __syncthreads();
    if (s_last) {
      __threadfence();
      for (int r = tid; r < R; r += blockDim.x) p.idx_out[r] = argmax_key_index(atomicExch(&p.keys[r], 0ull));
      if (tid == 0) atomicExch(p.ticket, 0u);
    }
  }
}

size_t gemm_lds_bytes(int wt, int xsrc, int R, int waves, int nb, int xstride) {
  const int rt = (R + 15) / 16;
  const size_t elt = wt == WT_F32 ? 4 : 2;
  size_t b = (size_t)waves * rt * nb * 1024;
  if (xsrc != XSRC_GLOBAL) b += (size_t)R * xstride * elt + (size_t)R * 4;
  return b;
}

template <int WT, int RT, int NB, int EPI, int XSRC>
static hipError_t launch_t(const GemmParams& p, int grid, hipStream_t s) {
  const size_t lds = gemm_lds_bytes(WT, XSRC, p.R, p.waves, NB, p.xstride);
  auto fn = gemm_kernel<WT, RT, NB, EPI, XSRC>;
  static size_t attr_lds = 64 * 1024;  // dynamic LDS this kernel is cleared for
  if (lds > attr_lds) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_lds = lds;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(p.waves * 64), lds, s, p);
  return hipGetLastError();
}

template <int WT, int RT, int EPI, int XSRC>
static hipError_t dispatch_nb(const GemmParams& p, int grid, hipStream_t s) {
  if constexpr (EPI == EPI_SWIGLU) return launch_t<WT, RT, 2, EPI, XSRC>(p, grid, s);
  else return launch_t<WT, RT, 1, EPI, XSRC>(p, grid, s);
}

template <int WT, int EPI, int XSRC>
static hipError_t dispatch_rt(const GemmParams& p, int grid, hipStream_t s) {
  const int rt = (p.R + 15) / 16;
  if (rt == 1) return dispatch_nb<WT, 1, EPI, XSRC>(p, grid, s);
  if (rt == 2) return dispatch_nb<WT, 2, EPI, XSRC>(p, grid, s);
  return dispatch_nb<WT, 3, EPI, XSRC>(p, grid, s);
}

template <int WT, int EPI>
static hipError_t dispatch_x(int xsrc, const GemmParams& p, int grid, hipStream_t s) {
  if (xsrc == XSRC_GLOBAL) return dispatch_rt<WT, EPI, XSRC_GLOBAL>(p, grid, s);
  if (xsrc == XSRC_LDS) return dispatch_rt<WT, EPI, XSRC_LDS>(p, grid, s);
  return dispatch_rt<WT, EPI, XSRC_NORM>(p, grid, s);
}

template <int WT>
static hipError_t dispatch_epi(int epi, int xsrc, const GemmParams& p, int grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return dispatch_x<WT, EPI_STORE>(xsrc, p, grid, s);
    case EPI_RESID: return dispatch_x<WT, EPI_RESID>(xsrc, p, grid, s);
    case EPI_SWIGLU: return dispatch_x<WT, EPI_SWIGLU>(xsrc, p, grid, s);
    default: return dispatch_x<WT, EPI_ARGMAX>(xsrc, p, grid, s);
  }
}

hipError_t launch_gemm(int wt, int epi, int xsrc, const GemmParams& p, int grid, hipStream_t s) {
  if (p.R < 1 || p.R > GEMM_MAX_ROWS || grid < 1) return hipErrorInvalidValue;
  if (wt == WT_F32) return dispatch_epi<WT_F32>(epi, xsrc, p, grid, s);
  if (wt == WT_BF16) return dispatch_epi<WT_BF16>(epi, xsrc, p, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace dflash
