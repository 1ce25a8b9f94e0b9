// The low-rank Markov token-transition head of the DSpark drafter, chained by argmax on the
// device (lablup/mlxcel #1751 "LFM2 / LFM2.5 DSpark drafter on the DFlash loop", opening
// paragraph; Implementation Review Summary, Verified against the issue; Security fixes).
//
// One launch is one step of the chain: with t the previous token (the anchor at step 0),
// score[v] = logits[v] + sum_j w2[v][j] * w1[t][j] over the vocabulary, and the step's
// token is the first index of the maximum score. The step is a matrix-vector product that
// streams w2 ([vocab, rank], row-major, 2 or 4 bytes per element) once: it is bound by the
// read bandwidth of w2, and the MFMA units have nothing to contract (one vector), so it
// runs on the vector ALUs. Every lane owns a fixed 16-byte slice of the rank axis (and so
// the same 16 bytes of u = w1[t] for the whole launch); the LPR lanes of a row read its
// rank * elt bytes as one contiguous run, a wave load reads 64 / LPR whole rows (1 KiB
// contiguous), and each wave keeps MK_LOADS such loads in flight (a pass) and issues the
// next pass after reducing this one: more requests queued per wave measured slower. The per-row sums finish
// with DPP row operations, and each work-group leaves one (score, index) key.
//
// The steps pass the token on through kernel boundaries, with no device-wide fence: every
// work-group of step i reduces the keys step i-1 left (a few KiB, read while its first w2
// loads, which do not depend on the token, are in flight) to the token t_i itself, and
// work-group 0 also stores it as the previous step's output. A last one-work-group launch
// reduces the final step's keys. (A fence per work-group, to let the last one finish the
// reduction in the same launch, writes back and invalidates the L2 each time: it measured
// four times slower than the whole stream.)
#include "common.h"
#include "kernels.h"

namespace dflash {

constexpr int MK_THREADS = 256;
constexpr int MK_WAVES = MK_THREADS / 64;
constexpr int MK_LOADS = 7;  // 16-byte loads in flight per lane (5-7 measured alike, 8 and more slower)

// sum over the LPR consecutive lanes that share a row (every one of them ends with the sum)
template <int LPR>
__device__ __forceinline__ float row_lanes_sum(float v) {
  if constexpr (LPR >= 2) v += dpp_f32<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  if constexpr (LPR >= 4) v += dpp_f32<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  if constexpr (LPR >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror: the two quads of 8 lanes
  if constexpr (LPR >= 16) v += dpp_f32<0x128>(v);  // row_ror 8: the two halves of 16 lanes
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <bool BF>
__device__ __forceinline__ float dot16(u32x4_t w, const float* u) {
  float d = 0.f;
  if constexpr (BF) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d = fmaf(__uint_as_float(w[q] << 16), u[2 * q], d);
      d = fmaf(__uint_as_float(w[q] & 0xffff0000u), u[2 * q + 1], d);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) d = fmaf(__uint_as_float(w[q]), u[q], d);
  }
  return d;
}

template <bool BF, int RANK>
__global__ __launch_bounds__(MK_THREADS) void markov_step_kernel(const void* __restrict__ w1,
                                                                 const u32x4_t* __restrict__ w2, int vocab,
                                                                 const float* __restrict__ logits,
                                                                 const unsigned long long* __restrict__ prev_keys,
                                                                 int prev_groups, int32_t anchor,
                                                                 int32_t* __restrict__ prev_out,
                                                                 unsigned long long* __restrict__ keys) {
  constexpr int EPL = BF ? 8 : 4;        // elements per 16-byte slice
  constexpr int LPR = RANK / EPL;        // lanes per row
  static_assert(LPR >= 2 && LPR <= 64 && 64 % LPR == 0, "rank slices must tile a wave");
  constexpr int RPL = 64 / LPR;          // rows per wave load
  constexpr int GROUP = RPL * MK_LOADS;  // rows per wave pass
  constexpr int SLICES = RANK / EPL;     // 16-byte slices per row
  constexpr int KPT = MK_MAX_GROUPS / MK_THREADS;  // previous keys per thread, at most
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane % LPR, rsub = lane / LPR;
  const int ngroups = (vocab + GROUP - 1) / GROUP;
  __shared__ unsigned long long red[MK_WAVES];
  __shared__ int32_t tok;

  // the previous step's keys first (a few KiB from L2: indices past them re-read the last
  // one, as max is idempotent), all in flight together, so that the token's reduction waits
  // for them alone
  unsigned long long kk[KPT];
  if (prev_keys) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) kk[i] = prev_keys[min(tid + i * MK_THREADS, prev_groups - 1)];
  }
  // then the first pass's loads (rows past the vocabulary re-read the last one, unused)
  int g = blockIdx.x * MK_WAVES + w;
  u32x4_t v[MK_LOADS];
  float lg[MK_LOADS];
  auto issue = [&](int gg) {
    const int r0 = gg * GROUP + rsub;
#pragma unroll
    for (int j = 0; j < MK_LOADS; ++j) {
      const int row = min(r0 + j * RPL, vocab - 1);
      v[j] = w2[(size_t)row * SLICES + sub];
      lg[j] = logits[row];
    }
  };
  issue(min(g, ngroups - 1));  // unconditional: no merge between the keys and their use

  // the previous token: the anchor, or the largest key step i-1 left
  if (prev_keys) {
    unsigned long long b = 0ull;
#pragma unroll
    for (int i = 0; i < KPT; ++i) b = kk[i] > b ? kk[i] : b;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long kk = shfl_xor_u64(b, o);
      b = kk > b ? kk : b;
    }
    if (lane == 0) red[w] = b;
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int i = 1; i < MK_WAVES; ++i) b = red[i] > b ? red[i] : b;
      const int32_t idx = argmax_key_index(b);
      tok = idx >= 0 && idx < vocab ? idx : 0;  // a vocabulary row whatever the keys held
      if (blockIdx.x == 0) prev_out[0] = tok;
    }
    __syncthreads();
  } else if (tid == 0) {
    tok = anchor;
  }
  if (!prev_keys) __syncthreads();
  const int32_t t = tok;

  float u[EPL];
  {
    const u32x4_t uw = ((const u32x4_t*)w1)[(size_t)t * SLICES + sub];
    if constexpr (BF) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u[2 * q] = __uint_as_float(uw[q] << 16);
        u[2 * q + 1] = __uint_as_float(uw[q] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = __uint_as_float(uw[q]);
    }
  }

  unsigned long long best = 0ull;  // below every real key
  for (; g < ngroups; g += gridDim.x * MK_WAVES) {
    const int r0 = g * GROUP + rsub;
#pragma unroll
    for (int j = 0; j < MK_LOADS; ++j) {
      const float d = row_lanes_sum<LPR>(dot16<BF>(v[j], u));
      const int row = r0 + j * RPL;
      // rows past the vocabulary get key 0 by a mask, not a branch (a branch would let the
      // compiler sink the logit load into it and wait there for every load in flight)
      const unsigned long long k = argmax_key(lg[j] + d, row) & (0ull - (unsigned long long)(row < vocab));
      best = k > best ? k : best;
    }
    const int gn = g + gridDim.x * MK_WAVES;
    if (gn < ngroups) issue(gn);
  }

#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long k = shfl_xor_u64(best, o);
    best = k > best ? k : best;
  }
  __syncthreads();  // every wave is past its read of red (the previous-token reduction)
  if (lane == 0) red[w] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = red[0];
#pragma unroll
    for (int i = 1; i < MK_WAVES; ++i) b = red[i] > b ? red[i] : b;
    keys[blockIdx.x] = b;
  }
}

bool markov_rank_supported(int bf, int rank) {
  return rank == 64 || rank == 128 || rank == 256 || (bf && rank == 512);
}

int markov_step_groups(int vocab, int rank, int bf, int cus) {
  const int lpr = rank / (bf ? 8 : 4);
  const int rows_per_pass = (64 / lpr) * MK_LOADS * MK_WAVES;
  const int need = (vocab + rows_per_pass - 1) / rows_per_pass;
  const int cap = MK_WG_PER_CU * (cus > 0 ? cus : 256);
  return need < cap ? need : (cap < MK_MAX_GROUPS ? cap : MK_MAX_GROUPS);
}

hipError_t launch_markov_step(int bf, int rank, const void* w1, const void* w2, int vocab, const float* logits,
                              const unsigned long long* prev_keys, int prev_groups, int32_t anchor, int32_t* prev_out,
                              unsigned long long* keys, int groups, hipStream_t s) {
  if (!markov_rank_supported(bf, rank) || groups < 1 || groups > MK_MAX_GROUPS || vocab < 1 ||
      (prev_keys && (prev_groups < 1 || prev_groups > MK_MAX_GROUPS || !prev_out)))
    return hipErrorInvalidValue;
  const dim3 grid(groups), block(MK_THREADS);
  const u32x4_t* w2v = (const u32x4_t*)w2;
#define MK_LAUNCH(B, R)                                                                                         \
  hipLaunchKernelGGL((markov_step_kernel<B, R>), grid, block, 0, s, w1, w2v, vocab, logits, prev_keys, prev_groups, \
                     anchor, prev_out, keys)
  if (bf) {
    if (rank == 64) MK_LAUNCH(true, 64);
    else if (rank == 128) MK_LAUNCH(true, 128);
    else if (rank == 256) MK_LAUNCH(true, 256);
    else MK_LAUNCH(true, 512);
  } else {
    if (rank == 64) MK_LAUNCH(false, 64);
    else if (rank == 128) MK_LAUNCH(false, 128);
    else MK_LAUNCH(false, 256);
  }
#undef MK_LAUNCH
  return hipGetLastError();
}

}  // namespace dflash
