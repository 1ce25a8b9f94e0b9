// Small kernels of the DFlash round: the argmax finish, block embedding gather, row
// RMSNorm, the greedy verify scan and the weight repack.
#include "common.h"
#include "kernels.h"

namespace dflash {

// One work-group per row: the largest (value, index) key over the lm_head work-groups'
// partial keys; the key order puts the larger logit first and then the lower index. Each
// thread loads its first FIN_PER keys at once (indices clamped: max is idempotent).
constexpr int FIN_THREADS = 1024, FIN_PER = 8;
__global__ __launch_bounds__(FIN_THREADS) void argmax_finalize_kernel(const unsigned long long* __restrict__ part,
                                                                      int groups, int32_t* idx) {
  __shared__ unsigned long long red[FIN_THREADS / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const unsigned long long* row = part + (size_t)r * groups;
  unsigned long long k[FIN_PER];
#pragma unroll
  for (int i = 0; i < FIN_PER; ++i) k[i] = row[min(tid + FIN_THREADS * i, groups - 1)];
  unsigned long long best = 0ull;
#pragma unroll
  for (int i = 0; i < FIN_PER; ++i) best = k[i] > best ? k[i] : best;
  for (int g = tid + FIN_THREADS * FIN_PER; g < groups; g += FIN_THREADS) best = row[g] > best ? row[g] : best;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long kk = shfl_xor_u64(best, o);
    best = kk > best ? kk : best;
  }
  if (lane == 0) red[w] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = red[0];
    for (int i = 1; i < FIN_THREADS / 64; ++i) b = red[i] > b ? red[i] : b;
    idx[r] = argmax_key_index(b);
  }
}

hipError_t launch_argmax_finalize(const unsigned long long* part, int groups, int R, int32_t* idx, hipStream_t s) {
  if (groups < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(R), dim3(FIN_THREADS), 0, s, part, groups, idx);
  return hipGetLastError();
}

// one embedding row (gathered from the table in its storage dtype) as f32: 16-byte loads
// when the table is 16-byte aligned (every row then is: hidden is a multiple of 16)
template <bool BF, bool VEC>
__device__ __forceinline__ void embed_row(const void* table, int hidden, int64_t tok, float* xr) {
  if constexpr (VEC) {
    constexpr int EPV = BF ? 8 : 4;  // elements per 16-byte load
    constexpr int U = 4;             // loads in flight per thread
    const int nv = hidden / EPV;
    const u32x4_t* src = (const u32x4_t*)table + (size_t)tok * nv;
    for (int v0 = threadIdx.x; v0 < nv; v0 += 256 * U) {
      u32x4_t t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) t[u] = src[min(v0 + 256 * u, nv - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + 256 * u;
        if (v >= nv) break;
        if constexpr (BF) {
          float4* d = (float4*)(xr + (size_t)v * 8);
          d[0] = make_float4(__uint_as_float(t[u][0] << 16), __uint_as_float(t[u][0] & 0xffff0000u),
                             __uint_as_float(t[u][1] << 16), __uint_as_float(t[u][1] & 0xffff0000u));
          d[1] = make_float4(__uint_as_float(t[u][2] << 16), __uint_as_float(t[u][2] & 0xffff0000u),
                             __uint_as_float(t[u][3] << 16), __uint_as_float(t[u][3] & 0xffff0000u));
        } else {
          *(u32x4_t*)(xr + (size_t)v * 4) = t[u];
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < hidden; i += blockDim.x) xr[i] = act_ld<BF>(table, tok * hidden + i);
  }
}

// the rotary rotation of position pos: (cos, sin) of pos * theta^(-2i/hd) for i < hd/2,
// evaluated in f64 and rounded to f32 as the per-element RoPE of the prep kernel does
__device__ __forceinline__ void rope_row(int64_t pos, float theta, int hd, float2* dst) {
  for (int i = threadIdx.x; i < hd / 2; i += blockDim.x) {
    const double inv = pow((double)theta, -2.0 * (double)i / (double)hd);
    double sn, cs;
    sincos((double)pos * inv, &sn, &cs);
    dst[i] = make_float2((float)cs, (float)sn);
  }
}

// Block rows [anchor, mask x (R-1)] from the target's raw embedding table (not the
// embed_norm lookup: lablup/mlxcel #1762, What changed), as f32 residual rows: work-group
// (r, 0) gathers row r. The draft's first kernel also tabulates the rotary rotation of
// every block position pos0 + r in work-group (r, 1); every layer's attention reads it
// (rope may be NULL).
template <bool BF, bool VEC>
__global__ __launch_bounds__(256) void embed_kernel(const void* table, int hidden, int vocab, int32_t anchor,
                                                    int32_t mask_id, const int32_t* toks, int R, int nprev,
                                                    const float* prev, float* x, float2* rope, int64_t pos0,
                                                    float theta, int hd) {
  const int r = blockIdx.x;
  if (blockIdx.y == 1) {
    rope_row(r < R ? pos0 + r : pos0 - nprev + (r - R), theta, hd, rope + (size_t)r * (hd / 2));
    return;
  }
  if (r >= R) {  // rows carried behind the embedded ones
    const float4* src = (const float4*)(prev + (size_t)(r - R) * hidden);
    float4* dst = (float4*)(x + (size_t)r * hidden);
    for (int v = threadIdx.x; v < hidden / 4; v += blockDim.x) dst[v] = src[v];
    return;
  }
  // block tokens from device memory (a target's verify rows) are clamped into the table: an
  // id past the last row would read whatever follows the table (lablup/mlxcel #1751, Review
  // fixes); the verify kernel reports out-of-range ids in its status word
  const int64_t tok = r == 0 ? anchor : (toks ? (int64_t)min(max(toks[r - 1], 0), vocab - 1) : mask_id);
  embed_row<BF, VEC>(table, hidden, tok, x + (size_t)r * hidden);
}

// Rows [anchor_q, mask x (R1 - 1)] of every sequence q of a batch, sequence after sequence,
// at positions pos0_q + j, with their rotary table (work-group (r, 1)).
template <bool BF, bool VEC>
__global__ __launch_bounds__(256) void embed_batch_kernel(const void* table, int hidden, EmbedSeqs seqs, int R1,
                                                          int32_t mask_id, float* x, float2* rope, float theta,
                                                          int hd) {
  const int r = blockIdx.x, q = r / R1, j = r - q * R1;
  if (blockIdx.y == 1) {
    rope_row(seqs.pos0[q] + j, theta, hd, rope + (size_t)r * (hd / 2));
    return;
  }
  embed_row<BF, VEC>(table, hidden, j == 0 ? seqs.anchor[q] : mask_id, x + (size_t)r * hidden);
}

hipError_t launch_embed(int bf, const void* table, int hidden, int vocab, int32_t anchor, int32_t mask_id,
                        const int32_t* toks, int R, int nprev, const float* prev, float* x, float2* rope, int64_t pos0,
                        float theta, int hd, hipStream_t s) {
  if (nprev < 0 || (nprev > 0 && (!rope || !prev || hidden % 4 || ((uintptr_t)prev & 15u) || ((uintptr_t)x & 15u))))
    return hipErrorInvalidValue;
  const bool vec = ((uintptr_t)table & 15u) == 0 && hidden % 8 == 0;
  const dim3 grid(R + nprev, rope ? 2 : 1);
  if (bf && vec)
    hipLaunchKernelGGL((embed_kernel<true, true>), grid, dim3(256), 0, s, table, hidden, vocab, anchor, mask_id, toks, R,
                       nprev, prev, x, rope, pos0, theta, hd);
  else if (bf)
    hipLaunchKernelGGL((embed_kernel<true, false>), grid, dim3(256), 0, s, table, hidden, vocab, anchor, mask_id, toks, R,
                       nprev, prev, x, rope, pos0, theta, hd);
  else if (vec)
    hipLaunchKernelGGL((embed_kernel<false, true>), grid, dim3(256), 0, s, table, hidden, vocab, anchor, mask_id, toks, R,
                       nprev, prev, x, rope, pos0, theta, hd);
  else
    hipLaunchKernelGGL((embed_kernel<false, false>), grid, dim3(256), 0, s, table, hidden, vocab, anchor, mask_id, toks, R,
                       nprev, prev, x, rope, pos0, theta, hd);
  return hipGetLastError();
}

hipError_t launch_embed_batch(int bf, const void* table, int hidden, const EmbedSeqs& seqs, int R1, int32_t mask_id,
                              float* x, float2* rope, float theta, int hd, hipStream_t s) {
  if (seqs.n < 1 || seqs.n > ATTN_MAX_SEQS || R1 < 1 || !rope) return hipErrorInvalidValue;
  const bool vec = ((uintptr_t)table & 15u) == 0 && hidden % 8 == 0;
  const dim3 grid(seqs.n * R1, 2);
  if (bf && vec)
    hipLaunchKernelGGL((embed_batch_kernel<true, true>), grid, dim3(256), 0, s, table, hidden, seqs, R1, mask_id, x, rope,
                       theta, hd);
  else if (bf)
    hipLaunchKernelGGL((embed_batch_kernel<true, false>), grid, dim3(256), 0, s, table, hidden, seqs, R1, mask_id, x,
                       rope, theta, hd);
  else if (vec)
    hipLaunchKernelGGL((embed_batch_kernel<false, true>), grid, dim3(256), 0, s, table, hidden, seqs, R1, mask_id, x,
                       rope, theta, hd);
  else
    hipLaunchKernelGGL((embed_batch_kernel<false, false>), grid, dim3(256), 0, s, table, hidden, seqs, R1, mask_id, x,
                       rope, theta, hd);
  return hipGetLastError();
}

// out[r] = RMSNorm(in[r]) * g as a GEMM operand (hi/lo bf16 planes for bf16 shapes, f32
// otherwise); one 256-thread group per row. Each thread holds its first RN_V groups of four
// values in registers (rows up to 4096 wide: one read), accumulates their squares, and the
// wave sums are added in wave order.
constexpr int RN_V = 4;
template <bool BF>
__global__ __launch_bounds__(256) void rownorm_kernel(const float* __restrict__ in, const void* gain, float eps, int H,
                                                      void* out, void* out_lo) {
  __shared__ float part[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nv = H / 4;  // H is a multiple of 16
  const float4* x = (const float4*)(in + (size_t)r * H);
  float4 xv[RN_V];
  float gv[RN_V][4];
  auto load_gain = [&](int v, float (&g)[4]) {
    if constexpr (BF) {
      const uint2 gw = *((const uint2*)gain + v);
      g[0] = __uint_as_float(gw.x << 16); g[1] = __uint_as_float(gw.x & 0xffff0000u);
      g[2] = __uint_as_float(gw.y << 16); g[3] = __uint_as_float(gw.y & 0xffff0000u);
    } else {
      const float4 gf = *((const float4*)gain + v);
      g[0] = gf.x; g[1] = gf.y; g[2] = gf.z; g[3] = gf.w;
    }
  };
#pragma unroll
  for (int j = 0; j < RN_V; ++j) {
    const int v = min(tid + 256 * j, nv - 1);
    xv[j] = x[v];
    load_gain(v, gv[j]);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < RN_V; ++j)
    if (tid + 256 * j < nv)
      ss = fmaf(xv[j].w, xv[j].w, fmaf(xv[j].z, xv[j].z, fmaf(xv[j].y, xv[j].y, fmaf(xv[j].x, xv[j].x, ss))));
  for (int v = tid + 256 * RN_V; v < nv; v += 256) {
    const float4 a = x[v];
    ss = fmaf(a.w, a.w, fmaf(a.z, a.z, fmaf(a.y, a.y, fmaf(a.x, a.x, ss))));
  }
  ss = wave_sum(ss);
  if (lane == 0) part[w] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float s = rsqrtf(tot / (float)H + eps);
  auto put = [&](int v, const float4 a, const float (&g)[4]) {
    const float y[4] = {a.x * s * g[0], a.y * s * g[1], a.z * s * g[2], a.w * s * g[3]};
    const size_t o = (size_t)r * H + 4 * (size_t)v;
    if constexpr (BF) {
      uint32_t h0, l0, h1, l1;
      split2_bf16(y[0], y[1], h0, l0);
      split2_bf16(y[2], y[3], h1, l1);
      *(uint2*)((uint16_t*)out + o) = make_uint2(h0, h1);
      *(uint2*)((uint16_t*)out_lo + o) = make_uint2(l0, l1);
    } else {
      *(float4*)((float*)out + o) = make_float4(y[0], y[1], y[2], y[3]);
    }
  };
#pragma unroll
  for (int j = 0; j < RN_V; ++j)
    if (tid + 256 * j < nv) put(tid + 256 * j, xv[j], gv[j]);
  for (int v = tid + 256 * RN_V; v < nv; v += 256) {
    float g[4];
    load_gain(v, g);
    put(v, x[v], g);
  }
}

hipError_t launch_rownorm(int bf, const float* in, const void* gain, float eps, int R, int H, void* out,
                          void* out_lo, hipStream_t s) {
  if (H % 16) return hipErrorInvalidValue;
  if (bf) hipLaunchKernelGGL(rownorm_kernel<true>, dim3(R), dim3(256), 0, s, in, gain, eps, H, out, out_lo);
  else hipLaunchKernelGGL(rownorm_kernel<false>, dim3(R), dim3(256), 0, s, in, gain, eps, H, out, out_lo);
  return hipGetLastError();
}

// Greedy exact-match verify on one wave: the first row i with draft[i] != target[i]
// (found by ballot over 64 rows at a time) is the accepted length k; bonus = target[k]
// (lablup/mlxcel #1751, Implementation Review Summary: greedy exact-match verify rule).
__global__ void verify_kernel(const int32_t* __restrict__ draft, const int32_t* __restrict__ target, int B,
                              int vocab, int32_t* out) {
  // one wave per sequence of a batch: its draft [B], target [B+1] and result [3]
  draft += (size_t)blockIdx.x * B;
  target += (size_t)blockIdx.x * (B + 1);
  out += (size_t)blockIdx.x * 3;
  const int lane = threadIdx.x;
  bool bad = false;
  for (int i = lane; i <= B; i += 64) {
    const int32_t a = target[i];
    bad |= (a < 0 || a >= vocab);
  }
  const bool any_bad = __any(bad);
  int k = B;
  for (int base = 0; base < B; base += 64) {
    const int i = base + lane;
    const bool mismatch = (i < B) && (draft[i] != target[i]);
    const unsigned long long m = __ballot(mismatch);
    if (m) {
      k = base + __ffsll((long long)m) - 1;
      break;
    }
  }
  if (lane == 0) {
    if (any_bad) {
      out[0] = 0;
      out[1] = -1;
      out[2] = 1;
    } else {
      out[0] = k;
      out[1] = target[k];
      out[2] = 0;
    }
  }
}

hipError_t launch_verify(const int32_t* draft, const int32_t* target, int B, int vocab, int32_t* out, hipStream_t s,
                         int n_seq) {
  if (n_seq < 1 || B < 1) return hipErrorInvalidValue;  // a block drafts at least one row
  hipLaunchKernelGGL(verify_kernel, dim3(n_seq), dim3(64), 0, s, draft, target, B, vocab, out);
  return hipGetLastError();
}

}  // namespace dflash

namespace dflash {

// Repack a row-major linear W [N, K] into fragment-major 1 KiB blocks: block (j, s) holds
// rows 16j..16j+15 and k in [s*KSTEP, (s+1)*KSTEP), and its lane l = li + 16*lg (li = row
// offset, lg = 0..3) owns the 16 bytes W[16j + li][s*KSTEP + lg*EPL .. + EPL). Blocks of a
// row tile are consecutive, so every 16-byte-per-lane wave load of the GEMM reads one
// contiguous kilobyte and lands directly in the MFMA B-operand layout.
// Row r of the packed matrix takes source row src_row(r): itself, or with perm_hd > 0 the
// deinterleaved order inside each run of perm_hd rows.
__device__ __forceinline__ int64_t src_row(int64_t r, int perm_hd) {
  if (perm_hd <= 0) return r;
  const int64_t h = r / perm_hd;
  return h * perm_hd + deinterleaved_row((int)(r - h * perm_hd), perm_hd);
}

__global__ void pack_kernel(const unsigned char* __restrict__ src, int64_t nblocks, int kblocks, int K, int elt,
                            int epl, int perm_hd, u32x4_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte lane slot
  if (i >= nblocks * 64) return;
  const int64_t blk = i >> 6;
  const int lane = (int)(i & 63), li = lane & 15, lg = lane >> 4;
  const int64_t j = blk / kblocks, s = blk - j * kblocks;
  const int kstep = 4 * epl;
  const size_t off = ((size_t)src_row(16 * j + li, perm_hd) * K + (size_t)s * kstep + (size_t)lg * epl) * elt;
  dst[i] = *(const u32x4_t*)(src + off);
}

hipError_t launch_pack(int wt, const void* src, int N, int K, void* dst, hipStream_t s, int perm_hd) {
  if (perm_hd < 0 || (perm_hd > 0 && (perm_hd % 2 || N % perm_hd))) return hipErrorInvalidValue;
  const int elt = wt == WT_F32 ? 4 : 2, epl = 16 / elt;
  const int kblocks = K / (4 * epl);
  const int64_t nblocks = (int64_t)(N / 16) * kblocks;
  const int64_t slots = nblocks * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, s, (const unsigned char*)src,
                     nblocks, kblocks, K, elt, epl, perm_hd, (u32x4_t*)dst);
  return hipGetLastError();
}

__global__ void deinterleave_kernel(const unsigned char* __restrict__ src, unsigned char* __restrict__ dst, int hd,
                                    int elt) {
  const int j = threadIdx.x;
  if (j >= hd) return;
  const int from = deinterleaved_row(j, hd);
  if (elt == 4) ((float*)dst)[j] = ((const float*)src)[from];
  else ((uint16_t*)dst)[j] = ((const uint16_t*)src)[from];
}

hipError_t launch_deinterleave(const void* src, void* dst, int hd, int elt, hipStream_t s) {
  if (hd < 2 || hd > 1024 || hd % 2 || (elt != 2 && elt != 4)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(deinterleave_kernel, dim3(1), dim3(hd), 0, s, (const unsigned char*)src, (unsigned char*)dst, hd,
                     elt);
  return hipGetLastError();
}


// 4-bit affine weights (w = s * q + b, group 64 along k) into fragment-major form.
// Codes: block (j, s4) holds rows 16j..16j+15 and k in [128*s4, 128*s4 + 128); lane
// l = li + 16*lg owns four words, word t carrying the eight codes of row 16j + li at
// k = 128*s4 + 32*t + 8*lg .. + 8. Inside a word the nibbles are reordered so that k0, k2,
// k4, k6 sit in bits 0-15 and k1, k3, k5, k7 in bits 16-31: (word >> 4e) & 0x000F000F then
// holds the codes of k = 2e and 2e + 1 in the two 16-bit halves, which become the bf16
// values 128 + q with one OR (the GEMM subtracts the 128 per group). Scales: a 128-byte
// block per (j, s4) with 8 bytes per row li: (s, b) of groups 2*s4 and 2*s4 + 1, bf16.
__device__ __forceinline__ uint32_t q4_reorder(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r |= ((w >> (8 * e)) & 0xFu) << (4 * e);             // k = 2e
    r |= ((w >> (8 * e + 4)) & 0xFu) << (16 + 4 * e);    // k = 2e + 1
  }
  return r;
}

__global__ void pack_q4_kernel(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                               const uint16_t* __restrict__ biases, int64_t nblocks, int kblocks, int K, int perm_hd,
                               u32x4_t* __restrict__ dst_codes, uint32_t* __restrict__ dst_scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte lane slot
  if (i >= nblocks * 64) return;
  const int64_t blk = i >> 6;
  const int lane = (int)(i & 63), li = lane & 15, lg = lane >> 4;
  const int64_t j = blk / kblocks, s4 = blk - j * kblocks;
  const int64_t row = src_row(16 * j + li, perm_hd);
  const uint32_t* src = codes + row * (K / 8) + (128 * s4 + 8 * lg) / 8;
  u32x4_t v;
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = q4_reorder(src[4 * t]);  // k advances 32 per word = 4 words
  dst_codes[i] = v;
  if (lg == 0) {
    const int groups = K / 64;
    const int64_t g0 = row * groups + 2 * s4;
    uint32_t* d = dst_scales + blk * 32 + li * 2;
    d[0] = (uint32_t)scales[g0] | ((uint32_t)biases[g0] << 16);
    d[1] = (uint32_t)scales[g0 + 1] | ((uint32_t)biases[g0 + 1] << 16);
  }
}

hipError_t launch_pack_q4(const void* codes, const void* scales, const void* biases, int N, int K, void* dst_codes,
                          void* dst_scales, hipStream_t s, int perm_hd) {
  if (perm_hd < 0 || (perm_hd > 0 && (perm_hd % 2 || N % perm_hd))) return hipErrorInvalidValue;
  const int kblocks = K / 128;
  const int64_t nblocks = (int64_t)(N / 16) * kblocks;
  const int64_t slots = nblocks * 64;
  hipLaunchKernelGGL(pack_q4_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, s, (const uint32_t*)codes,
                     (const uint16_t*)scales, (const uint16_t*)biases, nblocks, kblocks, K, perm_hd,
                     (u32x4_t*)dst_codes, (uint32_t*)dst_scales);
  return hipGetLastError();
}

}  // namespace dflash

namespace dflash {

// Streaming read of `bytes` from src: work-group g reads its contiguous share with 16-byte
// non-temporal loads, eight in flight per thread, and stores the XOR of everything it read
// to sink[g] (so the loads cannot be dropped). The practical HBM read ceiling the weight
// streams of the round are compared with.
constexpr int PROBE_THREADS = 256, PROBE_UNROLL = 8;
__global__ __launch_bounds__(PROBE_THREADS) void hbm_read_probe_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                                      uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per, hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  for (size_t i = lo + threadIdx.x; i < hi; i += (size_t)PROBE_THREADS * PROBE_UNROLL) {
    u32x4_t v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) {
      const size_t j = i + (size_t)u * PROBE_THREADS;
      v[u] = __builtin_nontemporal_load(src + (j < hi ? j : hi - 1));
    }
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t part[PROBE_THREADS / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int groups, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 < (size_t)groups * PROBE_THREADS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(groups), dim3(PROBE_THREADS), 0, s, (const u32x4_t*)src, n16, sink);
  return hipGetLastError();
}

}  // namespace dflash

