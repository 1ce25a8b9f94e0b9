// Attention side of the DFlash block forward: per-head q/k RMSNorm + RoPE, the ring
// context cache writes, and bidirectional sliding-window attention over the ring.
//
// The drafter attends with a bidirectional mask over absolute positions, |q - k| <= W,
// and its context cache is a temporal window whose wrapped ring hands out slots in
// physical order, so the mask must use absolute key positions (lablup/mlxcel #1762 "Muse
// Glimmer DFlash assistant drafter on the round loop", What changed). The block's own keys
// follow the context keys (lablup/mlxcel #1751 "LFM2 / LFM2.5 DSpark drafter on the DFlash
// loop", Verified against the issue: proposal K/V concatenated after the context K/V).
//
// Ring: the slot of absolute position p is (p + phase) mod Cs, with the storage capacity
// Cs and the phase multiples of 8 (AttnShape cap / phase). Per layer, K is stored as
// [kv head][slot][head dim] and V transposed, [kv head][head dim][slot], so that both MFMA
// operands of the attention read consecutive elements: a key row for the scores, a run of
// eight consecutive keys at one dim for the output. The keys of a query are positions
// max(0, e-W)..e+R-1: the committed context from the ring, then the block's own. The bf16
// MFMA kernel forms the block's own keys and values itself from the raw projections and
// uses them in place of the ring slots of positions e..e+R-1, which lie past the committed
// window; the other paths (f32 shapes, long blocks) write them into those slots first (the
// append of the verified rows overwrites them either way). The MFMA kernel also takes the
// last n committed rows, e-n..e-1, from the raw projections when an append left their K/V
// to this draft: it forms them the same way, uses them, and writes them into their slots. The ring is zeroed when the
// context is created, so every slot holds finite values and keys outside a query's window
// can be read and given weight exactly 0.
//
// The same kernels serve a target's verify forward (AttnShape causal): each query sees the
// keys q - W < p <= q (every earlier position on full-attention layers), and the block's own
// keys and values become cache rows: the MFMA kernel writes the ones it forms into their
// slots, the other paths write them first, as for the drafter (lablup/mlxcel #1762, What
// changed, "Muse target": trim rollback over mixed sliding and full caches).
//
// Work split: keys are cut into chunks of 64 absolute positions (aligned to multiples of
// 64, so the cut never depends on the phase and every 8-key run is one aligned 16-byte
// load). One work-group per (chunk, kv head) computes, for the kv group's query vectors,
// the chunk's max logit m, sum of exp l and unnormalised output; a combine kernel merges
// the chunks in chunk order (fixed, so results do not depend on scheduling) and writes the
// attention output as the O-projection operand.
#include "common.h"
#include "kernels.h"

namespace dflash {

// floats per (chunk, query) partial: the unnormalised output [hd], then m and l, padded to a
// multiple of four so that output rows stay 16-byte aligned
#define PART_STRIDE(hd) ((hd) + 4)

__device__ __forceinline__ int64_t ring_slot(const AttnShape& a, int64_t pos) { return (pos + a.phase) % a.cap; }

// ---- q/k RMSNorm + RoPE on the block rows -----------------------------------------------
// One wave per (row, head). Lane i < hd/2 owns the rotate-half pair (i, i + hd/2). q leaves
// as an attention operand (hi/lo bf16 planes, or f32); k and v go to the ring slots of
// positions pos0 + r in the cache dtype.
template <bool BF>
__global__ __launch_bounds__(256) void attn_prep_kernel(AttnShape a, const float* __restrict__ qkv,
                                                        const void* qnorm, const void* knorm, int R,
                                                        int64_t pos0, void* qb, void* qlo, void* ring_layer) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int heads = a.nq + 2 * a.nkv;
  if (item >= R * heads) return;
  const int r = item / heads, h = item - r * heads;
  const int hd = a.hd, half = hd >> 1;
  const float* src = qkv + (size_t)r * heads * hd + (size_t)h * hd;
  const bool act = lane < half;
  float x1 = act ? src[lane] : 0.f, x2 = act ? src[lane + half] : 0.f;
  const size_t slot = (size_t)ring_slot(a, pos0 + r);
  const size_t plane = (size_t)a.cap * hd;
  if (h >= a.nq + a.nkv) {  // v head: cast into V^T [head][dim][slot]
    const size_t vbase = (size_t)(a.nkv + (h - a.nq - a.nkv)) * plane;
    if (act) {
      act_st<BF>(ring_layer, vbase + (size_t)lane * a.cap + slot, x1);
      act_st<BF>(ring_layer, vbase + (size_t)(lane + half) * a.cap + slot, x2);
    }
    return;
  }
  const bool is_q = h < a.nq;
  const void* g = is_q ? qnorm : knorm;
  const float ss = wave_sum(x1 * x1 + x2 * x2);
  const float s = rsqrtf(ss / (float)hd + a.eps);
  if (!act) return;
  x1 = x1 * s * act_ld<BF>(g, lane);
  x2 = x2 * s * act_ld<BF>(g, lane + half);
  const double inv = pow((double)a.theta, -2.0 * (double)lane / (double)hd);
  double sn, cs;
  sincos((double)(pos0 + r) * inv, &sn, &cs);
  const float c = (float)cs, sf = (float)sn;
  const float y1 = x1 * c - x2 * sf, y2 = x2 * c + x1 * sf;
  if (is_q) {
    const size_t o = ((size_t)r * a.nq + h) * hd;
    op_st<BF>(qb, qlo, o + lane, y1);
    op_st<BF>(qb, qlo, o + lane + half, y2);
  } else {
    const size_t kbase = (size_t)(h - a.nq) * plane + slot * hd;
    act_st<BF>(ring_layer, kbase + lane, y1);
    act_st<BF>(ring_layer, kbase + lane + half, y2);
  }
}

// ---- one key row, 16 lanes per row ------------------------------------------------------
// Lane t16 of a 16-lane row holds dims EPT t16 .. + EPT (k1) and their rotate-half
// partners (k2), the gains of those dims and their (cos, sin) pairs. RMSNorm over the head
// (each lane's squares in dim order, then the 16 lanes' sums in a fixed order), gain, RoPE,
// then bf16 pairs. The attention's own block rows and the ring write of appended rows both
// form keys here, so a key has the same bits whichever of them wrote it.
template <int HD>
__device__ __forceinline__ void form_key16(const float (&k1)[HD / 32], const float (&k2)[HD / 32],
                                           const float (&g1)[HD / 32], const float (&g2)[HD / 32],
                                           const float (&cs)[HD / 16], float eps, uint32_t (&o1)[HD / 64],
                                           uint32_t (&o2)[HD / 64]) {
  constexpr int EPT = HD / 32;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPT; ++j) ss = fmaf(k1[j], k1[j], fmaf(k2[j], k2[j], ss));
  ss = row16_sum(ss);
  const float sc = rsqrtf(ss / (float)HD + eps);
#pragma unroll
  for (int j = 0; j < EPT; j += 2) {
    float y1[2], y2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float x1 = k1[j + u] * sc * g1[j + u], x2 = k2[j + u] * sc * g2[j + u];
      const float cc = cs[2 * (j + u)], sn = cs[2 * (j + u) + 1];
      y1[u] = fmaf(x1, cc, -(x2 * sn));
      y2[u] = fmaf(x2, cc, x1 * sn);
    }
    o1[j / 2] = f2bf2(y1[0], y1[1]);
    o2[j / 2] = f2bf2(y2[0], y2[1]);
  }
}

// ---- context K/V into the ring, bf16 shapes with head dim 64 or 128 -----------------------
// kv: f32 [n, L, 2, nkv, hd] (k then v per layer). Work-group (row r, y): 16 lanes per
// (layer, kv head) item 16 y .. 16 y + 15 of the row, in the lane layout of form_key16. The
// items' loads are issued first; the row's rotary pairs are computed meanwhile into LDS (as
// the embedding kernel's table computes them).
// One row r of kv at position pos (this work-group's 16 (layer, kv head) items) into `ring`;
// rot: the work-group's LDS for the row's rotation table.
template <int HD>
__device__ __forceinline__ void ring_write16_row(const AttnShape& a, const float* __restrict__ kv,
                                                 const void* const* knorms, int r, int64_t pos, uint16_t* ring,
                                                 float2* rot) {
  constexpr int HALF = HD / 2, EPT = HD / 32;
  const int t16 = threadIdx.x & 15;
  const int per_row = a.L * a.nkv;
  const int item = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int it = item < per_row ? item : per_row - 1;  // a whole 16-lane row shares its item
  const int l = it / a.nkv, h = it - l * a.nkv;
  const float* kr = kv + (((size_t)(r * a.L + l) * 2) * a.nkv + h) * HD + EPT * t16;
  const float* vr = kr + (size_t)a.nkv * HD;
  const uint16_t* g = (const uint16_t*)knorms[l] + EPT * t16;
  float k1[EPT], k2[EPT], v1[EPT], v2[EPT], g1[EPT], g2[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    k1[j] = kr[j];
    k2[j] = kr[HALF + j];
    v1[j] = vr[j];
    v2[j] = vr[HALF + j];
    g1[j] = bf2f(g[j]);
    g2[j] = bf2f(g[HALF + j]);
  }
  for (int i = threadIdx.x; i < HALF; i += blockDim.x) {
    const double inv = pow((double)a.theta, -2.0 * (double)i / (double)HD);
    double sn, c;
    sincos((double)pos * inv, &sn, &c);
    rot[i] = make_float2((float)c, (float)sn);
  }
  __syncthreads();
  float cs[2 * EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const float2 v = rot[EPT * t16 + j];
    cs[2 * j] = v.x;
    cs[2 * j + 1] = v.y;
  }
  uint32_t o1[EPT / 2], o2[EPT / 2];
  form_key16<HD>(k1, k2, g1, g2, cs, a.eps, o1, o2);
  if (item >= per_row) return;
  const size_t slot = (size_t)ring_slot(a, pos);
  uint16_t* K = ring + (((size_t)l * 2) * a.nkv + h) * (size_t)a.cap * HD + slot * HD + EPT * t16;
  uint16_t* VT = ring + (((size_t)l * 2 + 1) * a.nkv + h) * (size_t)a.cap * HD + slot;
#pragma unroll
  for (int j = 0; j < EPT / 2; ++j) {
    *(uint32_t*)(K + 2 * j) = o1[j];
    *(uint32_t*)(K + HALF + 2 * j) = o2[j];
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    VT[(size_t)(EPT * t16 + j) * a.cap] = f2bf(v1[j]);
    VT[(size_t)(HALF + EPT * t16 + j) * a.cap] = f2bf(v2[j]);
  }
}

template <int HD>
__global__ __launch_bounds__(256) void ring_write16_kernel(AttnShape a, const float* __restrict__ kv,
                                                           const void* const* knorms, int64_t pos0,
                                                           uint16_t* ring) {
  __shared__ float2 rot[HD / 2];
  ring_write16_row<HD>(a, kv, knorms, (int)blockIdx.x, pos0 + blockIdx.x, ring, rot);
}

// The rows of several sequences in one launch: row r belongs to the sequence whose rows
// first[q]..first[q+1]-1 hold it (one search per work-group over the by-value table), at
// position start[q] + r - first[q], into that sequence's ring.
template <int HD>
__global__ __launch_bounds__(256) void ring_write16_batch_kernel(AttnShape a, RingSeqs seqs,
                                                                 const float* __restrict__ kv,
                                                                 const void* const* knorms, uint16_t* ring0,
                                                                 size_t ring_stride) {
  __shared__ float2 rot[HD / 2];
  const int r = blockIdx.x;
  int q = 0;
  while (q + 1 < seqs.n && r >= seqs.first[q + 1]) ++q;
  uint16_t* ring = (uint16_t*)((unsigned char*)ring0 + (size_t)q * ring_stride);
  ring_write16_row<HD>(a, kv, knorms, r, seqs.start[q] + (r - seqs.first[q]), ring, rot);
}

// ---- context K/V into the ring, other shapes --------------------------------------------
// kv: f32 [n, L, 2, nkv, hd] (k then v per layer). One wave per (row, layer, kv slot).
// ring: act, per layer K [nkv][Cs][hd] then V^T [nkv][hd][Cs].
template <bool BF>
__global__ __launch_bounds__(256) void ring_write_kernel(AttnShape a, const float* __restrict__ kv,
                                                         const void* const* knorms, int n, int64_t pos0,
                                                         void* ring) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int per_row = a.L * 2 * a.nkv;
  if (item >= n * per_row) return;
  const int r = item / per_row;
  int rem = item - r * per_row;
  const int l = rem / (2 * a.nkv);
  rem -= l * 2 * a.nkv;
  const int isv = rem / a.nkv, h = rem - isv * a.nkv;
  const int hd = a.hd, half = hd >> 1;
  const float* src = kv + (size_t)item * hd;
  const bool act = lane < half;
  float x1 = act ? src[lane] : 0.f, x2 = act ? src[lane + half] : 0.f;
  const int64_t pos = pos0 + r;
  const size_t slot = (size_t)ring_slot(a, pos);
  // K row at (l, 0, h, slot); V element d at (l, 1, h, d, slot)
  const size_t plane = (((size_t)l * 2 + isv) * a.nkv + h) * (size_t)a.cap * hd;
  if (!isv) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float s = rsqrtf(ss / (float)hd + a.eps);
    if (!act) return;
    const void* g = knorms[l];
    x1 = x1 * s * act_ld<BF>(g, lane);
    x2 = x2 * s * act_ld<BF>(g, lane + half);
    const double inv = pow((double)a.theta, -2.0 * (double)lane / (double)hd);
    double sn, cs;
    sincos((double)pos * inv, &sn, &cs);
    const float c = (float)cs, sf = (float)sn;
    const float y1 = x1 * c - x2 * sf, y2 = x2 * c + x1 * sf;
    x1 = y1;
    x2 = y2;
  }
  if (act) {
    if (!isv) {
      act_st<BF>(ring, plane + slot * hd + lane, x1);
      act_st<BF>(ring, plane + slot * hd + lane + half, x2);
    } else {
      act_st<BF>(ring, plane + (size_t)lane * a.cap + slot, x1);
      act_st<BF>(ring, plane + (size_t)(lane + half) * a.cap + slot, x2);
    }
  }
}

// Keys of a query: absolute positions lo..e+R-1 (lo = max(0, e - W)); chunk c of a launch
// covers positions (lo/64 + c)*64 .. + 64.
__host__ __device__ inline int64_t attn_lo(const AttnShape& a, int64_t e) {
  if (a.causal) return e > a.window - 1 ? e - (a.window - 1) : 0;  // the query at e sees e-W+1..e
  return e > a.window ? e - a.window : 0;
}
__host__ __device__ inline int attn_nchunks(const AttnShape& a, int R, int64_t e) {
  return (int)((e + R - 1) / ATTN_CHUNK - attn_lo(a, e) / ATTN_CHUNK + 1);
}

// ---- attention: partial softmax per (kv head, key chunk), VALU path ---------------------
// (f32 shapes and head dims without an MFMA kernel.) Query vector qi = r * G + hh (G = nq
// / nkv query heads of kv head g). part layout: [nkv][nchunks][R*G][PART_STRIDE(hd)] =
// (unnormalised output, m, l).
template <bool BF>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnShape a, const void* ring_layer, const void* qb,
                                                           const void* qlo, int R, int64_t e, int nchunks,
                                                           float* __restrict__ part) {
  extern __shared__ __align__(16) float sm[];
  const int g = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hd = a.hd, G = a.nq / a.nkv, NQ = R * G;
  const int KS = hd + 1;  // padded row stride of staged K (bank spread)
  float* Ks = sm;                          // [64][hd+1]
  float* Vs = Ks + ATTN_CHUNK * KS;        // [64][hd]
  float* Qs = Vs + ATTN_CHUNK * hd;        // [ATTN_QG][hd]
  float* Ss = Qs + ATTN_QG * hd;           // [ATTN_QG][64]

  const int64_t lo = attn_lo(a, e), hi = e + R;
  const int64_t p0 = (lo / ATTN_CHUNK + c) * ATTN_CHUNK;
  const size_t plane = (size_t)a.cap * hd;
  const void* Kr = (const unsigned char*)ring_layer + ((size_t)g * plane) * (BF ? 2 : 4);
  const void* Vr = (const unsigned char*)ring_layer + ((size_t)(a.nkv + g) * plane) * (BF ? 2 : 4);

  // stage this chunk's keys and values (f32); every slot holds finite values
  for (int i = tid; i < ATTN_CHUNK * hd; i += blockDim.x) {
    const int kj = i / hd, d = i - kj * hd;
    const size_t slot = (size_t)ring_slot(a, p0 + kj);
    Ks[kj * KS + d] = act_ld<BF>(Kr, slot * hd + d);
    Vs[kj * hd + d] = act_ld<BF>(Vr, (size_t)d * a.cap + slot);
  }
  const float scale = 1.0f / sqrtf((float)hd);

  for (int q0 = 0; q0 < NQ; q0 += ATTN_QG) {
    const int nq = min(ATTN_QG, NQ - q0);
    __syncthreads();
    for (int i = tid; i < nq * hd; i += blockDim.x) {
      const int qi = i / hd, d = i - qi * hd;
      const int gq = q0 + qi, r = gq / G, hh = gq - r * G;
      const size_t qo = ((size_t)r * a.nq + (size_t)g * G + hh) * hd + d;
      if constexpr (BF) Qs[qi * hd + d] = bf2f(((const uint16_t*)qb)[qo]) + bf2f(((const uint16_t*)qlo)[qo]);
      else Qs[qi * hd + d] = ((const float*)qb)[qo];
    }
    __syncthreads();
    // scores: thread -> key lane, queries strided by waves
    {
      const int kj = lane;
      const int64_t kp = p0 + kj;
      for (int qi = w; qi < nq; qi += 4) {
        float sc = -INFINITY;
        const int64_t qp = e + (q0 + qi) / G;
        const int64_t dist = qp > kp ? qp - kp : kp - qp;
        const bool in_window = a.causal ? (kp <= qp && qp - kp < a.window) : dist <= a.window;
        if (kp >= lo && kp < hi && in_window) {
          float s = 0.f;
          const float* qv = Qs + qi * hd;
          const float* kv = Ks + kj * KS;
          for (int d = 0; d < hd; ++d) s += qv[d] * kv[d];
          sc = s * scale;
        }
        Ss[qi * ATTN_CHUNK + kj] = sc;
      }
    }
    __syncthreads();
    // per-query max / exp / sum, one wave per query
    for (int qi = w; qi < nq; qi += 4) {
      const float s = Ss[qi * ATTN_CHUNK + lane];
      const float m = wave_max(s);
      const float pexp = (s == -INFINITY) ? 0.f : expf(s - m);
      Ss[qi * ATTN_CHUNK + lane] = pexp;
      const float l = wave_sum(pexp);
      if (lane == 0) {
        float* dst = part + (((size_t)g * nchunks + c) * NQ + q0 + qi) * PART_STRIDE(hd);
        dst[hd] = m;
        dst[hd + 1] = l;
      }
    }
    __syncthreads();
    // unnormalised output: thread -> d, queries strided
    for (int i = tid; i < nq * hd; i += blockDim.x) {
      const int qi = i / hd, d = i - qi * hd;
      float o = 0.f;
      const float* pr = Ss + qi * ATTN_CHUNK;
      for (int kj = 0; kj < ATTN_CHUNK; ++kj) o += pr[kj] * Vs[kj * hd + d];
      part[(((size_t)g * nchunks + c) * NQ + q0 + qi) * PART_STRIDE(hd) + d] = o;
    }
  }
}

// N consecutive f32 (16-, 8- or 4-byte aligned for N = 4, 2, 1 per vector) and bf16 values
template <int N>
__device__ __forceinline__ void ld_f32(const float* p, float (&o)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 v = *(const float4*)(p + i);
      o[i] = v.x; o[i + 1] = v.y; o[i + 2] = v.z; o[i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      const float2 v = *(const float2*)(p + i);
      o[i] = v.x; o[i + 1] = v.y;
    }
  }
}
template <int N>
__device__ __forceinline__ void ld_bf16(const uint16_t* p, float (&o)[N]) {
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    const uint32_t w = *(const uint32_t*)(p + i);
    o[i] = __uint_as_float(w << 16);
    o[i + 1] = __uint_as_float(w & 0xffff0000u);
  }
}
template <int N>
__device__ __forceinline__ void st_u16(uint16_t* p, const uint16_t (&v)[N]) {
  if constexpr (N == 4) {
    *(uint2*)p = make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16));
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 2) *(uint32_t*)(p + i) = (uint32_t)v[i] | ((uint32_t)v[i + 1] << 16);
  }
}

// ---- attention on MFMA (bf16 operands): one work-group per (64-key chunk, kv head, query part)
// The work-group copies the chunk's keys and transposed values from the ring into LDS once
// (16-byte units spread over all its threads), and each wave takes at most one 16-query
// tile, reading its MFMA operands from LDS: scores S^T = K Q^T (16x16x32 bf16 MFMA; A = 16
// key rows, B = 16 queries), then O^T = V^T P^T (A = 16 dims x 32 keys of V^T, B = P). The
// key rows of the two score tiles of each 32-key half are ordered so that lane (li, lg)
// ends up with keys 8*lg .. 8*lg+7 of the half for query li, exactly its B operand of the
// output product, and the matching V^T run is one 16-byte read. Q (an f32 activation) and
// P (in [0, 1]) enter as bf16 pairs hi + lo, about 16 significant bits; K and V are bf16
// already, products are exact and sums f32. The launch splits the query tiles over
// gridDim.z work-groups of 4 waves, so no wave runs two tiles in turn.
//
// The kernel also does what the prep kernel does for the block rows. A query fragment holds
// dims 32s + 8lg .. + 8 of one query, so the lane's four lanes lg together hold the whole
// head (the RMSNorm sum is two shuffles) and each rotate-half partner, dim + hd/2, sits in
// the same lane (s + DS/2). The block's own keys and values, at positions e..e+R-1, are
// formed by the work-groups whose chunk holds them, one wave per position as in the prep
// kernel, and written into the LDS slots of those positions; the ring copy skips them (the
// ring slots past the committed window are not written).
//
// Loads retire in issue order: the raw block rows go out first, then the wave's query tile,
// then the ring copy, so the staging and the query arithmetic overlap the copy's fetch.
// NW waves per work-group (the chunk copy divides evenly over them); BLK: the chunk holds block
// positions. Every load is issued without a branch, so that each wait before the arithmetic
// covers only the loads it needs.
template <int HD, int NW, bool BLK>
__device__ __forceinline__ void attn_mfma_body(const AttnShape& a, uint16_t* ring_layer,
                                               const float* __restrict__ qkv, const uint16_t* __restrict__ qnorm,
                                               const uint16_t* __restrict__ knorm, const float2* __restrict__ rope,
                                               int R, int n, int64_t e, int nchunks, int tpw, int zi,
                                               float* __restrict__ part, uint16_t* __restrict__ kst,
                                               uint16_t* __restrict__ vst) {
  constexpr int KC = ATTN_CHUNK;  // 64 positions = two halves of 32
  constexpr int DS = HD / 32, DT = HD / 16, HALF = HD / 2;
  constexpr int KSTR = HD + 8;      // LDS key row stride (elements)
  constexpr int VSTR = KC + 8;      // LDS V^T row stride (elements)
  constexpr int KU = KC * HD / 8;   // 16-byte units of the chunk's keys (and of its values)
  constexpr int NIT = KU / (64 * NW);
  constexpr int EPT = HALF / 16;    // staging: dims per lane and half, 16 lanes per position
  static_assert(KC == 64 && KU % (64 * NW) == 0, "two 32-key halves, an even copy");
  const int g = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int G = a.nq / a.nkv, NQ = R * G;
  const int qt = zi * tpw + w;  // zi: this work-group's share of the query tiles
  const bool active = w < tpw && qt * 16 < NQ;  // other waves only copy and stage
  const int64_t lo = attn_lo(a, e), hi = e + R;
  const int64_t p0 = (lo / KC + c) * KC;
  const int C = a.cap;
  const size_t ldq = (size_t)(a.nq + 2 * a.nkv) * HD;  // raw projection row
  // positions formed from the raw projections: the n committed rows e-n..e-1 (projection
  // rows R..R+n-1, also written into their ring slots here) and the block e..e+R-1 (rows
  // 0..R-1); this chunk's share b0 .. b1-1 (non-empty when BLK)
  const int64_t bs = e - n;
  const int64_t b0 = p0 > bs ? p0 : bs, b1 = p0 + KC < hi ? p0 + KC : hi;
  auto row_of = [&](int64_t p) { return p >= e ? (int)(p - e) : R + (int)(p - bs); };
  const uint16_t* Kp = ring_layer + (size_t)g * C * HD;
  const uint16_t* VTp = ring_layer + (size_t)(a.nkv + g) * HD * C;
  // slot of the chunk's first position: a multiple of 8 (p0, phase and Cs are), so the
  // runs p0 + 8j .. + 8 sit in consecutive slots s0 + 8j (mod Cs) that never wrap
  const int s0 = (int)ring_slot(a, p0);
  auto slot_at = [&](int kk) { const int sl = s0 + kk; return sl >= C ? sl - C : sl; };

  // ---- (1) raw block rows: 16 lanes per position, four positions per wave and step; step k
  // of wave w takes positions b0 + 4 (w + NW k) + lg, and lane t16 of a position holds dims
  // EPT t16 .. + EPT and their rotate-half partners (+ HD/2). Step 0 loads up front, its
  // rows clamped into the block range.
  const int t16 = lane & 15;
  float bk1[EPT], bk2[EPT], bv1[EPT], bv2[EPT], bcs[2 * EPT], kg1[EPT], kg2[EPT];
  auto load_block_row = [&](int64_t p) {
    const int rr = row_of(p < b1 ? p : b1 - 1);
    const float* kr = qkv + (size_t)rr * ldq + (size_t)(a.nq + g) * HD + EPT * t16;
    const float* vr = qkv + (size_t)rr * ldq + (size_t)(a.nq + a.nkv + g) * HD + EPT * t16;
    ld_f32<EPT>(kr, bk1);
    ld_f32<EPT>(kr + HALF, bk2);
    ld_f32<EPT>(vr, bv1);
    ld_f32<EPT>(vr + HALF, bv2);
    ld_f32<2 * EPT>((const float*)(rope + (size_t)rr * HALF + EPT * t16), bcs);
  };
  if constexpr (BLK) {
    ld_bf16<EPT>(knorm + EPT * t16, kg1);
    ld_bf16<EPT>(knorm + HALF + EPT * t16, kg2);
    load_block_row(b0 + 4 * w + lg);
  }
  // ---- (2) the wave's query tile: raw q of (row r, head g*G + hh), gains, rotary table; a
  // wave without a tile loads row 0 and discards it ------------------------------------------
  const int qv = qt * 16 + li;
  const bool qok = active && qv < NQ;
  const int rq = (int)((unsigned)qv / (unsigned)G);
  const int r = qok ? rq : 0, hh = qok ? qv - rq * G : 0;
  float x[DS][8];
  u32x4_t gq[DS];
  float4 cs2[DS / 2][4];  // two (cos, sin) per float4
  {
    const float* src = qkv + (size_t)r * ldq + (size_t)(g * G + hh) * HD;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const float4 a0 = *(const float4*)(src + 32 * s + 8 * lg), a1 = *(const float4*)(src + 32 * s + 8 * lg + 4);
      x[s][0] = a0.x; x[s][1] = a0.y; x[s][2] = a0.z; x[s][3] = a0.w;
      x[s][4] = a1.x; x[s][5] = a1.y; x[s][6] = a1.z; x[s][7] = a1.w;
    }
#pragma unroll
    for (int s = 0; s < DS; ++s) gq[s] = *(const u32x4_t*)(qnorm + 32 * s + 8 * lg);
    const float4* rrow = (const float4*)(rope + (size_t)r * HALF);
#pragma unroll
    for (int s = 0; s < DS / 2; ++s)
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) cs2[s][j2] = rrow[(32 * s + 8 * lg) / 2 + j2];
  }
  // ---- (3) the ring copy: unit u is key row u / (HD/8), dims 8 (u % (HD/8)) .. + 8, and
  // V^T dim u / 8, chunk offsets 8 (u % 8) .. + 8 ---------------------------------------------
  u32x4_t kr[NIT], vr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int u = tid + 64 * NW * it;
    kr[it] = *(const u32x4_t*)(Kp + (size_t)slot_at(u / (HD / 8)) * HD + 8 * (u % (HD / 8)));
    vr[it] = *(const u32x4_t*)(VTp + (size_t)(u >> 3) * C + slot_at(8 * (u & 7)));
  }
  // every load above is issued before any of the arithmetic below
  __builtin_amdgcn_sched_barrier(0);

  // ---- (4) the block's own keys of step 0: RMSNorm, gain and RoPE, then bf16 (the ring's
  // dtype); values cast to bf16 --------------------------------------------------------------
  uint32_t sk1[EPT / 2], sk2[EPT / 2];  // packed bf16 pairs
  uint16_t sv1[EPT], sv2[EPT];
  auto stage = [&]() {
    form_key16<HD>(bk1, bk2, kg1, kg2, bcs, a.eps, sk1, sk2);
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      sv1[j] = f2bf(bv1[j]);
      sv2[j] = f2bf(bv2[j]);
    }
  };
  auto put = [&](int64_t p) {  // the staged position into its LDS slots
    if (p < b1) {
      const int i = (int)(p - p0);
#pragma unroll
      for (int j = 0; j < EPT / 2; ++j) {
        *(uint32_t*)(kst + i * KSTR + EPT * t16 + 2 * j) = sk1[j];
        *(uint32_t*)(kst + i * KSTR + HALF + EPT * t16 + 2 * j) = sk2[j];
      }
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        vst[(EPT * t16 + j) * VSTR + i] = sv1[j];
        vst[(HALF + EPT * t16 + j) * VSTR + i] = sv2[j];
      }
      if ((p < e || a.causal) && zi == 0) {  // a committed (or target block) row: also into its slots
        uint16_t* Kw = ring_layer + (size_t)g * C * HD + (size_t)slot_at(i) * HD + EPT * t16;
        uint16_t* VTw = ring_layer + (size_t)(a.nkv + g) * HD * C + slot_at(i);
#pragma unroll
        for (int j = 0; j < EPT / 2; ++j) {
          *(uint32_t*)(Kw + 2 * j) = sk1[j];
          *(uint32_t*)(Kw + HALF + 2 * j) = sk2[j];
        }
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          VTw[(size_t)(EPT * t16 + j) * C] = sv1[j];
          VTw[(size_t)(HALF + EPT * t16 + j) * C] = sv2[j];
        }
      }
    }
  };
  if constexpr (BLK) stage();

  // ---- (5) the query tile as hi/lo operand pairs: RMSNorm over the head, gain, RoPE --------
  u32x4_t qf[DS], qfl[DS];
  {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(x[s][j], x[s][j], ss);
    ss += __shfl_xor(ss, 16, 64);  // the four lanes of query li, in a fixed order
    ss += __shfl_xor(ss, 32, 64);
    const float sq = rsqrtf(ss / (float)HD + a.eps);
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t gw = gq[s][j >> 1];
        x[s][j] = x[s][j] * sq * __uint_as_float((j & 1) ? (gw & 0xffff0000u) : (gw << 16));
      }
#pragma unroll
    for (int s = 0; s < DS / 2; ++s)
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * j2 + u;
          const float cc = u ? cs2[s][j2].z : cs2[s][j2].x, sn = u ? cs2[s][j2].w : cs2[s][j2].y;
          const float x1 = x[s][j], x2 = x[s + DS / 2][j];
          x[s][j] = x1 * cc - x2 * sn;
          x[s + DS / 2][j] = x2 * cc + x1 * sn;
        }
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t hp, lp;
        split2_bf16(x[s][2 * t], x[s][2 * t + 1], hp, lp);
        qf[s][t] = hp;
        qfl[s][t] = lp;
      }
  }

  // the operands are formed here, while the ring copy is in flight: the compiler may not
  // move their loads and arithmetic past the barrier below
#pragma unroll
  for (int s = 0; s < DS; ++s) asm volatile("" : "+v"(qf[s]), "+v"(qfl[s]));
  if constexpr (BLK) {
#pragma unroll
    for (int j = 0; j < EPT / 2; ++j) asm volatile("" : "+v"(sk1[j]), "+v"(sk2[j]));
#pragma unroll
    for (int j = 0; j < EPT; ++j) asm volatile("" : "+v"(sv1[j]), "+v"(sv2[j]));
  }

  // ---- (6) the ring values into LDS; in a chunk with block positions the staged values
  // then overwrite their slots (a barrier apart) ------------------------------------------------
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int u = tid + 64 * NW * it;
    *(u32x4_t*)(kst + (u / (HD / 8)) * KSTR + 8 * (u % (HD / 8))) = kr[it];
    *(u32x4_t*)(vst + (u >> 3) * VSTR + 8 * (u & 7)) = vr[it];
  }
  __syncthreads();
  if constexpr (BLK) {
    put(b0 + 4 * w + lg);
    for (int64_t pb = b0 + 4 * (w + NW); pb < b1; pb += 4 * NW) {  // long blocks
      load_block_row(pb + lg);
      stage();
      put(pb + lg);
    }
    __syncthreads();
  }
  if (!active) return;  // no barrier below

  // ---- (7) scores, softmax over the chunk, output -----------------------------------------
  // Logits are carried in base 2: t = (q . k) scale log2(e), p = 2^(t - m2); the partial
  // stores m = m2 ln(2), the chunk maximum of the natural logits.
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  // key offsets relative to e: the query is at e + r; visible keys lie in lo..e+R-1 with
  // |query - key| <= W, all within int range (the chunk is within W + 64 of e)
  const int kbase = (int)(p0 - e), klo = (int)(lo - e);
  // key fragments: the A operand row li of tile (h, tb) is chunk offset 32h + 8*(li/4) +
  // 4*tb + li%4; value fragments: dims dt*16 + li, chunk offsets 32h + 8*lg .. + 8
  u32x4_t kf[2][2][DS], vf[2][DT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int s = 0; s < DS; ++s)
        kf[h][tb][s] = *(const u32x4_t*)(kst + (32 * h + 8 * (li >> 2) + 4 * tb + (li & 3)) * KSTR + 32 * s + 8 * lg);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[h][dt] = *(const u32x4_t*)(vst + (dt * 16 + li) * VSTR + 32 * h + 8 * lg);
  float S[2][2][4];
  float m = -INFINITY;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      // element i of tile (h, tb) is chunk offset 32h + 8*lg + 4*tb + i for query li
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        acc = mfma_bf16(kf[h][tb][s], qf[s], acc);
        acc = mfma_bf16(kf[h][tb][s], qfl[s], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kp = kbase + 32 * h + 8 * lg + 4 * tb + i;
        const int dist = r > kp ? r - kp : kp - r;
        const bool in_window = a.causal ? (kp <= r && r - kp < a.window) : dist <= a.window;
        const bool vis = qok && kp >= klo && kp < R && in_window;
        S[h][tb][i] = vis ? acc[i] * sl2 : -INFINITY;
        m = fmaxf(m, S[h][tb][i]);
      }
    }
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  float l = 0.f;
  u32x4_t phi[2], plo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // word t holds keys 8*lg + 2t, 2t + 1 of the half
      float pv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 2 * t + u, tb = j >> 2, i = j & 3;
        const float sv = S[h][tb][i];
        pv[u] = sv == -INFINITY ? 0.f : exp2f(sv - m);
        l += pv[u];
      }
      uint32_t hp, lp;
      split2_bf16(pv[0], pv[1], hp, lp);
      phi[h][t] = hp;
      plo[h][t] = lp;
    }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  float* dst = part + (((size_t)g * nchunks + c) * NQ + qv) * PART_STRIDE(HD);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      o = mfma_bf16(vf[h][dt], phi[h], o);
      o = mfma_bf16(vf[h][dt], plo[h], o);
    }
    if (qok) *(f32x4_t*)&dst[dt * 16 + 4 * lg] = o;  // dims dt*16 + 4*lg .. + 4 of query qv
  }
  if (qok && lg == 0) {
    dst[HD] = m * 0.6931471805599453f;
    dst[HD + 1] = l;
  }
}

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) void attn_mfma_kernel(AttnShape a, uint16_t* ring_layer,
                                                            const float* __restrict__ qkv,
                                                            const uint16_t* __restrict__ qnorm,
                                                            const uint16_t* __restrict__ knorm,
                                                            const float2* __restrict__ rope, int R, int n, int64_t e,
                                                            int nchunks, int tpw, float* __restrict__ part) {
  // the chunk's keys [chunk position][hd + 8] and values transposed [dim][64 + 8]
  __shared__ __align__(16) uint16_t kst[ATTN_CHUNK * (HD + 8)];
  __shared__ __align__(16) uint16_t vst[HD * (ATTN_CHUNK + 8)];
  const int64_t p0 = (attn_lo(a, e) / ATTN_CHUNK + blockIdx.x) * ATTN_CHUNK;
  if (p0 < e + R && e - n < p0 + ATTN_CHUNK)
    attn_mfma_body<HD, NW, true>(a, ring_layer, qkv, qnorm, knorm, rope, R, n, e, nchunks, tpw, blockIdx.z, part, kst,
                                 vst);
  else
    attn_mfma_body<HD, NW, false>(a, ring_layer, qkv, qnorm, knorm, rope, R, n, e, nchunks, tpw, blockIdx.z, part, kst,
                                  vst);
}

// Independent sequences in one launch (a batch round): blockIdx.z = sequence * zq + query
// part. Sequence s has its own committed end, ring (ring_seq elements after s - 1's), R
// rows of raw projections and rotary table after s - 1's, and a partial region of
// part_seq floats laid out as a single sequence's with its own chunk count; chunks past
// that count return at once. No committed rows travel with a batch draft (n = 0).
template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) void attn_mfma_batch_kernel(AttnShape a, AttnSeqs seqs, uint16_t* ring0,
                                                                  size_t ring_seq, const float* __restrict__ qkv,
                                                                  const uint16_t* __restrict__ qnorm,
                                                                  const uint16_t* __restrict__ knorm,
                                                                  const float2* __restrict__ rope, int R, int zq,
                                                                  int tpw, size_t part_seq, float* __restrict__ part) {
  __shared__ __align__(16) uint16_t kst[ATTN_CHUNK * (HD + 8)];
  __shared__ __align__(16) uint16_t vst[HD * (ATTN_CHUNK + 8)];
  const int s = blockIdx.z / zq, zi = blockIdx.z - s * zq;
  const int64_t e = seqs.e[s];
  const int nch = attn_nchunks(a, R, e);
  if ((int)blockIdx.x >= nch) return;
  const size_t ldq = (size_t)(a.nq + 2 * a.nkv) * HD;
  uint16_t* ring_layer = ring0 + (size_t)s * ring_seq;
  const float* q_s = qkv + (size_t)s * R * ldq;
  const float2* rope_s = rope + (size_t)s * R * (HD / 2);
  float* part_s = part + (size_t)s * part_seq;
  const int64_t p0 = (attn_lo(a, e) / ATTN_CHUNK + blockIdx.x) * ATTN_CHUNK;
  if (p0 < e + R && e < p0 + ATTN_CHUNK)  // the chunk holds block positions
    attn_mfma_body<HD, NW, true>(a, ring_layer, q_s, qnorm, knorm, rope_s, R, 0, e, nch, tpw, zi, part_s, kst, vst);
  else
    attn_mfma_body<HD, NW, false>(a, ring_layer, q_s, qnorm, knorm, rope_s, R, 0, e, nch, tpw, zi, part_s, kst, vst);
}

// ---- combine chunks in chunk order --------------------------------------------------------
// One work-group (hd threads) per (row, query head); out: the O-projection operand [R,
// nq*hd] (hi/lo bf16 planes, or f32). The chunk maxima and sums are staged in LDS first so
// the output loop issues independent loads.
constexpr int COMBINE_MAX_CHUNKS = 80;
template <bool BF>
__global__ void attn_combine_kernel(AttnShape a, const float* __restrict__ part, int R, int nchunks, void* out,
                                    void* out_lo) {
  __shared__ float sm_m[COMBINE_MAX_CHUNKS], sm_l[COMBINE_MAX_CHUNKS];
  const int item = blockIdx.x;
  const int r = item / a.nq, h = item - r * a.nq;
  const int G = a.nq / a.nkv, g = h / G, hh = h - g * G;
  const int NQ = R * G, qi = r * G + hh;
  const int d = threadIdx.x, hd = a.hd;
  const size_t stride = (size_t)NQ * PART_STRIDE(hd);
  const float* base = part + ((size_t)g * nchunks * NQ + qi) * PART_STRIDE(hd);
  for (int c = d; c < nchunks; c += blockDim.x) {
    sm_m[c] = base[c * stride + hd];
    sm_l[c] = base[c * stride + hd + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, sm_m[c]);
  float L = 0.f, O = 0.f;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) {
    const float m = sm_m[c];
    const float f = m == -INFINITY ? 0.f : expf(m - M);
    L += sm_l[c] * f;
    O += base[c * stride + d] * f;
  }
  op_st<BF>(out, out_lo, (size_t)r * a.nq * hd + (size_t)h * hd + d, O / L);
}

// The same for a batch round: blockIdx.x = sequence * R * nq + item, each sequence with its
// own chunk count, partial region (part_seq floats) and output rows s * R ..
template <bool BF>
__global__ void attn_combine_batch_kernel(AttnShape a, AttnSeqs seqs, const float* __restrict__ part, size_t part_seq,
                                          int R, void* out, void* out_lo) {
  __shared__ float sm_m[COMBINE_MAX_CHUNKS], sm_l[COMBINE_MAX_CHUNKS];
  const int per = R * a.nq;
  const int s = blockIdx.x / per, item = blockIdx.x - s * per;
  const int nchunks = attn_nchunks(a, R, seqs.e[s]);
  const int r = item / a.nq, h = item - r * a.nq;
  const int G = a.nq / a.nkv, g = h / G, hh = h - g * G;
  const int NQ = R * G, qi = r * G + hh;
  const int d = threadIdx.x, hd = a.hd;
  const size_t stride = (size_t)NQ * PART_STRIDE(hd);
  const float* base = part + (size_t)s * part_seq + ((size_t)g * nchunks * NQ + qi) * PART_STRIDE(hd);
  for (int c = d; c < nchunks; c += blockDim.x) {
    sm_m[c] = base[c * stride + hd];
    sm_l[c] = base[c * stride + hd + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, sm_m[c]);
  float L = 0.f, O = 0.f;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) {
    const float m = sm_m[c];
    const float f = m == -INFINITY ? 0.f : expf(m - M);
    L += sm_l[c] * f;
    O += base[c * stride + d] * f;
  }
  op_st<BF>(out, out_lo, ((size_t)s * R + r) * a.nq * hd + (size_t)h * hd + d, O / L);
}

// ---- live window read-back (parity checks) -----------------------------------------------
template <bool BF>
__global__ void cache_read_kernel(AttnShape a, const void* ring_layer, int64_t lo, int n, void* kout, void* vout,
                                  int deint) {
  const int hd = a.hd;
  const size_t total = (size_t)a.nkv * n * hd;
  const size_t plane = (size_t)a.cap * hd;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(i % hd);
    const size_t t = i / hd;
    const int j = (int)(t % n), h = (int)(t / n);
    const size_t slot = (size_t)ring_slot(a, lo + j);
    // K [h][slot][d], element d of the original order at d/2 or hd/2 + d/2 when deinterleaved
    const int dk = deint ? (d & 1 ? hd / 2 + (d >> 1) : d >> 1) : d;
    const size_t ko = (size_t)h * plane + slot * hd + dk;
    const size_t vo = (size_t)(a.nkv + h) * plane + (size_t)d * a.cap + slot;  // V^T [h][d][slot]
    if constexpr (BF) {
      ((uint16_t*)kout)[i] = ((const uint16_t*)ring_layer)[ko];
      ((uint16_t*)vout)[i] = ((const uint16_t*)ring_layer)[vo];
    } else {
      ((float*)kout)[i] = ((const float*)ring_layer)[ko];
      ((float*)vout)[i] = ((const float*)ring_layer)[vo];
    }
  }
}

// ---- launchers ------------------------------------------------------------------------------
static hipError_t launch_attn_prep(int bf, const AttnShape& a, const float* qkv, const void* qnorm, const void* knorm,
                            int R, int64_t pos0, void* qb, void* qlo, void* ring_layer, hipStream_t s) {
  const int items = R * (a.nq + 2 * a.nkv);
  const int grid = (items + 3) / 4;
  if (bf)
    hipLaunchKernelGGL(attn_prep_kernel<true>, dim3(grid), dim3(256), 0, s, a, qkv, qnorm, knorm, R, pos0, qb, qlo,
                       ring_layer);
  else
    hipLaunchKernelGGL(attn_prep_kernel<false>, dim3(grid), dim3(256), 0, s, a, qkv, qnorm, knorm, R, pos0, qb, qlo,
                       ring_layer);
  return hipGetLastError();
}

static bool use_mfma(int bf, const AttnShape& a) { return bf && (a.hd == 64 || a.hd == 128); }

hipError_t launch_ring_write_batch(int bf, const AttnShape& a, const float* kv, const void* const* knorms,
                                   const RingSeqs& seqs, void* ring0, size_t ring_stride, hipStream_t s) {
  if (!use_mfma(bf, a)) return hipErrorNotSupported;
  if (seqs.n < 1 || seqs.n > ATTN_MAX_SEQS || seqs.first[0] != 0 || seqs.first[seqs.n] < 1)
    return hipErrorInvalidValue;
  for (int q = 0; q < seqs.n; ++q)
    if (seqs.first[q + 1] < seqs.first[q]) return hipErrorInvalidValue;
  auto* fn = a.hd == 128 ? ring_write16_batch_kernel<128> : ring_write16_batch_kernel<64>;
  hipLaunchKernelGGL(fn, dim3(seqs.first[seqs.n], (a.L * a.nkv + 15) / 16), dim3(256), 0, s, a, seqs, kv, knorms,
                     (uint16_t*)ring0, ring_stride);
  return hipGetLastError();
}

hipError_t launch_ring_write(int bf, const AttnShape& a, const float* kv, const void* const* knorms, int n,
                             int64_t pos0, void* ring, hipStream_t s) {
  if (use_mfma(bf, a)) {  // keys formed as the attention forms its own
    auto* fn = a.hd == 128 ? ring_write16_kernel<128> : ring_write16_kernel<64>;
    hipLaunchKernelGGL(fn, dim3(n, (a.L * a.nkv + 15) / 16), dim3(256), 0, s, a, kv, knorms, pos0, (uint16_t*)ring);
    return hipGetLastError();
  }
  const int items = n * a.L * 2 * a.nkv;
  const int grid = (items + 3) / 4;
  if (bf) hipLaunchKernelGGL(ring_write_kernel<true>, dim3(grid), dim3(256), 0, s, a, kv, knorms, n, pos0, ring);
  else hipLaunchKernelGGL(ring_write_kernel<false>, dim3(grid), dim3(256), 0, s, a, kv, knorms, n, pos0, ring);
  return hipGetLastError();
}

size_t attention_partial_floats_span(const AttnShape& a, int R, int span) {
  // chunks of a launch: positions lo..e+R-1 (at most span + R of them) cut at multiples of 64
  const int nch = (span + R + 2 * ATTN_CHUNK - 2) / ATTN_CHUNK;
  return (size_t)a.nkv * nch * R * (a.nq / a.nkv) * PART_STRIDE(a.hd);
}

size_t attention_partial_floats(const AttnShape& a, int R) { return attention_partial_floats_span(a, R, a.window); }

bool attention_forms_committed_rows(int bf, const AttnShape& a) { return use_mfma(bf, a); }

hipError_t launch_block_attention(int bf, const AttnShape& a, const float* qkv, const void* qnorm, const void* knorm,
                                  const float2* rope, void* ring_layer, int R, int n, int64_t e, void* qb, void* qlo,
                                  float* part, void* out, void* out_lo, hipStream_t s) {
  const int nch = attn_nchunks(a, R, e);
  if (nch > COMBINE_MAX_CHUNKS || R < 1 || n < 0 || n > e || n > a.window) return hipErrorInvalidValue;
  if (n > 0 && !use_mfma(bf, a)) return hipErrorInvalidValue;
  dim3 grid(nch, a.nkv);
  if (use_mfma(bf, a)) {
    if (!rope) return hipErrorInvalidValue;
    uint16_t* rl = (uint16_t*)ring_layer;
    const uint16_t *qn = (const uint16_t*)qnorm, *kn = (const uint16_t*)knorm;
    // query tiles over z work-groups of 4 waves, at most one tile per wave: two such
    // work-groups fit a CU, where an 8-wave one (150 registers) leaves room for no second
    const int nqt = (R * (a.nq / a.nkv) + 15) / 16;
    const int z = (nqt + 3) / 4, tpw = (nqt + z - 1) / z;
    const dim3 mgrid(nch, a.nkv, z);
    auto* fn = a.hd == 128 ? attn_mfma_kernel<128, 4> : attn_mfma_kernel<64, 4>;
    hipLaunchKernelGGL(fn, mgrid, dim3(256), 0, s, a, rl, qkv, qn, kn, rope, R, n, e, nch, tpw, part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(attn_combine_kernel<true>, dim3(R * a.nq), dim3(a.hd), 0, s, a, part, R, nch, out, out_lo);
    return hipGetLastError();
  }
  // queries as operands, the block's own k/v into the ring slots of positions e..e+R-1
  {
    const hipError_t pe = launch_attn_prep(bf, a, qkv, qnorm, knorm, R, e, qb, qlo, ring_layer, s);
    if (pe != hipSuccess) return pe;
  }
  const size_t lds = (size_t)(ATTN_CHUNK * (a.hd + 1) + ATTN_CHUNK * a.hd + ATTN_QG * a.hd + ATTN_QG * ATTN_CHUNK) * 4;
  const void* fn = bf ? (const void*)attn_partial_kernel<true> : (const void*)attn_partial_kernel<false>;
  static std::atomic<bool> cleared[2][MAX_DEVICES];
  hipError_t err = clear_dynamic_lds(fn, lds, cleared[bf ? 1 : 0]);
  if (err != hipSuccess) return err;
  if (bf)
    hipLaunchKernelGGL(attn_partial_kernel<true>, grid, dim3(256), lds, s, a, ring_layer, qb, qlo, R, e, nch, part);
  else
    hipLaunchKernelGGL(attn_partial_kernel<false>, grid, dim3(256), lds, s, a, ring_layer, qb, qlo, R, e, nch, part);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (bf) hipLaunchKernelGGL(attn_combine_kernel<true>, dim3(R * a.nq), dim3(a.hd), 0, s, a, part, R, nch, out, out_lo);
  else hipLaunchKernelGGL(attn_combine_kernel<false>, dim3(R * a.nq), dim3(a.hd), 0, s, a, part, R, nch, out, out_lo);
  return hipGetLastError();
}

hipError_t launch_block_attention_batch(int bf, const AttnShape& a, const AttnSeqs& seqs, const float* qkv,
                                        const void* qnorm, const void* knorm, const float2* rope, void* ring0,
                                        size_t ring_seq_bytes, int R, void* qb, void* qlo, float* part, void* out,
                                        void* out_lo, hipStream_t s) {
  if (seqs.n < 1 || seqs.n > ATTN_MAX_SEQS || R < 1) return hipErrorInvalidValue;
  const size_t elt = bf ? 2 : 4;
  if (!use_mfma(bf, a)) {  // f32 shapes: one launch pair per sequence
    const size_t ldq = (size_t)(a.nq + 2 * a.nkv) * a.hd, op_row = (size_t)a.nq * a.hd * elt;
    for (int q = 0; q < seqs.n; ++q) {
      const size_t r0 = (size_t)q * R;
      const hipError_t err = launch_block_attention(
          bf, a, qkv + r0 * ldq, qnorm, knorm, rope ? rope + r0 * (a.hd / 2) : nullptr,
          (unsigned char*)ring0 + (size_t)q * ring_seq_bytes, R, 0, seqs.e[q], (unsigned char*)qb + r0 * op_row,
          qlo ? (unsigned char*)qlo + r0 * op_row : nullptr, part, (unsigned char*)out + r0 * op_row,
          out_lo ? (unsigned char*)out_lo + r0 * op_row : nullptr, s);
      if (err != hipSuccess) return err;
    }
    return hipSuccess;
  }
  if (!rope || ring_seq_bytes % 2) return hipErrorInvalidValue;
  int nch_max = 1;
  for (int q = 0; q < seqs.n; ++q) {
    const int nch = attn_nchunks(a, R, seqs.e[q]);
    if (nch > COMBINE_MAX_CHUNKS || seqs.e[q] < 1) return hipErrorInvalidValue;
    nch_max = nch > nch_max ? nch : nch_max;
  }
  const size_t part_seq = (size_t)a.nkv * nch_max * R * (a.nq / a.nkv) * PART_STRIDE(a.hd);
  const int nqt = (R * (a.nq / a.nkv) + 15) / 16;
  const int zq = (nqt + 3) / 4, tpw = (nqt + zq - 1) / zq;
  const dim3 grid(nch_max, a.nkv, zq * seqs.n);
  auto* fn = a.hd == 128 ? attn_mfma_batch_kernel<128, 4> : attn_mfma_batch_kernel<64, 4>;
  hipLaunchKernelGGL(fn, grid, dim3(256), 0, s, a, seqs, (uint16_t*)ring0, ring_seq_bytes / 2, qkv,
                     (const uint16_t*)qnorm, (const uint16_t*)knorm, rope, R, zq, tpw, part_seq, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(attn_combine_batch_kernel<true>, dim3(seqs.n * R * a.nq), dim3(a.hd), 0, s, a, seqs, part,
                     part_seq, R, out, out_lo);
  return hipGetLastError();
}

size_t attention_partial_floats_batch(const AttnShape& a, int R, int n_seq) {
  return (size_t)n_seq * attention_partial_floats(a, R);
}

hipError_t launch_cache_read(int bf, const AttnShape& a, const void* ring_layer, int64_t lo, int n, void* kout,
                             void* vout, hipStream_t s, int deint) {
  if (n <= 0) return hipSuccess;
  const size_t total = (size_t)a.nkv * n * a.hd;
  const int grid = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  if (bf)
    hipLaunchKernelGGL(cache_read_kernel<true>, dim3(grid), dim3(256), 0, s, a, ring_layer, lo, n, kout, vout, deint);
  else
    hipLaunchKernelGGL(cache_read_kernel<false>, dim3(grid), dim3(256), 0, s, a, ring_layer, lo, n, kout, vout, deint);
  return hipGetLastError();
}

}  // namespace dflash
