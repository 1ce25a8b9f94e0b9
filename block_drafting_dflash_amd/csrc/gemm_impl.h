// Skinny weight-streaming GEMM for the DFlash block forward: Y[r, n] = sum_k X[r, k] W[n, k]
// with at most 48 activation rows against weight matrices of up to 202048 rows.
//
// The block forward multiplies B+1 (or B) rows by every drafter weight once, so each
// weight byte is read exactly once per pass and the kernel is bound by HBM bandwidth. The
// contraction uses MFMA tiles (A = 16 activation rows, B = 16 weight rows, 32 k per
// bf16 instruction, 4 k per f32 instruction); weights go straight from global memory into
// the B operand with one 16-byte load per lane per step.
//
// Work decomposition: a work-group owns T output tiles of 16 columns (32 weight rows for
// the SwiGLU gate/up pair) and all of K for each; its waves split K evenly and sum their
// partial tiles through LDS in a fixed order, so an output's reduction order never depends
// on the row count (a row gives bit-identical results in a 4-row or a 16-row call). The
// (tile, chunk) sequence of a work-group is a compile-time constant and fully unrolled:
// every wave keeps the next chunk of weights in flight while it multiplies the current
// one, and the compiler's wait counts stay exact (a loop back-edge would make it drain
// the prefetch at every iteration). Activations come straight from global memory
// (L2-resident) or are formed once per wave in registers, optionally through the RMSNorm
// prologue y = x * rsqrt(mean(x^2) + eps) * g. With bf16 weights an f32 activation enters
// as a bf16 pair hi + lo and costs two MFMA products (SPLIT); activations given in bf16
// (the residual slab, verify rows) take one. Epilogues: store,
// residual add, SwiGLU, and the fused lm_head argmax, which keeps each lane's best
// (value, index) key over the work-group's tiles, reduces a row's 16 lanes with wavefront
// shuffles once at the end and stores one key per row and work-group; a finalize kernel
// reduces those (no fence or atomic in the streaming kernel: a device-scope fence per
// work-group cost a third of the lm_head's time).
#pragma once
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
// 4-bit weights: bf16 activation steps of 32 k; one 16-byte lane load of codes covers four
// steps (a 128-k block), see launch_pack_q4.
template <> struct WTr<WT_Q4> {
  static constexpr int KSTEP = 32;
  static constexpr int EPL = 8;
  static constexpr int ELT = 2;
  static constexpr bool BF = true;
};

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// Eight reordered 4-bit codes -> the bf16 values 128 + q in MFMA operand order (element
// 2e in the low half of word e): bf16 0x4300 is 128 and its 7 mantissa bits count units.
// m = 0x000F000F and c = 0x43004300 come in as register values the compiler cannot see
// through (the kernel hides them once): with literal constants it emits an AND and an OR
// per word (gfx9 three-operand encodings take no literal), with registers one AND-OR.
__device__ __forceinline__ u32x4_t q4_expand(uint32_t w, uint32_t m, uint32_t c) {
  u32x4_t f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = ((w >> (4 * e)) & m) | c;
  return f;
}

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

// The segment holding output column col: its weight and scale blocks and the column's tile
// within it. Every segment entry is read in one batch of scalar loads and picked by
// selects, so the first weight address waits for one kernel-argument fetch, not a chain.
struct SegSel {
  const unsigned char* w;
  const unsigned char* sc;
  int tj;
};
__device__ __forceinline__ SegSel select_seg(const GemmParams& p, int col) {
  const unsigned char* w = (const unsigned char*)p.seg[0].w;
  const unsigned char* sc = (const unsigned char*)p.seg[0].scales;
  int c0 = p.seg[0].col0;
#pragma unroll
  for (int i = 1; i < GEMM_MAXSEG; ++i) {
    const bool take = i < p.nseg && col >= p.seg[i].col0;
    w = take ? (const unsigned char*)p.seg[i].w : w;
    sc = take ? (const unsigned char*)p.seg[i].scales : sc;
    c0 = take ? p.seg[i].col0 : c0;
  }
  return SegSel{w, sc, (col - c0) >> 4};
}

// Minimum resident waves per SIMD (the second launch-bounds argument), sized so that the
// live registers (weights in flight, operand fragments, accumulators) never spill:
// single-chunk single-tile launches of one row tile run hundreds of 8-wave work-groups
// and get two per CU (<= 128 VGPRs); launches with more row tiles, normed operands, or
// hi/lo operand pairs across several chunks or weight blocks take the full budget and
// fewer, larger work-groups; the multi-tile argmax launches three.
template <int WT, int RT, int NB, int XSRC, int T, int NCH, bool SPLIT> constexpr int gemm_min_waves_per_simd() {
  // 4-bit heads over a few hi/lo rows, four tiles per work-group, read their lo fragments
  // from LDS at each step (gemm_kernel), which brings them to four waves per SIMD: two
  // 8-wave work-groups per CU
  if (WT == WT_Q4 && SPLIT && XSRC == XSRC_LDS && RT == 1 && NCH == 1 && T == 4) return 4;
  if (RT > 1 || XSRC == XSRC_NORM) return 2;
  if (T > 1) return 3;
  if (SPLIT && (NCH > 1 || NB > 1)) return 2;
  return NCH == 1 ? 4 : 2;
}

// Weight chunks a wave issues before its first product. The layer GEMMs with streamed
// operands put every chunk of the launch in flight at once (a launch is one round trip, not
// a pipeline) as far as the registers beside the operands allow: streamed operands staged
// through LDS hold one chunk of compact rows plus the fragments read back; unstaged
// streamed operands two chunks of fragments; staged (LDS-source) operands every chunk; and
// about 48 registers go to accumulators, addresses and sums; normed operands of two row
// tiles hold their raw rows while the pairs are formed. Normed operands of one row tile
// issue one chunk, form their pairs, then issue the rest: a wave stalls while the memory
// pipeline refuses its loads, and with every chunk issued first the norm prologue waited
// behind that stall (gate/up 13.2 -> 12.5 us, QKV 8.6 -> 8.4 us at 5 rows; two row tiles,
// whose prologue is longer, measured slower that way). Streamed operands (folded bf16 and
// 4-bit) also keep one chunk ahead, so that staging a chunk's operand rows does not wait
// behind the whole stream (bf16 O 7.2 -> 6.9 us, down 8.9 -> 8.4 us at 5 rows). The
// vocabulary argmax keeps shallow look-ahead: it runs thousands of work-groups, several per
// CU, which keep the stream busy between them (three chunks for 4-bit single-plane rows,
// whose chunks carry a quarter of the bytes). f32 weights (the exact-arithmetic shapes)
// keep one chunk ahead.
template <int WT, int RT, int NB, int EPI, int XSRC_IN, int T, int NCH, int CH, bool SPLIT>
constexpr int gemm_chunks_ahead() {
  constexpr int XSRC = xsrc_base(XSRC_IN);
  constexpr bool Q4 = WT == WT_Q4, BF = WT != WT_F32;
  constexpr bool fold = WT == WT_BF16 && XSRC == XSRC_GLOBAL;  // RT counts 8-row groups
  constexpr int nit = T * NCH;
  // 4-bit argmax over hi/lo pairs: the operand pairs and group sums leave no room (measured)
  constexpr int argmax_ahead = Q4 && !SPLIT ? 3 : 1;
  if (EPI == EPI_ARGMAX || !BF) return nit < argmax_ahead ? nit : argmax_ahead;
  if ((XSRC == XSRC_NORM && RT == 1) || XSRC == XSRC_GLOBAL) return 1;
  constexpr int budget = 512 / gemm_min_waves_per_simd<WT, RT, NB, XSRC, T, NCH, SPLIT>();
  constexpr int planes = SPLIT ? 2 : 1;
  constexpr int frag = RT * CH * 4 * planes;  // operand VGPRs of one chunk's fragments
  constexpr int raw = XSRC == XSRC_NORM ? RT * CH * 4 * 2 + CH * 4 : 0;
  constexpr int gupi = 64 / (CH * 32 * 2 / 16);  // staged rows per load instruction
  constexpr int staged = planes * (((fold ? 8 : 16) * RT + gupi - 1) / gupi) * 4 + 32;
  // normed rows of a later chunk are loaded while the earlier chunks' pairs are held, unless
  // the raw rows of the wave's whole k range are staged through LDS first (then they are
  // dead before the pairs are formed)
  constexpr bool stg_n = XSRC == XSRC_NORM && RT <= 2 && NCH * CH * 32 == 256;
  constexpr int raw_stg = (GEMM_NORM_STAGED_ROWS + 1) * 4;
  // two-phase staging (XSRC_NORMP) loads its later rows, eight at a time, beside the first
  // row tile's pairs
  constexpr int raw_p2 = xsrc_two_phase(XSRC_IN) ? 8 * 4 : 0;
  constexpr int opnd = XSRC == XSRC_GLOBAL ? ((fold ? 8 : 16) * RT <= 32 ? staged : 2 * frag)
                       : XSRC == XSRC_LDS  ? NCH * frag
                       : stg_n             ? (raw_stg > NCH * frag + raw_p2 ? raw_stg : NCH * frag + raw_p2)
                       : NCH == 1          ? (raw > frag ? raw : frag)
                                           : NCH * frag + raw;
  constexpr int wreg = Q4 ? NB * (CH / 4) * 6 : NB * (fold ? CH / 2 : CH) * 4;
  constexpr int fit = (budget - opnd - 48) / wreg;
  // a launch with more chunks than fit streams the rest: one more chunk buffer is live
  return fit >= nit ? nit : (fit - 1 < 1 ? 1 : (fit - 1 > 8 ? 8 : fit - 1));
}

// T tiles per work-group, NCH chunks of CH steps per wave per tile, all compile-time.
template <int WT, int RT, int NB, int EPI, int XSRC_IN, int T, int NCH, int CH, bool SPLIT>
__global__ __launch_bounds__(512, (gemm_min_waves_per_simd<WT, RT, NB, xsrc_base(XSRC_IN), T, NCH, SPLIT>())) void
gemm_kernel(const GemmParams p) {
  constexpr int XSRC = xsrc_base(XSRC_IN);
  using Tr = WTr<WT>;
  constexpr bool BF = Tr::BF;
  static_assert(!SPLIT || BF, "hi/lo operand pairs feed bf16 MFMA only");
  constexpr bool Q4 = WT == WT_Q4;
  constexpr int CB = Q4 ? CH / 4 : 1;  // 128-k code blocks per chunk
  static_assert(!Q4 || CH % 4 == 0, "a q4 chunk is whole code blocks");
  const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
  // q4_expand's mask (a scalar register) and bf16 128 pair (a vector register), opaque
  uint32_t q4m = 0x000F000Fu, q4c = 0x43004300u;
  if constexpr (Q4) {
    asm volatile("" : "+s"(q4m));
    asm volatile("" : "+v"(q4c));
  }
  static_assert(!(BF && XSRC == XSRC_NORM && !SPLIT), "a normed bf16 operand is always a hi/lo pair");
  constexpr int SR = SPLIT ? RT : 1;  // row tiles of lo fragments held (1 = unused)
  constexpr int NIT = T * NCH;
  constexpr int NRED = T > 1 ? 2 : 1;  // reduction buffers (double-buffered across tiles)
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int nw = p.waves;
  const int K = p.K, R = p.R;
  const int kw = K / nw;  // k owned by this wave in every tile (= NCH * CH * KSTEP)

  const GemmLds lds = gemm_lds_layout(WT, XSRC_IN, SPLIT ? 1 : 0, R, nw, NB, K, T);
  float* red = (float*)smem;  // [NRED][nw][RT][NB][64 lanes][4]
  // XSRC_NORM: per wave, the sum of squares of each row over the wave's k range [nw][RT*16]
  float* ssq = (float*)(smem + lds.ssq_off);
  // this wave's operand staging slot (see gemm_lds_layout)
  unsigned char* xs = smem + lds.xs_off + (size_t)w * lds.xs_wave;
  // staged operands: streamed rows (STG_G) of one chunk, [plane][row][CH * KSTEP] bf16; or the
  // normed raw rows (STG_N) of the wave's whole k range, [row][CH * KSTEP] f32 then the gains
  // FOLD (bf16 weights, streamed operands): a work-group owns 8 output columns, half h of
  // a 16-row weight block, and RT counts groups of 8 operand rows. One MFMA takes two k
  // steps s, s+1: lanes li < 8 supply weight rows 8h + li of step s and operand rows of step
  // s, lanes li >= 8 the same rows of step s+1, so the product's top-left 8x8 block is step
  // s, its bottom-right block step s+1 and the rest is discarded; the finishing wave adds
  // the two blocks (lane l and lane l + 40).
  constexpr bool FOLD = WT == WT_BF16 && XSRC == XSRC_GLOBAL;
  constexpr int RROWS = FOLD ? 8 : 16;      // operand rows per MFMA row group
  constexpr int WST = FOLD ? CH / 2 : CH;   // weight loads (and products) per chunk
  static_assert(!FOLD || CH % 2 == 0, "a folded chunk pairs its k steps");
  constexpr bool STG_G = BF && XSRC == XSRC_GLOBAL && RROWS * RT <= 32;
  constexpr bool STG_N = BF && XSRC == XSRC_NORM && RT <= 2 && NCH * CH * Tr::KSTEP == 256;
  // two-phase staging (XSRC_NORMP): rows 0-15, then rows 16.. over the same slot
  constexpr bool STG_N2 = xsrc_two_phase(XSRC_IN);
  static_assert(!STG_N2 || (STG_N && RT == 2), "two-phase staging: two row tiles of staged raw rows");
  constexpr int STG_N_ROWS = RT == 1 || STG_N2 ? 16 : GEMM_NORM_STAGED_ROWS;  // rows one staging holds
  constexpr bool STG_L = BF && XSRC == XSRC_LDS && RT == 1 && NCH == 1;
  // 4-bit weights over hi/lo rows staged once per work-group, four tiles per work-group: each
  // step's lo fragment is read from the staged rows where it is used instead of being held
  // with the hi fragments (vocabulary argmax at 4 and 5 rows 65 -> 58 us; at 8 and 16 rows
  // it measured slower, and those launches keep eight tiles and held fragments)
  constexpr bool LO_LDS = Q4 && SPLIT && STG_L && T == 4;
  constexpr int SP = SPLIT ? 2 : 1;          // operand planes
  constexpr int LK = CH * Tr::KSTEP;          // k of one chunk
  constexpr int GU = LK * 2 / 16;             // lanes per staged bf16 row (32 or 16)
  constexpr int GUPI = 64 / GU;               // staged rows per load instruction
  constexpr int GIMAX = (RROWS * RT + GUPI - 1) / GUPI;
  static_assert(!STG_N || NCH * LK * 4 == 1024, "a normed row of the wave's k range is one wave load");

  // tiles past the end repeat the last one: harmless for the argmax (max is idempotent);
  // the other epilogues run with T dividing the tile count
  const int ntl = FOLD ? 2 * p.ntiles : p.ntiles;  // tiles of 8 (FOLD) or 16 columns
  auto tile_of = [&](int t) {
    const int j = (int)blockIdx.x * T + t;
    return j < ntl ? j : ntl - 1;
  };

  // weights of (tile, chunk) it: the fragment-major blocks of every segment
  auto load_w = [&](u32x4_t (&wb)[NB][CH], u32x2_t (&sb)[NB][CB], int it) {
    const int j = tile_of(it / NCH), c = it % NCH;
    const int j16 = FOLD ? j >> 1 : j;  // the 16-row weight block
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      SegSel sel;
      if constexpr (EPI == EPI_ARGMAX) {  // one matrix (checked at launch)
        sel = SegSel{(const unsigned char*)p.seg[0].w, (const unsigned char*)p.seg[0].scales, j};
      } else if constexpr (NB == 1) {
        sel = select_seg(p, 16 * j16);
      } else {
        sel = SegSel{(const unsigned char*)p.seg[nb].w, (const unsigned char*)p.seg[nb].scales, j16};
      }
      const int tj = sel.tj;
      if constexpr (Q4) {
        // one kilobyte of codes and 128 bytes of (scale, bias) per (16-row tile, 128 k)
        const size_t kblocks = (size_t)K / 128;
        const size_t blk0 = ((size_t)w * kw + (size_t)c * CH * Tr::KSTEP) / 128;
        const size_t bo = (size_t)tj * kblocks + blk0;
        const unsigned char* wr = sel.w + bo * 1024 + lane * 16;
        const unsigned char* sr = sel.sc + bo * 128 + li * 8;
#pragma unroll
        for (int b = 0; b < CB; ++b) {
          wb[nb][b] = __builtin_nontemporal_load((const u32x4_t*)(wr + (size_t)b * 1024));
          sb[nb][b] = __builtin_nontemporal_load((const u32x2_t*)(sr + (size_t)b * 128));
        }
      } else if constexpr (FOLD) {
        // half h of the 16-row blocks of steps 2*st2 + li/8: 8 rows x 8 k per 128 bytes
        const size_t kblocks = (size_t)K / Tr::KSTEP;
        const size_t blk0 = (size_t)w * (kw / Tr::KSTEP) + (size_t)c * CH + (li >> 3);
        const int fl = lg * 16 + 8 * (j & 1) + (li & 7);  // the lane of that row in the block
        const unsigned char* wr = sel.w + ((size_t)tj * kblocks + blk0) * 1024 + fl * 16;
#pragma unroll
        for (int st2 = 0; st2 < WST; ++st2)
          wb[nb][st2] = __builtin_nontemporal_load((const u32x4_t*)(wr + (size_t)st2 * 2048));
      } else {
        // fragment-major weights: one contiguous kilobyte per (16-row tile, KSTEP) block
        const size_t kblocks = (size_t)K / Tr::KSTEP;
        const size_t blk0 = (size_t)w * (kw / Tr::KSTEP) + (size_t)c * CH;
        const unsigned char* wr = sel.w + ((size_t)tj * kblocks + blk0) * 1024 + lane * 16;
#pragma unroll
        for (int st = 0; st < CH; ++st)
          wb[nb][st] = __builtin_nontemporal_load((const u32x4_t*)(wr + (size_t)st * 1024));
      }
    }
  };

  // Operand rows past R load row R - 1 instead of branching around the load (a divergent
  // branch makes the compiler wait for every load in flight): MFMA output row r depends on
  // operand row r alone, and rows past R are never stored.
  auto xrow = [&](int rt) { return min(rt * 16 + li, R - 1); };

  // streamed operand fragments of chunk it (hi and, for pairs, lo planes)
  auto load_x = [&](u32x4_t (&xb)[RT][CH], u32x4_t (&xlb)[SR][CH], int it) {
    const int c = it % NCH;
    const size_t kb = ((size_t)w * kw + (size_t)c * CH * Tr::KSTEP + lg * Tr::EPL) * Tr::ELT;
    if constexpr (XSRC == XSRC_GLOBAL) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const size_t xo = (size_t)xrow(rt) * p.ldx * Tr::ELT + kb;
        const unsigned char* xr = (const unsigned char*)p.x + xo;
#pragma unroll
        for (int st = 0; st < CH; ++st) xb[rt][st] = *(const u32x4_t*)(xr + (size_t)st * Tr::KSTEP * Tr::ELT);
        if constexpr (SPLIT) {
          const unsigned char* xl = (const unsigned char*)p.xlo + xo;
#pragma unroll
          for (int st = 0; st < CH; ++st) xlb[rt][st] = *(const u32x4_t*)(xl + (size_t)st * Tr::KSTEP * Tr::ELT);
        }
      }
    }
  };

  // STG_G: the R rows of each plane for chunk it, GU lanes of 16 bytes per row, rows past
  // R-1 repeating row R-1 in the last instruction; then stored to the staging slot
  // XCD chunks of operand rows in flight: with one row group, every chunk of a short launch
  // up front and a ring of three ahead for longer ones (one chunk ahead made each chunk's
  // staging wait a round trip); more row groups have no registers to spare
  constexpr int XCD = STG_G && RT == 1 ? (NIT < 3 ? NIT : 3) : 1;
  u32x4_t xc[XCD][STG_G ? SP : 1][STG_G ? GIMAX : 1];
  const int gipp = (R + GUPI - 1) / GUPI;  // load instructions per plane
  auto load_xc = [&](int it) {
    if constexpr (STG_G) {
      const size_t k0 = (size_t)w * kw + (size_t)(it % NCH) * LK;
      const int piece = lane % GU;
#pragma unroll
      for (int pl = 0; pl < SP; ++pl)
#pragma unroll
        for (int i = 0; i < GIMAX; ++i)
          if (i < gipp) {
            const int r = min(i * GUPI + lane / GU, R - 1);
            const unsigned char* src = (const unsigned char*)(pl ? p.xlo : p.x);
            xc[it % XCD][pl][i] = *(const u32x4_t*)(src + ((size_t)r * p.ldx + k0) * 2 + piece * 16);
          }
    }
  };
  auto stage_xc = [&](int it) {
    if constexpr (STG_G) {
      const int piece = lane % GU;
#pragma unroll
      for (int pl = 0; pl < SP; ++pl)
#pragma unroll
        for (int i = 0; i < GIMAX; ++i)
          if (i < gipp) {
            const int r = min(i * GUPI + lane / GU, R - 1);
            *(u32x4_t*)(xs + ((size_t)pl * R + r) * lds.row_bytes + piece * 16) = xc[it % XCD][pl][i];
          }
    }
  };
  // MFMA fragment (row tile rt, step st) of plane pl from the staged rows
  auto frag_xs = [&](int rt, int st, int pl) {
    const int r = min(rt * 16 + li, R - 1);
    return *(const u32x4_t*)(xs + ((size_t)pl * R + r) * lds.row_bytes + (st * Tr::KSTEP + lg * Tr::EPL) * 2);
  };
  // FOLD: row group rt, step pair st2 (rows rt*8 + li%8 of step 2*st2 + li/8)
  auto frag_xs_fold = [&](int rt, int st2, int pl) {
    const int r = min(rt * 8 + (li & 7), R - 1);
    const int st = 2 * st2 + (li >> 3);
    return *(const u32x4_t*)(xs + ((size_t)pl * R + r) * lds.row_bytes + (st * Tr::KSTEP + lg * Tr::EPL) * 2);
  };

  f32x4_t acc[RT][NB];
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rt][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // operand fragments of this wave's K slice, built once (staged sources only)
  constexpr int XR = XSRC == XSRC_GLOBAL ? 1 : NCH;
  u32x4_t xr[XR][RT][CH];
  u32x4_t xrl[SPLIT && !LO_LDS ? XR : 1][SR][LO_LDS ? 1 : CH];  // lo halves of staged pairs
  // q4: per 64-k group, the sum of the operand values of each accumulator row (staged
  // sources: built once from the staged fragments)
  constexpr int NG = (Q4 && XSRC != XSRC_GLOBAL) ? XR * CH / 2 : 1;
  f32x4_t xg[NG][RT];

  auto compute = [&](u32x4_t (&wb)[NB][CH], u32x2_t (&sb)[NB][CB], u32x4_t (&xb)[RT][CH], u32x4_t (&xlb)[SR][CH],
                     int it) {
    const int c = it % NCH;
    auto xfrag = [&](int rt, int st, u32x4_t& xf, u32x4_t& xl) {
      if constexpr (STG_G) {
        xf = frag_xs(rt, st, 0);
        if constexpr (SPLIT) xl = frag_xs(rt, st, 1);
      } else if constexpr (XSRC == XSRC_GLOBAL) {
        xf = xb[rt][st];
        if constexpr (SPLIT) xl = xlb[rt][st];
      } else {
        xf = xr[XSRC == XSRC_GLOBAL ? 0 : c][rt][st];
        if constexpr (LO_LDS) xl = frag_xs(rt, st, 1);
        else if constexpr (SPLIT) xl = xrl[XSRC == XSRC_GLOBAL ? 0 : c][rt][st];
      }
    };
    if constexpr (Q4) {
      // y += s * sum(x (128 + q)) + (b - 128 s) * sum(x) per 64-k group: the codes enter the
      // MFMA as exact bf16 integers and the 128 offset cancels against the operand sums
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        float sc[NB][2], cc[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const uint32_t v = sb[nb][b][g2];
            sc[nb][g2] = __uint_as_float(v << 16);
            cc[nb][g2] = __uint_as_float(v & 0xffff0000u) - 128.0f * sc[nb][g2];
          }
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          f32x4_t ag[RT][NB], ax[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            ax[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) ag[rt][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * g2 + tt, st = 4 * b + t;
            u32x4_t fr[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) fr[nb] = q4_expand(wb[nb][b][t], q4m, q4c);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              u32x4_t xf, xl;
              xfrag(rt, st, xf, xl);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                ag[rt][nb] = mfma_bf16(xf, fr[nb], ag[rt][nb]);
                if constexpr (SPLIT) ag[rt][nb] = mfma_bf16(xl, fr[nb], ag[rt][nb]);
              }
              if constexpr (XSRC == XSRC_GLOBAL) {  // streamed operands: their group sums here
                ax[rt] = mfma_bf16(xf, ones, ax[rt]);
                if constexpr (SPLIT) ax[rt] = mfma_bf16(xl, ones, ax[rt]);
              }
            }
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int gi = (c * CH + 4 * b) / 2 + g2;  // group within this wave's k range
            f32x4_t xs;
            if constexpr (XSRC == XSRC_GLOBAL) xs = ax[rt];
            else xs = xg[XSRC == XSRC_GLOBAL ? 0 : gi][rt];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                acc[rt][nb][q] = fmaf(sc[nb][g2], ag[rt][nb][q], acc[rt][nb][q]);
                acc[rt][nb][q] = fmaf(cc[nb][g2], xs[q], acc[rt][nb][q]);
              }
              // the accumulator's only reader is the final reduction: without this empty
              // read-write the compiler sinks every group's update there and keeps all the
              // group partials, scales and sums alive across the stream
              asm volatile("" : "+v"(acc[rt][nb]));
            }
          }
        }
      }
      return;
    }
    if constexpr (FOLD) {
#pragma unroll
      for (int st2 = 0; st2 < WST; ++st2) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const u32x4_t xf = frag_xs_fold(rt, st2, 0);
          u32x4_t xl = xf;
          if constexpr (SPLIT) xl = frag_xs_fold(rt, st2, 1);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            acc[rt][nb] = mfma_bf16(xf, wb[nb][st2], acc[rt][nb]);
            if constexpr (SPLIT) acc[rt][nb] = mfma_bf16(xl, wb[nb][st2], acc[rt][nb]);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int st = 0; st < CH; ++st) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        u32x4_t xf, xl;
        xfrag(rt, st, xf, xl);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[rt][nb] = step_mfma<WT>(xf, wb[nb][st], acc[rt][nb]);
          if constexpr (SPLIT) acc[rt][nb] = step_mfma<WT>(xl, wb[nb][st], acc[rt][nb]);
        }
      }
    }
  };

  // EPI_RESID: the residual values of the first row tile this wave finishes (row tile w:
  // all of them when the work-group has at least RT waves), fetched with the operands so
  // that the epilogue only stores; every output is read and written by one lane
  static_assert(EPI != EPI_RESID || T == 1, "residual launches own one tile per work-group");
  float yres[4] = {0.f, 0.f, 0.f, 0.f};
  float zg = 0.f;  // the gain of this lane's output column for the z rows
  auto load_resid = [&]() {
    if constexpr (EPI == EPI_RESID) {
      const int col = FOLD ? 8 * tile_of(0) + (li & 7) : 16 * tile_of(0) + li;
      if (w < RT) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = min(w * RROWS + 4 * lg + q, R - 1);
          yres[q] = ((const float*)p.y)[(size_t)r * p.ldy + col];
        }
      }
      if (p.z) {
        if constexpr (BF) zg = bf2f(((const uint16_t*)p.zgain)[col]);
        else zg = ((const float*)p.zgain)[col];
      }
    }
  };

  auto finalize = [&](int t) {
    const int j = tile_of(t);
    float* rb = red + (size_t)(t % NRED) * nw * RT * NB * 256;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        *(f32x4_t*)&rb[((size_t)((w * RT + rt) * NB + nb) * 64 + lane) * 4] = acc[rt][nb];
        acc[rt][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    __syncthreads();
    // wave w finishes row tiles w, w+nw, ... (the argmax launch guarantees nw >= RT)
    for (int rt = w; rt < RT; rt += nw) {
      f32x4_t v[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        v[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int ww = 0; ww < nw; ++ww) v[nb] += *(const f32x4_t*)&rb[((size_t)((ww * RT + rt) * NB + nb) * 64 + lane) * 4];
        if constexpr (FOLD) {  // the odd steps: lane l + 40 holds rows 4lg + 8 + q, column li + 8
          f32x4_t v2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
          for (int ww = 0; ww < nw; ++ww)
            v2 += *(const f32x4_t*)&rb[((size_t)((ww * RT + rt) * NB + nb) * 64 + ((lane + 40) & 63)) * 4];
          v[nb] += v2;
        }
      }
      if constexpr (XSRC == XSRC_NORM) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rt * 16 + 4 * lg + q;
          float tot = 0.f;
          for (int ww = 0; ww < nw; ++ww) tot += ssq[ww * RT * 16 + r];
          const float rs = rsqrtf(tot / (float)K + p.eps);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) v[nb][q] *= rs;
        }
      }
      const int col = FOLD ? 8 * j + li : 16 * j + li;
      if constexpr (EPI == EPI_ARGMAX) {
        // each lane keeps the best key of its own columns over the tiles; the 16 columns of
        // a row are reduced once, after the last tile (max is exact and order-free). With
        // p.y the f32 logits are stored as well (a DSpark block's rows, which its Markov
        // chain scores)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rt * 16 + 4 * lg + q;
          const unsigned long long key = (r < R) ? argmax_key(v[0][q], col) : 0ull;
          best[q] = key > best[q] ? key : best[q];
          if (p.y && r < R) ((float*)p.y)[(size_t)r * p.ldy + col] = v[0][q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rt * RROWS + 4 * lg + q;
          if (r >= R || (FOLD && (li >= 8 || lg >= 2))) continue;
          const size_t o = (size_t)r * p.ldy + col;
          if constexpr (EPI == EPI_STORE) {
            ((float*)p.y)[o] = v[0][q];
          } else if constexpr (EPI == EPI_RESID) {
            const float nv = (rt == w ? yres[q] : ((const float*)p.y)[o]) + v[0][q];
            ((float*)p.y)[o] = nv;
            if (p.y2) {  // a target's captured residual stream
              const size_t o2 = (size_t)r * p.ldy2 + col;
              if (p.y2_bf16) ((uint16_t*)p.y2)[o2] = f2bf(nv);
              else ((float*)p.y2)[o2] = nv;
            }
            if (p.z) {  // gained rows for the vocabulary argmax (every row, or runs of zper
                        // with the first row of each left out)
              const int ar = p.zrow0 + r, run = p.zper ? ar / p.zper : 0, i = ar - run * p.zper;
              if (!p.zper || i > 0)
                op_st<SPLIT>(p.z, p.zlo, (int64_t)(p.zper ? run * (p.zper - 1) + i - 1 : ar) * p.ldz + col, nv * zg);
            }
          } else if constexpr (EPI == EPI_SWIGLU) {
            const float g = v[0][q], u = v[NB - 1][q];
            op_st<SPLIT>(p.y, p.ylo, o, g / (1.0f + expf(-g)) * u);
          }
        }
      }
    }
    if constexpr (NRED == 1) __syncthreads();
  };

  // ---- issue order: operands, the weight stream, then operand arithmetic ---------------
  // The memory counter retires loads in issue order, so a value can be used only once
  // every load issued before it has arrived. The small L2-resident operands therefore go
  // first and the weights right behind them, before any arithmetic: the normed operands
  // are ready when their own loads land, and every weight chunk the register budget holds
  // (all of them for the layer GEMMs) is in flight from the start.
  constexpr int AHEAD = gemm_chunks_ahead<WT, RT, NB, EPI, XSRC_IN, T, NCH, CH, SPLIT>();
  constexpr int PDW = AHEAD + 1;
  u32x4_t wbuf[PDW][NB][CH];
  u32x2_t sbuf[PDW][NB][CB];
  u32x4_t xbuf[2][RT][CH];  // streamed fragments (not STG_G)
  u32x4_t xlbuf[2][SR][CH];

  // normed operands: raw f32 rows and gains. A single-chunk launch loads them ahead of the
  // weights (NORM_FIRST). With more chunks, each value is loaded behind the weights and
  // formed at once, under a row guard: without the branch the scheduler hoists the loads of
  // every chunk and holds them beside the formed pairs.
  constexpr int XRAW = BF ? 2 : 1;  // 16-byte f32 loads per (row tile, step)
  constexpr bool NORM_FIRST = XSRC == XSRC_NORM && XR == 1;
  f32x4_t xa[STG_N ? 1 : RT][CH][XRAW];
  u32x4_t ga[CH];
  // STG_N: raw row i of the wave's k range in load i (64 lanes x 4 f32), the gains in the last
  // (one row tile: lanes 0-31 the gains of rows below r2, lanes 32-63 those of rows r2 and up)
  u32x4_t xn[STG_N ? STG_N_ROWS + 1 : 1];
  constexpr bool GAIN2 = xsrc_gain2(XSRC_IN);
  static_assert(!GAIN2 || (STG_N && (RT == 1 || STG_N2)), "two gain rows: staged raw rows");
  // LDS offset of the gain row of this lane's operand row in row tile rt (row rt*16+li,
  // clamped to the real rows)
  auto g2off = [&](int rt) { return GAIN2 && min(rt * 16 + li, R - 1) >= p.r2 ? 512 : 0; };
  auto kof = [&](int c, int st) { return w * kw + (c * CH + st) * Tr::KSTEP + lg * Tr::EPL; };
  auto raw_ld = [&](int c, int rt, int st, int h) {
    return *(const f32x4_t*)((const float*)p.x + (size_t)xrow(rt) * p.ldx + kof(c, st) + 4 * h);
  };
  auto gain_ld = [&](int c, int st) {
    if constexpr (BF) return *(const u32x4_t*)((const uint16_t*)p.gain + kof(c, st));
    else return *(const u32x4_t*)((const float*)p.gain + kof(c, st));
  };
  // one normed operand fragment: sums of squares from the raw values, and x * g as a hi/lo
  // bf16 pair (bf16 weights) or f32
  auto form = [&](const f32x4_t a0, const f32x4_t a1, const u32x4_t gb, float& ss, u32x4_t& f, u32x4_t& fl) {
    if constexpr (BF) {
      const float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float g0 = __uint_as_float(gb[e2] << 16), g1 = __uint_as_float(gb[e2] & 0xffff0000u);
        uint32_t hp, lp;
        split2_bf16(v[2 * e2] * g0, v[2 * e2 + 1] * g1, hp, lp);
        f[e2] = hp;
        fl[e2] = lp;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss = fmaf(a0[e], a0[e], ss);
        f[e] = __float_as_uint(a0[e] * __uint_as_float(gb[e]));
      }
    }
  };
  if constexpr (STG_G) {
#pragma unroll
    for (int c = 0; c < XCD; ++c) load_xc(c);
  } else if constexpr (XSRC == XSRC_GLOBAL) {
    load_x(xbuf[0], xlbuf[0], 0);
  } else if constexpr (STG_N) {
    const size_t k0 = (size_t)w * kw;
#pragma unroll
    for (int i = 0; i < STG_N_ROWS; ++i)
      if (i < R) xn[i] = *(const u32x4_t*)((const float*)p.x + (size_t)i * p.ldx + k0 + lane * 4);
    xn[STG_N_ROWS] =
        *(const u32x4_t*)((const uint16_t*)(GAIN2 && lane >= 32 ? p.gain2 : p.gain) + k0 + (lane & 31) * 8);
  } else if constexpr (NORM_FIRST) {
#pragma unroll
    for (int st = 0; st < CH; ++st) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int h = 0; h < XRAW; ++h) xa[rt][st][h] = raw_ld(0, rt, st, h);
      ga[st] = gain_ld(0, st);
    }
  }
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) load_w(wbuf[i], sbuf[i], i);
  load_resid();
  if constexpr (STG_L) {
    // LDS-source rows (the argmax rows), behind the first weight chunk: the R real rows of
    // each plane over the wave's k range (512 bytes: 32 lanes, two rows per load) into the
    // wave's staging slot, then the MFMA fragments from there
    u32x4_t xc2[SP][8];
    const int npairs = (R + 1) / 2;
    const int half = lane >> 5, piece = lane & 31;
#pragma unroll
    for (int pl = 0; pl < SP; ++pl)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < npairs) {
          const int r = min(2 * i + half, R - 1);
          const unsigned char* src = (const unsigned char*)(pl ? p.xlo : p.x);
          xc2[pl][i] = *(const u32x4_t*)(src + ((size_t)r * p.ldx + (size_t)w * kw) * 2 + piece * 16);
        }
#pragma unroll
    for (int pl = 0; pl < SP; ++pl)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < npairs) {
          const int r = min(2 * i + half, R - 1);
          *(u32x4_t*)(xs + ((size_t)pl * R + r) * lds.row_bytes + piece * 16) = xc2[pl][i];
        }
#pragma unroll
    for (int st = 0; st < CH; ++st) {
      const int r = min(li, R - 1);
      const size_t o = (size_t)r * lds.row_bytes + (st * Tr::KSTEP + lg * Tr::EPL) * 2;
      xr[0][0][st] = *(const u32x4_t*)(xs + o);
      if constexpr (SPLIT && !LO_LDS) xrl[0][0][st] = *(const u32x4_t*)(xs + (size_t)R * lds.row_bytes + o);
    }
  } else if constexpr (XSRC == XSRC_LDS) {
    // LDS-source planes of more row tiles or chunks: every chunk into the operand
    // fragments, behind the first weight chunk and only for the real rows
#pragma unroll
    for (int c = 0; c < XR; ++c)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int st = 0; st < CH; ++st) {
          const int r = rt * 16 + li;
          const size_t xo = ((size_t)r * p.ldx + kof(c, st)) * Tr::ELT;
          u32x4_t v = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
          if (r < R) {
            v = *(const u32x4_t*)((const unsigned char*)p.x + xo);
            if constexpr (SPLIT) vl = *(const u32x4_t*)((const unsigned char*)p.xlo + xo);
          }
          xr[c][rt][st] = v;
          if constexpr (SPLIT) xrl[c][rt][st] = vl;
        }
  }

  if constexpr (XSRC == XSRC_NORM) {
    // RMSNorm operands: the row scale rsqrt(mean(x^2) + eps) is one number per row, so the
    // operand is x * g and the scale multiplies the finished dot products (finalize); the
    // sums of squares come from the same loads, per lane, then per wave, then across waves
    float ssl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) ssl[rt] = 0.f;
    // the gain row sits after the staged rows (after the first phase's 16 with two phases)
    const int grow = STG_N2 ? 16 : R;
    if constexpr (STG_N) {
#pragma unroll
      for (int i = 0; i < STG_N_ROWS; ++i)
        if (i < R) *(u32x4_t*)(xs + (size_t)i * lds.row_bytes + lane * 16) = xn[i];
      *(u32x4_t*)(xs + (size_t)grow * lds.row_bytes + (GAIN2 ? lane : lane & 31) * 16) = xn[STG_N_ROWS];
    }
    // lane (li, lg) of step st holds row rt*16+li, k = w*kw + st*KSTEP + lg*EPL .. + EPL
    auto form_at = [&](int c, int rt, int st) {
      u32x4_t f = {0u, 0u, 0u, 0u}, fl = {0u, 0u, 0u, 0u};
      if constexpr (STG_N) {
        const int kk = (c * CH + st) * Tr::KSTEP + lg * Tr::EPL;  // within the wave's k range
        // the slot holds rows 0.. (one phase), or the row tile's own rows (two phases)
        const int row = STG_N2 ? min(li, R - 1 - 16 * rt) : min(rt * 16 + li, R - 1);
        const unsigned char* xrw = xs + (size_t)row * lds.row_bytes + kk * 4;
        const u32x4_t gb = *(const u32x4_t*)(xs + (size_t)grow * lds.row_bytes + g2off(rt) + kk * 2);
        form(*(const f32x4_t*)xrw, *(const f32x4_t*)(xrw + 16), gb, ssl[rt], f, fl);
      } else if constexpr (NORM_FIRST) {
        form(xa[rt][st][0], xa[rt][st][XRAW - 1], ga[st], ssl[rt], f, fl);
      } else if (rt * 16 + li < R) {
        const float* src = (const float*)p.x + (size_t)(rt * 16 + li) * p.ldx + kof(c, st);
        form(*(const f32x4_t*)src, *(const f32x4_t*)(src + 4 * (XRAW - 1)), gain_ld(c, st), ssl[rt], f, fl);
      }
      xr[c][rt][st] = f;
      if constexpr (SPLIT) xrl[c][rt][st] = fl;
    };
    if constexpr (STG_N2) {
      // the first row tile forms; then rows 16.., eight at a time in the registers the first
      // phase freed (more beside the first tile's pairs and the weights in flight spill),
      // overwrite the slot (a wave's LDS operations complete in order) and the second row
      // tile forms; every row's sums keep the order of one phase (chunk, then step)
#pragma unroll
      for (int c = 0; c < XR; ++c)
#pragma unroll
        for (int st = 0; st < CH; ++st) form_at(c, 0, st);
      const size_t k0 = (size_t)w * kw;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (16 + 8 * h >= R) break;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (16 + 8 * h + i < R)
            xn[i] = *(const u32x4_t*)((const float*)p.x + (size_t)(16 + 8 * h + i) * p.ldx + k0 + lane * 4);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (16 + 8 * h + i < R) *(u32x4_t*)(xs + (size_t)(8 * h + i) * lds.row_bytes + lane * 16) = xn[i];
      }
#pragma unroll
      for (int c = 0; c < XR; ++c)
#pragma unroll
        for (int st = 0; st < CH; ++st) form_at(c, 1, st);
    } else {
#pragma unroll
      for (int c = 0; c < XR; ++c)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int st = 0; st < CH; ++st) form_at(c, rt, st);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float v = ssl[rt];
      v += __shfl_xor(v, 16, 64);  // the four lanes of row li, in a fixed order
      v += __shfl_xor(v, 32, 64);
      if (lg == 0) ssq[w * RT * 16 + rt * 16 + li] = v;
    }
  }
  if constexpr (Q4 && XSRC != XSRC_GLOBAL) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int st = 2 * gi + tt;
          a = mfma_bf16(xr[st / CH][rt][st % CH], ones, a);
          if constexpr (LO_LDS) a = mfma_bf16(frag_xs(rt, st % CH, 1), ones, a);
          else if constexpr (SPLIT) a = mfma_bf16(xrl[st / CH][rt][st % CH], ones, a);
        }
        xg[gi][rt] = a;
      }
  }
  // the normed staging slots share their bytes with the reduction buffers
  if constexpr (STG_N) __syncthreads();

  // ---- straight-line (tile, chunk) pipeline ---------------------------------------------
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (it + PDW - 1 < NIT) load_w(wbuf[(it + PDW - 1) % PDW], sbuf[(it + PDW - 1) % PDW], it + PDW - 1);
    if constexpr (STG_G) {
      // this chunk's rows into the staging slot, then a later chunk's loads into the
      // registers they free (behind the weights in flight)
      stage_xc(it);
      if (it + XCD < NIT) load_xc(it + XCD);
    } else if constexpr (XSRC == XSRC_GLOBAL) {
      if (it + 1 < NIT) load_x(xbuf[(it + 1) & 1], xlbuf[(it + 1) & 1], it + 1);
    }
    compute(wbuf[it % PDW], sbuf[it % PDW], xbuf[it & 1], xlbuf[it & 1], it);
    if (it % NCH == NCH - 1) finalize(it / NCH);
  }

  if constexpr (EPI == EPI_ARGMAX) {
    if (w < RT) {  // the finishing wave of row tile w: its 16 columns per row, then one key
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const unsigned long long other = shfl_xor_u64(best[q], o);
          best[q] = other > best[q] ? other : best[q];
        }
      }
      if (li == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = w * 16 + 4 * lg + q;
          if (r < R) p.part[(size_t)r * gridDim.x + blockIdx.x] = best[q];
        }
      }
    }
  }
}

// ---- instantiation tables -----------------------------------------------------------------
template <int WT, int RT, int NB, int EPI, int XSRC, int T, int NCH, int CH, bool SPLIT>
static hipError_t launch_t(const GemmParams& p, int grid, hipStream_t s) {
  const size_t lds = gemm_lds_layout(WT, XSRC, SPLIT ? 1 : 0, p.R, p.waves, NB, p.K, T).total;
  auto fn = gemm_kernel<WT, RT, NB, EPI, XSRC, T, NCH, CH, SPLIT>;
  static std::atomic<bool> cleared[MAX_DEVICES];
  const hipError_t e = clear_dynamic_lds((const void*)fn, lds, cleared);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(p.waves * 64), lds, s, p);
  return hipGetLastError();
}

// The plan counts NCH chunks of 8 steps per wave; launches with two or three row tiles
// run twice as many chunks of chunk_steps(rt) = 4 steps (same k order per wave, so the
// same sums) to halve the weight and operand buffers in flight.
template <int WT, int NB, int EPI, int XSRC, int T, int NCH, int CH, bool SPLIT>
static hipError_t by_rt(const GemmParams& p, int grid, hipStream_t s) {
  static_assert(CH == 8, "plans count 8-step chunks");
  static_assert(chunk_steps(1) == 8 && chunk_steps(2) == 4 && chunk_steps(3) == 4, "chunk depth by row tiles");
  if constexpr (WT == WT_BF16 && XSRC == XSRC_GLOBAL) {
    // folded launches (see gemm_kernel): groups of 8 operand rows, 4-step chunks past 16 rows
    // (their staged rows would not fit beside 8-step chunks)
    switch ((p.R + 7) / 8) {
      case 1: return launch_t<WT, 1, NB, EPI, XSRC, T, NCH, 8, SPLIT>(p, grid, s);
      case 2: return launch_t<WT, 2, NB, EPI, XSRC, T, NCH, 8, SPLIT>(p, grid, s);
      case 3: return launch_t<WT, 3, NB, EPI, XSRC, T, 2 * NCH, 4, SPLIT>(p, grid, s);
      case 4: return launch_t<WT, 4, NB, EPI, XSRC, T, 2 * NCH, 4, SPLIT>(p, grid, s);
      default: return hipErrorInvalidValue;  // bf16 launches take at most 32 rows
    }
  } else {
    const int rt = (p.R + 15) / 16;
    if constexpr (xsrc_two_phase(XSRC)) {
      // normed hi/lo operands of two row tiles staged in two phases (up to 32 rows)
      if constexpr (NCH == 1 && SPLIT) {
        if (rt == 2) return launch_t<WT, 2, NB, EPI, XSRC, T, 2, 4, SPLIT>(p, grid, s);
      }
      return hipErrorInvalidValue;
    } else if (rt == 1) {
      return launch_t<WT, 1, NB, EPI, XSRC, T, NCH, 8, SPLIT>(p, grid, s);
    }
    if constexpr (xsrc_two_phase(XSRC)) {
      return hipErrorInvalidValue;
    } else if constexpr (XSRC == XSRC_NORM2) {
      return hipErrorInvalidValue;
    } else if constexpr (XSRC == XSRC_NORM && SPLIT) {
      // normed hi/lo operands of two row tiles: staged raw rows over a 256-element k range
      // per wave (at most GEMM_NORM_STAGED_ROWS rows; up to 32 as XSRC_NORMP)
      if constexpr (NCH == 1) {
        if (rt == 2 && p.R <= GEMM_NORM_STAGED_ROWS) return launch_t<WT, 2, NB, EPI, XSRC, T, 2, 4, SPLIT>(p, grid, s);
      }
      return hipErrorInvalidValue;
    } else {
      if (rt == 2) return launch_t<WT, 2, NB, EPI, XSRC, T, 2 * NCH, 4, SPLIT>(p, grid, s);
      // the vocabulary argmax over hi/lo pairs takes at most 32 rows; over single-plane rows
      // (bf16 and 4-bit weights, T as argmax_tiles_per_wg picks them) 48
      if constexpr (EPI == EPI_ARGMAX && (SPLIT || WT == WT_F32 || T > 8)) return hipErrorInvalidValue;
      else return launch_t<WT, 3, NB, EPI, XSRC, T, 2 * NCH, 4, SPLIT>(p, grid, s);
    }
  }
}

// one-tile launches: CH = 8 steps per chunk, NCH chunks per wave (staged operands hold
// every chunk in registers, so they stop at two chunks)
template <int WT, int NB, int EPI, int XSRC, bool SPLIT>
static hipError_t by_nch(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  if constexpr (xsrc_gain2(XSRC)) {  // one chunk per wave (raw rows staged)
    if (pl.nch != 1) return hipErrorInvalidValue;
    return pl.tiles_per_wg == 2 ? by_rt<WT, NB, EPI, XSRC, 2, 1, 8, SPLIT>(p, pl.grid, s)
                                : by_rt<WT, NB, EPI, XSRC, 1, 1, 8, SPLIT>(p, pl.grid, s);
  } else if constexpr (XSRC != XSRC_GLOBAL) {
    // normed operands: one tile per work-group, or two (the registers holding the
    // operand pairs then serve both tiles)
    if (pl.tiles_per_wg == 2) {
      switch (pl.nch) {
        case 1: return by_rt<WT, NB, EPI, XSRC, 2, 1, 8, SPLIT>(p, pl.grid, s);
        case 2: return by_rt<WT, NB, EPI, XSRC, 2, 2, 8, SPLIT>(p, pl.grid, s);
        default: return hipErrorInvalidValue;
      }
    }
    switch (pl.nch) {
      case 1: return by_rt<WT, NB, EPI, XSRC, 1, 1, 8, SPLIT>(p, pl.grid, s);
      case 2: return by_rt<WT, NB, EPI, XSRC, 1, 2, 8, SPLIT>(p, pl.grid, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (pl.nch) {
      case 1: return by_rt<WT, NB, EPI, XSRC, 1, 1, 8, SPLIT>(p, pl.grid, s);
      case 2: return by_rt<WT, NB, EPI, XSRC, 1, 2, 8, SPLIT>(p, pl.grid, s);
      case 3: return by_rt<WT, NB, EPI, XSRC, 1, 3, 8, SPLIT>(p, pl.grid, s);
      case 4: return by_rt<WT, NB, EPI, XSRC, 1, 4, 8, SPLIT>(p, pl.grid, s);
      case 5: return by_rt<WT, NB, EPI, XSRC, 1, 5, 8, SPLIT>(p, pl.grid, s);
      case 10: return by_rt<WT, NB, EPI, XSRC, 1, 10, 8, SPLIT>(p, pl.grid, s);
      default: return hipErrorInvalidValue;
    }
  }
}

// argmax launches: T tiles per work-group, NCH chunks of 8 steps per wave and tile
template <int WT, int XSRC, int NCH, bool SPLIT>
static hipError_t argmax_by_t(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  switch (pl.tiles_per_wg) {
    case 1: return by_rt<WT, 1, EPI_ARGMAX, XSRC, 1, NCH, 8, SPLIT>(p, pl.grid, s);
    case 2: return by_rt<WT, 1, EPI_ARGMAX, XSRC, 2, NCH, 8, SPLIT>(p, pl.grid, s);
    case 4: return by_rt<WT, 1, EPI_ARGMAX, XSRC, 4, NCH, 8, SPLIT>(p, pl.grid, s);
    case 8: return by_rt<WT, 1, EPI_ARGMAX, XSRC, 8, NCH, 8, SPLIT>(p, pl.grid, s);
    case 16: return by_rt<WT, 1, EPI_ARGMAX, XSRC, 16, NCH, 8, SPLIT>(p, pl.grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int WT, int XSRC, bool SPLIT>
static hipError_t argmax_by_ch(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  switch (pl.nch) {
    case 1: return argmax_by_t<WT, XSRC, 1, SPLIT>(pl, p, s);
    case 2: return argmax_by_t<WT, XSRC, 2, SPLIT>(pl, p, s);
    default: return hipErrorInvalidValue;
  }
}

// f32 weights take f32 operands (one f32 MFMA product). bf16 weights take a hi/lo pair for
// every computed activation (normed rows, attention output, SwiGLU output, encoder rows)
// and a single plane only where the rows are given in bf16 (fc over the residual slab,
// the lm_head over verify rows).
template <int WT>
static hipError_t by_kind(const GemmPlan& pl, int epi, int xsrc, const GemmParams& p, hipStream_t s) {
  if constexpr (WT == WT_F32) {
    if (p.split) return hipErrorInvalidValue;
    if (epi == EPI_ARGMAX) return xsrc == XSRC_LDS ? argmax_by_ch<WT, XSRC_LDS, false>(pl, p, s) : hipErrorInvalidValue;
    if (epi == EPI_STORE && xsrc == XSRC_GLOBAL) return by_nch<WT, 1, EPI_STORE, XSRC_GLOBAL, false>(pl, p, s);
    if (epi == EPI_STORE && xsrc == XSRC_NORM) return by_nch<WT, 1, EPI_STORE, XSRC_NORM, false>(pl, p, s);
    if (epi == EPI_RESID && xsrc == XSRC_GLOBAL) return by_nch<WT, 1, EPI_RESID, XSRC_GLOBAL, false>(pl, p, s);
    if (epi == EPI_SWIGLU && xsrc == XSRC_NORM) return by_nch<WT, 2, EPI_SWIGLU, XSRC_NORM, false>(pl, p, s);
  } else {
    if (epi == EPI_ARGMAX) {
      if (xsrc != XSRC_LDS) return hipErrorInvalidValue;
      return p.split ? argmax_by_ch<WT, XSRC_LDS, true>(pl, p, s) : argmax_by_ch<WT, XSRC_LDS, false>(pl, p, s);
    }
    if (epi == EPI_STORE && xsrc == XSRC_GLOBAL)
      return p.split ? by_nch<WT, 1, EPI_STORE, XSRC_GLOBAL, true>(pl, p, s)
                     : by_nch<WT, 1, EPI_STORE, XSRC_GLOBAL, false>(pl, p, s);
    if (!p.split) return hipErrorInvalidValue;
    if (epi == EPI_STORE && xsrc == XSRC_NORM) return by_nch<WT, 1, EPI_STORE, XSRC_NORM, true>(pl, p, s);
    if (epi == EPI_STORE && xsrc == XSRC_NORM2) return by_nch<WT, 1, EPI_STORE, XSRC_NORM2, true>(pl, p, s);
    if (epi == EPI_STORE && xsrc == XSRC_NORMP) return by_nch<WT, 1, EPI_STORE, XSRC_NORMP, true>(pl, p, s);
    if (epi == EPI_STORE && xsrc == XSRC_NORM2P) return by_nch<WT, 1, EPI_STORE, XSRC_NORM2P, true>(pl, p, s);
    if (epi == EPI_SWIGLU && xsrc == XSRC_NORMP) return by_nch<WT, 2, EPI_SWIGLU, XSRC_NORMP, true>(pl, p, s);
    if (epi == EPI_RESID && xsrc == XSRC_GLOBAL) return by_nch<WT, 1, EPI_RESID, XSRC_GLOBAL, true>(pl, p, s);
    if (epi == EPI_SWIGLU && xsrc == XSRC_NORM) return by_nch<WT, 2, EPI_SWIGLU, XSRC_NORM, true>(pl, p, s);
    if (epi == EPI_SWIGLU && xsrc == XSRC_GLOBAL) return by_nch<WT, 2, EPI_SWIGLU, XSRC_GLOBAL, true>(pl, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dflash
