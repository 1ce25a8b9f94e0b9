// Internal launch interface between the runtime (dflash.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace dflash {

constexpr int LDS_BYTES = 160 * 1024;  // gfx950 LDS per compute unit

// A kernel may take more than 64 KiB of dynamic LDS only once it has been cleared for it,
// and the clearance holds per device. `cleared` is the kernel's own per-device flag array:
// the first launch past 64 KiB on a device clears the kernel for the whole LDS of a compute
// unit there (one value, so racing host threads agree on it).
constexpr int MAX_DEVICES = 64;
inline hipError_t clear_dynamic_lds(const void* fn, size_t lds, std::atomic<bool>* cleared) {
  if (lds <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  if (cleared[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e == hipSuccess) cleared[dev].store(true, std::memory_order_release);
  return e;
}

enum { WT_F32 = 0, WT_BF16 = 1, WT_Q4 = 2 };  // weight storage (matches dflash_dtype)

constexpr int GEMM_MAXSEG = 12;
constexpr int GEMM_MAX_ROWS = 48;  // rows per GEMM launch (3 MFMA row tiles)
// normed hi/lo operands of two row tiles stage at most this many raw rows per wave in LDS
constexpr int GEMM_NORM_STAGED_ROWS = 18;
constexpr int ATTN_CHUNK = 64;     // keys per attention work-group
constexpr int ATTN_QG = 64;        // query vectors per attention pass
constexpr int MAX_WINDOW = 4096;   // attention chunks of one query stay within the combine's LDS

// XSRC_NORM2: XSRC_NORM whose rows r2 and up take the gains gain2 (one row tile, raw rows
// staged through LDS). XSRC_NORMP: XSRC_NORM over two row tiles of more rows than one
// staging of GEMM_NORM_STAGED_ROWS holds (up to 32), staged in two phases of at most 16
// rows, one per row tile. XSRC_NORM2P: XSRC_NORM2 over two row tiles (17-32 rows), staged
// the same way. Plans, LDS layouts and the kernel body otherwise treat them as XSRC_NORM.
enum { XSRC_GLOBAL = 0, XSRC_LDS = 1, XSRC_NORM = 2, XSRC_NORM2 = 3, XSRC_NORMP = 4, XSRC_NORM2P = 5 };
__host__ __device__ constexpr int xsrc_base(int xsrc) {
  return xsrc == XSRC_NORM2 || xsrc == XSRC_NORMP || xsrc == XSRC_NORM2P ? XSRC_NORM : xsrc;
}
__host__ __device__ constexpr bool xsrc_two_phase(int xsrc) { return xsrc == XSRC_NORMP || xsrc == XSRC_NORM2P; }
__host__ __device__ constexpr bool xsrc_gain2(int xsrc) { return xsrc == XSRC_NORM2 || xsrc == XSRC_NORM2P; }

// MFMA steps per pipelined chunk (16-byte weight loads per lane per chunk): deeper for one
// row tile, shallower when 2-3 row tiles of activations also sit in registers.
__host__ __device__ constexpr int chunk_steps(int rt) { return rt == 1 ? 8 : 4; }
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3 };

// One weight matrix [rows, K] in fragment-major blocks (launch_pack) whose outputs occupy
// columns col0..col0+rows-1.
struct GemmSeg {
  const void* w;
  const void* scales;  // q4 only: the packed scale blocks (launch_pack_q4)
  const void* biases;  // unused
  int32_t col0;
  int32_t rows;
};

// Y[r, n] = sum_k X[r, k] W[n, k] for r < R over the concatenated segments.
struct GemmParams {
  GemmSeg seg[GEMM_MAXSEG];
  int32_t nseg;
  int32_t ntiles;   // 16-column output tiles
  int32_t K;
  int32_t R;        // rows of X (<= GEMM_MAX_ROWS)
  int32_t waves;    // waves per work-group; each owns K/waves of every tile
  // split != 0 (bf16 weights only): operands are f32 values carried as bf16 hi/lo pairs,
  // two MFMA products per weight fragment. XSRC_GLOBAL/LDS read the hi plane at x and the
  // lo plane at xlo; XSRC_NORM forms the pair in registers; SWIGLU writes y (hi) and ylo.
  // split == 0: XSRC_GLOBAL/LDS read one plane of the weight dtype (inputs given in bf16
  // or f32 shapes).
  int32_t split;
  const void* x;    // XSRC_GLOBAL/LDS: [R, ldx] (see split); XSRC_NORM: f32 [R, ldx]
  const void* xlo;
  int64_t ldx;
  const void* gain;  // XSRC_NORM: act-dtype storage [K]
  // XSRC_NORM2: rows r2..R-1 are normalised with gains gain2 (the same storage as gain)
  const void* gain2;
  int32_t r2;
  float eps;
  void* y;          // STORE/RESID: f32 [R, ldy]; SWIGLU: hi/lo planes (split) or f32
  void* ylo;
  int64_t ldy;
  // RESID: when y2 is set, the finished rows are also stored there, [R, ldy2], in bf16
  // (y2_bf16) or f32 (a target's captured residual stream)
  void* y2;
  int64_t ldy2;
  int32_t y2_bf16;
  // RESID: when z is set, the finished rows times zgain (act-dtype storage [ldy]) are also
  // stored as operand rows of the next GEMM (hi/lo planes z/zlo when split, else f32 at z),
  // [.., ldz]: every row (zper 0), or runs of zper rows with the first of each left out;
  // launch row r is row zrow0 + r of the whole call
  const void* zgain;
  void* z;
  void* zlo;
  int64_t ldz;
  int32_t zper;
  int32_t zrow0;
  unsigned long long* part;  // ARGMAX: per-work-group best keys, [R][grid]
};

// Launch shape of one GEMM: waves per work-group and, per wave and tile, nch chunks of ch
// MFMA steps; tiles_per_wg output tiles per work-group; grid work-groups. It depends on K
// (never on the row count) so that every output keeps one reduction order.
struct GemmPlan {
  int waves, ch, nch, tiles_per_wg, grid;
};
bool gemm_plan_supported(const GemmPlan& pl, int epi, int xsrc);
hipError_t launch_gemm(int wt, int epi, int xsrc, const GemmPlan& pl, const GemmParams& p, hipStream_t s);
// LDS of a GEMM work-group: the cross-wave reduction buffers (double-buffered across tiles
// when a work-group owns several), the per-wave row sums of squares of the RMSNorm operands
// (XSRC_NORM), and, for bf16 and 4-bit weights, a per-wave slot that stages operand rows:
// XSRC_GLOBAL with at most two row tiles, the R rows of each plane for one chunk of the
// wave's k range; XSRC_NORM with at most two row tiles and a 256-element k range per wave,
// the R raw f32 rows of that range and its gains; XSRC_LDS (the argmax rows) with one row
// tile and one chunk per wave, the R rows of each plane, once per work-group.
// Staging loads only the R real rows with every lane busy, where the MFMA fragments would
// load 16 rows per row tile; the fragments are then read from LDS. The normed slot is dead
// once the operand pairs are formed and shares its bytes with the reduction buffers.
struct GemmLds {
  int stage;       // 0 none, 1 streamed rows, 2 normed rows, 3 LDS-source rows
  int row_bytes;   // staged bytes per row and plane, padded by 16 against bank conflicts
  size_t ssq_off;  // byte offsets in the work-group's LDS
  size_t xs_off;
  size_t xs_wave;  // staged bytes per wave
  size_t total;
};
// bf16 weights with streamed operands run folded: an MFMA takes 8 output columns over two
// k steps (one per half of its 16 columns) against groups of 8 operand rows, so a 16-row
// weight block serves two work-groups (see gemm_impl.h)
__host__ __device__ inline bool gemm_fold(int wt, int xsrc) { return wt == WT_BF16 && xsrc == XSRC_GLOBAL; }
// MFMA row groups of R operand rows (8 rows folded, else 16) and their k steps per chunk
__host__ __device__ inline int gemm_row_groups(int wt, int xsrc, int R) {
  return gemm_fold(wt, xsrc) ? (R + 7) / 8 : (R + 15) / 16;
}
__host__ __device__ inline int gemm_chunk_steps(int wt, int xsrc, int R) {
  return gemm_fold(wt, xsrc) ? ((R + 7) / 8 <= 2 ? 8 : 4) : chunk_steps((R + 15) / 16);
}
__host__ __device__ inline GemmLds gemm_lds_layout(int wt, int xsrc_in, int split, int R, int waves, int nb, int K,
                                                   int tiles_per_wg) {
  const int xsrc = xsrc_base(xsrc_in);
  const bool fold = gemm_fold(wt, xsrc);
  const int rt = gemm_row_groups(wt, xsrc, R), rows_pad = (fold ? 8 : 16) * rt;
  const int ch = gemm_chunk_steps(wt, xsrc, R), kstep = wt == WT_F32 ? 16 : 32;
  const int nch = K / (waves * ch * kstep);
  const size_t red = (size_t)(tiles_per_wg > 1 ? 2 : 1) * waves * rt * nb * 1024;
  const size_t ssq = xsrc == XSRC_NORM ? (size_t)waves * rows_pad * 4 : 0;
  GemmLds l{};
  if (wt != WT_F32 && xsrc == XSRC_GLOBAL && rows_pad <= 32) {
    l.stage = 1;
    l.row_bytes = ch * kstep * 2 + 16;
    l.xs_wave = (size_t)(split ? 2 : 1) * R * l.row_bytes;
  } else if (wt != WT_F32 && xsrc == XSRC_LDS && rt == 1 && nch == 1) {
    l.stage = 3;  // the LDS-source rows of the wave's k range, once per work-group
    l.row_bytes = ch * kstep * 2 + 16;
    l.xs_wave = (size_t)(split ? 2 : 1) * R * l.row_bytes;
  } else if (wt != WT_F32 && xsrc == XSRC_NORM && rt <= 2 && nch * ch * kstep == 256) {
    l.stage = 2;  // the raw rows of the wave's whole k range (256 f32) and its gain row(s)
    l.row_bytes = 256 * 4 + 16;
    const int rows = xsrc_two_phase(xsrc_in) ? 16 : R;  // two phases of at most 16 rows
    l.xs_wave = (size_t)rows * l.row_bytes + (xsrc_gain2(xsrc_in) ? 2 : 1) * 256 * 2;
  }
  if (l.stage == 2) {
    l.xs_off = 0;
    const size_t xs = (size_t)waves * l.xs_wave;
    l.ssq_off = ((xs > red ? xs : red) + 15) & ~(size_t)15;
    l.total = l.ssq_off + ssq;
  } else {
    l.ssq_off = red;
    l.xs_off = (red + ssq + 15) & ~(size_t)15;
    l.total = l.xs_off + (size_t)waves * l.xs_wave;
  }
  l.total = (l.total + 15) & ~(size_t)15;
  return l;
}
// Whole LDS of a GEMM work-group.
size_t gemm_lds_bytes(int wt, int xsrc, int split, int R, int waves, int nb, int K, int tiles_per_wg);

// ---- small kernels --------------------------------------------------------------------
struct AttnShape {
  int32_t nq, nkv, hd, L;
  int32_t window;
  int32_t cap, phase;  // ring slots stored (a multiple of 8, >= 64) and phase (a multiple of 8)
  float eps, theta;
  // 0 (the drafter): a query at q sees keys with |q - p| <= window, both directions, and the
  // block's own rows stay out of the cache. 1 (a target's verify forward): it sees keys
  // q - window < p <= q (a window past every distance on full-attention layers), and the
  // block's own keys and values are written into their cache slots.
  int32_t causal = 0;
};

// Row-major [N, K] linear -> fragment-major 1 KiB blocks (see misc.hip). perm_hd > 0 takes
// the rows of each run of perm_hd (one attention head) in the order 0, 2, 4, .., 1, 3, 5, ..
// (deinterleaved_row below).
hipError_t launch_pack(int wt, const void* src, int N, int K, void* dst, hipStream_t s, int perm_hd = 0);
// 4-bit linear (codes uint32 [N, K/8], bf16 scales/biases [N, K/64]) -> fragment-major
// code blocks (N*K/2 bytes) and scale blocks (N*K/16 bytes), see misc.hip; perm_hd as above.
hipError_t launch_pack_q4(const void* codes, const void* scales, const void* biases, int N, int K, void* dst_codes,
                          void* dst_scales, hipStream_t s, int perm_hd = 0);
// Source element of stored element j of a head of hd elements held in deinterleaved order:
// the evens first, then the odds. The rotate-half RoPE of that order pairs (2i, 2i + 1).
__host__ __device__ constexpr int deinterleaved_row(int j, int hd) {
  return j < hd / 2 ? 2 * j : 2 * (j - hd / 2) + 1;
}
// dst[j] = src[deinterleaved_row(j, hd)] for one vector of hd elements of elt bytes.
hipError_t launch_deinterleave(const void* src, void* dst, int hd, int elt, hipStream_t s);
// idx[r] = index of the largest key among part[r][0..groups) (lm_head argmax finish).
hipError_t launch_argmax_finalize(const unsigned long long* part, int groups, int R, int32_t* idx, hipStream_t s);
// Embedding rows [anchor, t_1 .. t_{R-1}] as f32 residual rows x, where t_i = toks[i-1]
// (device int32, clamped into [0, vocab)) or the mask token when toks is NULL; with rope != NULL also the
// rotary table rope[r][i] = (cos, sin), i < hd/2, of positions pos0..pos0+R-1 (rows 0..R-1)
// and pos0-nprev..pos0-1 (rows R..R+nprev-1). With nprev > 0, the f32 rows prev [nprev][hidden]
// are copied into x rows R..R+nprev-1.
hipError_t launch_embed(int act_bf16, const void* table, int hidden, int vocab, int32_t anchor, int32_t mask_id,
                        const int32_t* toks, int R, int nprev, const float* prev, float* x, float2* rope, int64_t pos0,
                        float theta, int hd, hipStream_t s);
// RMSNorm rows of in: act_bf16 -> hi/lo bf16 planes out/out_lo, else f32 out.
hipError_t launch_rownorm(int act_bf16, const float* in, const void* gain, float eps, int R, int H, void* out,
                          void* out_lo, hipStream_t s);
hipError_t launch_ring_write(int act_bf16, const AttnShape& a, const float* kv, const void* const* knorms,
                             int n, int64_t pos0, void* ring, hipStream_t s);
// Attention side of one layer of the block forward: q/k RMSNorm + RoPE of the R block rows
// (positions e..e+R-1, raw projections qkv f32 [R][(nq + 2 nkv) hd]), then attention over
// positions max(0, e-W)..e+R-1, writing the O-projection operand out/out_lo. The context
// keys come from the ring layer; the block's own keys and values are formed where they are
// used (bf16 shapes with head dim 64 or 128, reading the rotary table rope of launch_embed)
// or written into the ring slots of positions e..e+R-1 first (other shapes, which also use
// qb/qlo for the formed queries). With n > 0 (bf16 MFMA shapes only, n <= W), projection
// rows R..R+n-1 are the committed positions e-n..e-1 whose keys and values are not yet in
// the ring: they are formed like the block's own, used, and written into their ring slots.
hipError_t launch_block_attention(int act_bf16, const AttnShape& a, const float* qkv, const void* qnorm,
                                  const void* knorm, const float2* rope, void* ring_layer, int R, int n, int64_t e,
                                  void* qb, void* qlo, float* part, void* out, void* out_lo, hipStream_t s);
// Committed ends of the sequences of a batch round, passed by value.
constexpr int ATTN_MAX_SEQS = 64;
struct AttnSeqs {
  int32_t n;
  int64_t e[ATTN_MAX_SEQS];
};
// Rows of one ring write over several sequences: rows first[q]..first[q+1]-1 of kv belong
// to sequence q, at positions start[q].., into the ring at ring0 + q * ring_stride bytes
// (first[0] = 0, non-decreasing; empty ranges allowed).
struct RingSeqs {
  int32_t n;
  int32_t first[ATTN_MAX_SEQS + 1];
  int64_t start[ATTN_MAX_SEQS];
};
// launch_ring_write over several sequences in one launch: the bf16 MFMA shapes (otherwise
// hipErrorNotSupported, and callers write sequence by sequence).
hipError_t launch_ring_write_batch(int act_bf16, const AttnShape& a, const float* kv, const void* const* knorms,
                                   const RingSeqs& seqs, void* ring0, size_t ring_stride, hipStream_t s);
// Anchors and first positions of a batch round's sequences, passed by value.
struct EmbedSeqs {
  int32_t n;
  int32_t anchor[ATTN_MAX_SEQS];
  int64_t pos0[ATTN_MAX_SEQS];
};
// launch_embed for a batch: rows [anchor_q, mask x (R1 - 1)] of every sequence, sequence
// after sequence, at positions pos0_q.., with their rotary table (required).
hipError_t launch_embed_batch(int act_bf16, const void* table, int hidden, const EmbedSeqs& seqs, int R1,
                              int32_t mask_id, float* x, float2* rope, float theta, int hd, hipStream_t s);
// launch_block_attention for n sequences at once (no committed rows): sequence s's R rows of
// raw projections and of the rotary table follow s - 1's, its ring sits ring_seq_bytes after
// s - 1's, and its output rows follow s - 1's in out/out_lo; part holds
// attention_partial_floats_batch floats. bf16 MFMA shapes run one launch pair for all
// sequences, other shapes one per sequence.
hipError_t launch_block_attention_batch(int act_bf16, const AttnShape& a, const AttnSeqs& seqs, const float* qkv,
                                        const void* qnorm, const void* knorm, const float2* rope, void* ring0,
                                        size_t ring_seq_bytes, int R, void* qb, void* qlo, float* part, void* out,
                                        void* out_lo, hipStream_t s);
size_t attention_partial_floats_batch(const AttnShape& a, int R, int n_seq);
// whether launch_block_attention takes committed rows (n > 0) for this shape
bool attention_forms_committed_rows(int act_bf16, const AttnShape& a);
size_t attention_partial_floats(const AttnShape& a, int R);
// the same for queries whose keys span at most `span` positions before the block
size_t attention_partial_floats_span(const AttnShape& a, int R, int span);
// greedy verify of n_seq sequences, one wave each: draft [n_seq][B], target [n_seq][B+1], out [n_seq][3]
hipError_t launch_verify(const int32_t* draft, const int32_t* target, int B, int vocab, int32_t* out,
                         hipStream_t s, int n_seq = 1);
// Streaming read of `bytes` (a multiple of 16, at least groups * 4096) by `groups` work-groups
// of contiguous shares; sink [groups] receives an XOR of what each read (misc.hip).
hipError_t launch_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int groups, hipStream_t s);
// Live window read-back; deint: the ring holds keys in deinterleaved order, restored here.
hipError_t launch_cache_read(int act_bf16, const AttnShape& a, const void* ring_layer, int64_t lo, int n,
                             void* kout, void* vout, hipStream_t s, int deint = 0);

// ---- the DSpark Markov head (markov.hip) ---------------------------------------------------
constexpr int MK_WG_PER_CU = 4;     // work-groups per compute unit of a chain step
constexpr int MK_MAX_GROUPS = 4096;  // bound on a step's work-groups (its key array)
bool markov_rank_supported(int act_bf16, int rank);
// work-groups of one chain step on a device of `cus` compute units
int markov_step_groups(int vocab, int rank, int act_bf16, int cus);
// One chain step over the vocabulary: keys[g] (g < groups) = the largest (score, index) key of
// work-group g, score[v] = logits[v] + w2[v] . w1[t]. t is the anchor when prev_keys is NULL,
// else the index of the largest of the previous step's prev_groups keys, which work-group 0
// also stores to prev_out[0]. The last step's keys are reduced by launch_argmax_finalize.
hipError_t launch_markov_step(int act_bf16, int rank, const void* w1, const void* w2, int vocab, const float* logits,
                              const unsigned long long* prev_keys, int prev_groups, int32_t anchor, int32_t* prev_out,
                              unsigned long long* keys, int groups, hipStream_t s);

}  // namespace dflash
