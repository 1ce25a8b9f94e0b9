// Host runtime of the DFlash round: the C-ABI declared in include/dflash.h.
//
// It validates the drafter shape, lays out the caller's workspace, keeps the ring's
// bookkeeping (committed end e, pending rows, slack S, capacity C) and enqueues the
// kernels of each call on the caller's stream. It never allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <new>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"
#include "noalloc.h"

using namespace dflash;

namespace {

constexpr int MAX_BLOCK_LIMIT = 256;

struct Lin {
  const void *w, *s, *b;
};
struct Layer {
  Lin q, k, v, o, gate, up, down;
  const void *in_norm, *post_norm, *q_norm, *k_norm;
};

struct Layout {  // byte offsets into the workspace
  size_t argmax_part, knorm_ptrs, x, hn, qkv, qb, attn, mlp, zrows, part, rope, app_fc, app_kv;
  size_t logits, mk_part;  // DSpark: backbone logits of a block, the chain's keys (two steps' worth)
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int64_t slack_rows(int64_t block) {
  // clamp(block * 8, 32, 128) rows of speculative buffer, floored at the block size
  // (lablup/mlxcel #1762, What changed; Pre-merge review round, second finding)
  return std::max(std::min(std::max(block * 8, (int64_t)32), (int64_t)128), block);
}

struct Cfg {
  dflash_config c;
  int wt;       // WT_* of the linears
  bool bf;      // act dtype bf16
  int act_elt;  // bytes per activation / ring element
  int R;        // max rows of a block forward = max_block + 1
  int64_t S, C;  // slack and capacity of the window (C = W + S)
  int64_t Cs;    // slots stored: C rounded up to a multiple of 8, at least W + R and 64
  bool dspark;   // the DSpark form (gamma rows, every row's logits, the Markov chain)
  bool trad;     // adjacent-pair RoPE, run as rotate-half over deinterleaved q/k elements
  AttnShape a;
};

}  // namespace

struct dflash_ctx {
  Cfg cfg;
  Layout lay;
  Lin embed_lin, lm_head, fc;
  const void *embed, *enc_norm, *final_norm;
  const void *markov_w1 = nullptr, *markov_w2 = nullptr;
  int mk_groups = 0;  // work-groups of a Markov chain step
  std::vector<Layer> layers;
  unsigned char* ring;
  unsigned char* ws;
  int cus = 256;        // compute units of the device the context was created on
  int device = 0;       // that device
  // that device's copy of the fixed argmax key array (dflash_lm_head_argmax_noalloc)
  unsigned long long* noalloc_keys = nullptr;
  int64_t e = 0;        // committed context end (absolute position)
  int64_t pending = 0;  // rows appended since the last trim
  // rows at positions kv_pos .. kv_pos + kv_rows - 1 whose encoder rows (fc output) sit in
  // the append buffer while their K/V are not yet in the ring: the next draft projects them
  // in its own per-layer QKV launches and its attention writes them into the ring; any
  // other call that needs the ring projects them first (flush_kv)
  int64_t kv_pos = 0;
  int32_t kv_rows = 0;
  int fold_rows = 0;  // rows of a QKV launch that may carry such rows (0: never deferred)
  // events around the first argmax GEMM launch of the next dflash_lm_head_argmax call
  // (dflash_time_next_argmax); `active` while that call runs
  hipEvent_t tev_start = nullptr, tev_end = nullptr;
  bool tev_active = false;
  // events around the Markov chain of the next DSpark draft (dflash_time_next_chain)
  hipEvent_t cev_start = nullptr, cev_end = nullptr;
  char err[512] = {0};
};

namespace {

dflash_status fail(dflash_ctx* ctx, dflash_status st, const char* fmt, ...) {
  if (ctx) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(ctx->err, sizeof ctx->err, fmt, ap);
    va_end(ap);
  }
  return st;
}

thread_local char g_create_err[512];

dflash_status cfg_fail(char* buf, dflash_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, 512, fmt, ap);
  va_end(ap);
  return st;
}

int kstep(int wt) { return wt == WT_F32 ? 16 : 32; }

constexpr int CHUNK_STEPS = 8;
// rows of a QKV launch with committed rows folded in: draft rows plus committed rows in one
// MFMA row tile, or in two row tiles staged in two phases
constexpr int FOLD_ROWS = 16;
constexpr int FOLD_ROWS_TWO = 32;

// Launch plan of a GEMM with contraction length K. Waves and chunking depend on K only.
bool plan_gemm(int wt, int epi, int xsrc, int K, GemmPlan* pl) {
  const int ks = kstep(wt);
  if (K % (CHUNK_STEPS * ks)) return false;
  const int units = K / (CHUNK_STEPS * ks);
  for (int w = 8; w >= 1; --w) {
    if (units % w) continue;
    GemmPlan p{w, CHUNK_STEPS, units / w, epi == EPI_ARGMAX ? 4 : 1, 0};
    if (gemm_plan_supported(p, epi, xsrc)) {
      *pl = p;
      return true;
    }
  }
  return false;
}

// Tiles per work-group of an argmax launch: small work-groups keep the dispatcher
// balancing the vocabulary stream; with more rows, more tiles per work-group bound how
// often the operand rows are re-read. Measured over a vocabulary-sized head (202048 x
// 2048, operand rows of one row tile staged through LDS): bf16 single-plane rows run
// fastest at two tiles (four past 16 rows), bf16 hi/lo pairs, with twice the operand loads
// and products, at four (eight past 8 rows, where whole-round runs favoured it); 4-bit
// heads at eight for hi/lo pairs (four up to 5 rows, where that launch reads its lo
// fragments from LDS and fits two work-groups per CU) and four (eight past 16 rows) for
// single-plane rows.
int argmax_tiles_per_wg(int wt, int split, int ntiles, int rows) {
  if (ntiles < 1024) return 1;
  if (ntiles < 8192) return 2;
  if (wt == WT_Q4) return split ? (rows <= 5 ? 4 : 8) : (rows > 16 ? 8 : 4);
  if (!split) return rows > 16 ? 4 : 2;
  return rows > 8 ? 8 : 4;
}

dflash_status check_cfg(const dflash_config* c, Cfg* out, char* err) {
  if (!c) return cfg_fail(err, DFLASH_E_ARG, "config is NULL");
  const int32_t dims[] = {c->hidden, c->layers, c->q_heads, c->kv_heads, c->head_dim, c->intermediate,
                          c->vocab, c->target_streams, c->target_width, c->window, c->max_block};
  for (int32_t d : dims)
    if (d <= 0) return cfg_fail(err, DFLASH_E_SHAPE, "every dimension must be positive");
  int wt;
  if (c->weight_dtype == DFLASH_F32) wt = WT_F32;
  else if (c->weight_dtype == DFLASH_BF16) wt = WT_BF16;
  else if (c->weight_dtype == DFLASH_Q4G64) wt = WT_Q4;
  else return cfg_fail(err, DFLASH_E_ARG, "unknown weight dtype %d", c->weight_dtype);
  const bool bf = wt != WT_F32;
  if (c->act_dtype != (bf ? DFLASH_BF16 : DFLASH_F32))
    return cfg_fail(err, DFLASH_E_ARG, "act dtype must be f32 with f32 weights and bf16 otherwise");
  if (c->max_block > MAX_BLOCK_LIMIT) return cfg_fail(err, DFLASH_E_RANGE, "max_block above %d", MAX_BLOCK_LIMIT);
  if (c->window > MAX_WINDOW) return cfg_fail(err, DFLASH_E_SHAPE, "window above %d", MAX_WINDOW);
  if (c->q_heads % c->kv_heads) return cfg_fail(err, DFLASH_E_SHAPE, "q_heads must be a multiple of kv_heads");
  if (c->head_dim % 2 || c->head_dim > 128 || c->head_dim % 16)
    return cfg_fail(err, DFLASH_E_SHAPE, "head_dim must be a multiple of 16 and at most 128");
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return cfg_fail(err, DFLASH_E_RANGE, "mask_token_id %d outside [0, %d)", c->mask_token_id, c->vocab);
  if (c->vocab % 16) return cfg_fail(err, DFLASH_E_SHAPE, "vocab must be a multiple of 16");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f) || !std::isfinite(c->rms_eps) || !std::isfinite(c->rope_theta))
    return cfg_fail(err, DFLASH_E_ARG, "rms_eps and rope_theta must be positive and finite");
  if (c->rope_traditional != 0 && c->rope_traditional != 1)
    return cfg_fail(err, DFLASH_E_ARG, "rope_traditional must be 0 or 1");
  if (c->variant == DFLASH_VARIANT_DSPARK) {
    // the verify width (block + 1 rows) is clamped at 32 (lablup/mlxcel #1751, Security fixes)
    if (c->max_block + 1 > 32)
      return cfg_fail(err, DFLASH_E_RANGE, "a DSpark verify width of %d rows is above 32", c->max_block + 1);
    if (!markov_rank_supported(bf, c->markov_rank))
      return cfg_fail(err, DFLASH_E_SHAPE, "markov_rank %d is not one of 64, 128, 256%s", c->markov_rank,
                      bf ? ", 512" : "");
  } else if (c->variant != DFLASH_VARIANT_DFLASH) {
    return cfg_fail(err, DFLASH_E_ARG, "unknown variant %d", c->variant);
  } else if (c->markov_rank != 0) {
    return cfg_fail(err, DFLASH_E_ARG, "markov_rank is for DSpark contexts only");
  }
  // every extent and element count handed to a kernel fits an int32; the products are
  // bounded factor by factor (every factor is positive and below 2^31 + 512), so that no
  // partial product can pass the int64 range either
  const int64_t qd = (int64_t)c->q_heads * c->head_dim, kvd = (int64_t)c->kv_heads * c->head_dim;
  const int64_t fin = (int64_t)c->target_streams * c->target_width;
  const int64_t H = c->hidden;
  const int64_t slots = (int64_t)c->window + 128 + c->max_block + 72;
  const std::initializer_list<int64_t> products[] = {
      {qd}, {kvd}, {fin}, {H, c->vocab}, {H, c->intermediate}, {H, fin}, {H, qd}, {c->layers, 2, kvd, slots}};
  for (const auto& f : products) {
    int64_t v = 1;
    for (int64_t x : f)
      if (x > INT32_MAX || (v *= x) > INT32_MAX)
        return cfg_fail(err, DFLASH_E_SHAPE, "a dimension product would wrap an int32");
  }
  const int unit = chunk_steps(1) * kstep(wt);
  const int64_t ks[] = {H, c->intermediate, qd, fin};
  for (int64_t k : ks)
    if (k % unit) return cfg_fail(err, DFLASH_E_SHAPE, "hidden, intermediate, q_heads*head_dim and fc width must be multiples of %d", unit);
  if (H % 16 || c->intermediate % 16 || qd % 16 || kvd % 16)
    return cfg_fail(err, DFLASH_E_SHAPE, "output dimensions must be multiples of 16");
  // every contraction of the round needs a launch plan, and the LDS-staged norm prologue
  // must fit at least 16 rows of hidden
  GemmPlan pl;
  const struct { int epi, xsrc; int64_t K; } gemms[] = {
      {EPI_STORE, XSRC_NORM, H},           {EPI_RESID, XSRC_GLOBAL, qd},  {EPI_SWIGLU, XSRC_NORM, H},
      {EPI_SWIGLU, XSRC_GLOBAL, H},
      {EPI_RESID, XSRC_GLOBAL, c->intermediate}, {EPI_STORE, XSRC_GLOBAL, fin}, {EPI_STORE, XSRC_GLOBAL, H},
      {EPI_ARGMAX, XSRC_LDS, H}};
  for (const auto& gm : gemms)
    if (!plan_gemm(wt, gm.epi, gm.xsrc, (int)gm.K, &pl))
      return cfg_fail(err, DFLASH_E_SHAPE, "no GEMM launch plan for a contraction of length %lld", (long long)gm.K);
  if (gemm_lds_bytes(wt, XSRC_NORM, 1, 16, 8, 2, c->hidden, 2) > (size_t)LDS_BYTES)
    return cfg_fail(err, DFLASH_E_SHAPE, "hidden too large for the staged operand");
  Cfg g;
  g.c = *c;
  g.wt = wt;
  g.bf = bf;
  g.act_elt = bf ? 2 : 4;
  g.R = c->max_block + 1;
  g.dspark = c->variant == DFLASH_VARIANT_DSPARK;
  g.trad = c->rope_traditional != 0;
  g.S = slack_rows(c->max_block);
  g.C = c->window + g.S;
  // storage: the block's own keys (positions e..e+R-1) get slots of their own past the
  // window, and the slot grid is 8-aligned so that attention reads aligned 8-key runs
  g.Cs = std::max<int64_t>({g.C, (int64_t)c->window + g.R, (int64_t)64});
  g.Cs = (g.Cs + 7) & ~(int64_t)7;
  if (c->ring_phase < 0) return cfg_fail(err, DFLASH_E_ARG, "ring_phase must be >= 0");
  g.a.nq = c->q_heads;
  g.a.nkv = c->kv_heads;
  g.a.hd = c->head_dim;
  g.a.L = c->layers;
  g.a.window = c->window;
  g.a.cap = (int32_t)g.Cs;
  g.a.phase = (int32_t)((c->ring_phase % g.Cs) & ~(int64_t)7);
  g.a.eps = c->rms_eps;
  g.a.theta = c->rope_theta;
  *out = g;
  return DFLASH_OK;
}

// rows of the normed-operand planes: a draft's rows or one append chunk, whichever is more
size_t hn_rows(const Cfg& g) { return std::max<size_t>((size_t)g.R, (size_t)GEMM_MAX_ROWS); }

Layout make_layout(const Cfg& g) {
  const dflash_config& c = g.c;
  const size_t H = c.hidden, R = g.R;
  const size_t qd = (size_t)c.q_heads * c.head_dim, kvd = (size_t)c.kv_heads * c.head_dim;
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  // per-work-group argmax keys of one lm_head launch: <= 48 rows x <= V/16 work-groups
  L.argmax_part = take(sizeof(unsigned long long) * GEMM_MAX_ROWS * (size_t)(c.vocab / 16));
  L.knorm_ptrs = take(sizeof(void*) * c.layers);
  // operand buffers (q, attention output, SwiGLU output, normed rows) hold 4 bytes per
  // element: f32, or for bf16 shapes a hi plane followed by a lo plane (see lo_plane)
  const size_t RQ = std::max<size_t>(R, FOLD_ROWS_TWO);  // draft rows and folded committed rows
  L.x = take(4 * RQ * H);
  L.hn = take(4 * hn_rows(g) * H);  // normed rows of launches past one row tile
  L.qkv = take(4 * RQ * (qd + 2 * kvd));
  L.qb = take(4 * R * qd);
  L.attn = take(4 * R * qd);
  L.mlp = take(4 * R * c.intermediate);
  L.zrows = take(4 * R * H);  // drafted rows through the final norm (or its gain alone): lm_head operand
  L.part = take(4 * attention_partial_floats(g.a, (int)R));
  L.rope = take(sizeof(float2) * RQ * (c.head_dim / 2));  // rotary table of a draft's positions
  L.app_fc = take(4 * (size_t)GEMM_MAX_ROWS * H);
  L.app_kv = take(4 * (size_t)GEMM_MAX_ROWS * c.layers * 2 * kvd);
  if (g.dspark) {
    L.logits = take(4 * (size_t)c.max_block * c.vocab);
    L.mk_part = take(sizeof(unsigned long long) * 2 * MK_MAX_GROUPS);
  }
  L.total = o;
  return L;
}

size_t ring_bytes_of(const Cfg& g) {
  return (size_t)g.act_elt * g.c.layers * 2 * g.c.kv_heads * (size_t)g.Cs * g.c.head_dim;
}

// Fragment-major copies of every linear live in the caller's packed buffer, in this order:
// fc, lm_head, then per layer q, k, v, o, gate, up, down; with adjacent-pair RoPE the
// deinterleaved copies of every layer's q_norm and k_norm follow.
struct PackedLayout {
  size_t total = 0;
  std::vector<size_t> off;  // byte offset of each linear, in the order above
  size_t gains = 0;         // offset of the deinterleaved gains: per layer q_norm, k_norm
  size_t gain_stride = 0;   // bytes per gain copy
};

// f32/bf16: the fragment-major matrix; q4: code blocks (K/2 bytes per row) followed by
// scale blocks (K/16 bytes per row)
size_t q4_code_bytes(int64_t N, int64_t K) { return (size_t)N * K / 2; }
size_t linear_bytes(const Cfg& g, int64_t N, int64_t K) {
  if (g.wt == WT_Q4) return q4_code_bytes(N, K) + (size_t)N * K / 16;
  return (size_t)N * K * (g.wt == WT_F32 ? 4 : 2);
}

PackedLayout make_packed_layout(const Cfg& g) {
  const dflash_config& c = g.c;
  const int64_t H = c.hidden, qd = (int64_t)c.q_heads * c.head_dim, kvd = (int64_t)c.kv_heads * c.head_dim;
  const int64_t F = (int64_t)c.target_streams * c.target_width, I = c.intermediate;
  PackedLayout P;
  auto add = [&](int64_t N, int64_t K) {
    P.off.push_back(P.total);
    P.total = align256(P.total + linear_bytes(g, N, K));
  };
  add(H, F);
  add(c.vocab, H);
  for (int l = 0; l < c.layers; ++l) {
    add(qd, H);
    add(kvd, H);
    add(kvd, H);
    add(H, qd);
    add(I, H);
    add(I, H);
    add(H, I);
  }
  if (g.trad) {
    P.gains = P.total;
    P.gain_stride = align256((size_t)c.head_dim * (g.wt == WT_F32 ? 4 : 2));
    P.total += P.gain_stride * 2 * c.layers;
  }
  return P;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// lo plane of an operand buffer of rows x ld elements (bf16 shapes), or NULL (f32 shapes)
void* lo_plane(const Cfg& g, void* base, size_t rows, size_t ld) {
  return g.bf ? (unsigned char*)base + rows * ld * 2 : nullptr;
}

dflash_status dev(dflash_ctx* ctx, hipError_t e, const char* what) {
  if (e == hipSuccess) return DFLASH_OK;
  return fail(ctx, DFLASH_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// ---- GEMM driver: chunks rows, fills parameters, picks the grid -------------------------
struct GemmCall {
  int epi, xsrc;
  std::vector<GemmSeg> segs;
  int K;
  const void* x;
  int64_t ldx;  // elements
  const void* gain;
  void* y;
  int64_t ldy;  // elements
  int32_t* idx;
  int split = 0;  // operands are hi/lo bf16 pairs (x/xlo planes, or formed by the norm prologue)
  const void* xlo = nullptr;
  void* ylo = nullptr;
  // normed operands only: rows r2 and up take the gains gain2, in one launch of one row
  // tile whose raw rows are staged through LDS
  const void* gain2 = nullptr;
  int r2 = 0;
  // argmax only: per-work-group keys go here (part_bytes long) instead of the workspace
  unsigned long long* part = nullptr;
  size_t part_bytes = 0;
  // residual only: also store the finished rows here ([rows, ldy2], act dtype)
  void* y2 = nullptr;
  int64_t ldy2 = 0;
  // residual only: the finished rows times zgain as operand rows (GemmParams::z)
  const void* zgain = nullptr;
  void* z = nullptr;
  void* zlo = nullptr;
  int64_t ldz = 0;
  int zper = 0;
};

dflash_status run_gemm(dflash_ctx* ctx, const GemmCall& gc_in, int rows, hipStream_t st) {
  const Cfg& g = ctx->cfg;
  GemmCall gc = gc_in;
  const int wt = g.wt;
  GemmPlan plan;
  if (gc.gain2 && (gc.xsrc != XSRC_NORM || !gc.split || rows > 32 || gc.r2 < 0 || gc.r2 > rows))
    return fail(ctx, DFLASH_E_SHAPE, "operand rows with two gains (%d rows, split at %d) need one staged normed launch",
                rows, gc.r2);
  // normed hi/lo operands run directly when each wave's k range is 256 elements (their raw
  // rows are staged through LDS: one staging up to GEMM_NORM_STAGED_ROWS rows, two phases up
  // to a launch's 32); otherwise rows past one row tile are normalised once into planes and
  // streamed
  if (gc.xsrc == XSRC_NORM && gc.split && rows > 16 && !(plan_gemm(wt, gc.epi, gc.xsrc, gc.K, &plan) && plan.nch == 1)) {
    void* hn = ctx->ws + ctx->lay.hn;
    void* hn_lo = lo_plane(g, hn, hn_rows(g), gc.K);
    const dflash_status s0 =
        dev(ctx, launch_rownorm(1, (const float*)gc.x, gc.gain, g.c.rms_eps, rows, gc.K, hn, hn_lo, st), "row norm");
    if (s0 != DFLASH_OK) return s0;
    gc.xsrc = XSRC_GLOBAL;
    gc.x = hn;
    gc.xlo = hn_lo;
    gc.ldx = gc.K;
    gc.gain = nullptr;
  }
  const int nb = gc.epi == EPI_SWIGLU ? 2 : 1;
  if (!plan_gemm(wt, gc.epi, gc.xsrc, gc.K, &plan)) return fail(ctx, DFLASH_E_SHAPE, "no GEMM plan for K = %d", gc.K);
  const int waves = plan.waves;
  const size_t x_elt = gc.xsrc == XSRC_NORM ? 4 : g.act_elt;  // a split operand is two bf16 planes
  const size_t y_elt = gc.epi == EPI_SWIGLU ? g.act_elt : 4;
  int N = 0;
  for (const auto& s : gc.segs) N = std::max(N, s.col0 + s.rows);
  int r0 = 0;
  while (r0 < rows) {
    // bf16 and 4-bit weights take at most two row tiles per launch: their operand rows are
    // staged through LDS there, while a three-tile launch loads 48-row fragments per wave
    // (measured slower than two staged launches over the same rows)
    int rc = std::min(rows - r0, g.bf ? 32 : GEMM_MAX_ROWS);
    if (gc.epi == EPI_ARGMAX) {
      // one finishing wave per row tile; single-plane rows over bf16 or 4-bit weights (the
      // verify rows) take three row tiles, so 48 verify rows stream the head once
      const int cap = g.bf && !gc.split ? GEMM_MAX_ROWS : 32;
      rc = std::min(rows - r0, std::min(cap, 16 * waves));
    }
    // tiles per work-group that size the reduction buffers: two or more for the argmax, two
    // for normed hi/lo operands over an even tile count (the launch below)
    const bool norm_two = gc.xsrc == XSRC_NORM && gc.split && (N / 16) % 2 == 0 && (rc <= 16 || nb == 1);
    const int tpw_lds = gc.epi == EPI_ARGMAX || norm_two ? 2 : 1;
    // staged normed rows past one staging (past one row tile with two gain rows) take two
    // phases
    auto xsrc_for = [&](int r) {
      if (gc.gain2) return r > 16 ? (int)XSRC_NORM2P : (int)XSRC_NORM2;
      return gc.xsrc == XSRC_NORM && gc.split && r > GEMM_NORM_STAGED_ROWS ? (int)XSRC_NORMP : gc.xsrc;
    };
    while (rc > 1 && gemm_lds_bytes(wt, xsrc_for(rc), gc.split, rc, waves, nb, gc.K, tpw_lds) > (size_t)LDS_BYTES) --rc;
    if (gc.gain2 && (rc < rows || gemm_lds_layout(wt, xsrc_for(rc), gc.split, rc, waves, nb, gc.K, tpw_lds).stage != 2))
      return fail(ctx, DFLASH_E_SHAPE, "operand rows with two gains (%d rows) do not fit one staged launch", rows);
    GemmParams p{};
    for (size_t i = 0; i < gc.segs.size(); ++i) p.seg[i] = gc.segs[i];
    p.nseg = (int)gc.segs.size();
    p.ntiles = N / 16;
    p.K = gc.K;
    p.R = rc;
    p.waves = waves;
    p.split = gc.split;
    p.x = (const unsigned char*)gc.x + (size_t)r0 * gc.ldx * x_elt;
    p.xlo = gc.xlo ? (const unsigned char*)gc.xlo + (size_t)r0 * gc.ldx * x_elt : nullptr;
    p.ldx = gc.ldx;
    p.gain = gc.gain;
    p.gain2 = gc.gain2 ? gc.gain2 : gc.gain;
    p.r2 = gc.gain2 ? gc.r2 : rc;
    p.eps = g.c.rms_eps;
    GemmPlan pl = plan;
    pl.grid = gemm_fold(wt, gc.xsrc) ? 2 * p.ntiles : p.ntiles;  // folded: 8-column tiles
    if (norm_two) {
      // normed hi/lo operands: two tiles per work-group share the operand registers and
      // halve the operand reads from L2 (two row tiles of the gate/up pair keep one: its
      // weights of two tiles would not fit beside the operand pairs)
      pl.tiles_per_wg = 2;
      pl.grid = p.ntiles / 2;
    }
    if (gc.epi == EPI_ARGMAX) {
      pl.tiles_per_wg = argmax_tiles_per_wg(wt, gc.split, p.ntiles, rc);
      pl.grid = (p.ntiles + pl.tiles_per_wg - 1) / pl.tiles_per_wg;
      p.part = (unsigned long long*)(ctx->ws + ctx->lay.argmax_part);
      if (gc.y) {  // the f32 logits too ([rows, ldy])
        p.y = (unsigned char*)gc.y + (size_t)r0 * gc.ldy * sizeof(float);
        p.ldy = gc.ldy;
      }
      if (gc.part) {  // callers check the bound before the first launch (argmax_key_bytes)
        if ((size_t)rc * pl.grid * sizeof(unsigned long long) > gc.part_bytes)
          return fail(ctx, DFLASH_E_SHAPE, "argmax keys of %d rows x %d work-groups exceed %zu bytes", rc, pl.grid,
                      gc.part_bytes);
        p.part = gc.part;
      }
    } else {
      p.y = (unsigned char*)gc.y + (size_t)r0 * gc.ldy * y_elt;
      p.ylo = gc.ylo ? (unsigned char*)gc.ylo + (size_t)r0 * gc.ldy * y_elt : nullptr;
      p.ldy = gc.ldy;
      p.y2 = gc.y2 ? (unsigned char*)gc.y2 + (size_t)r0 * gc.ldy2 * g.act_elt : nullptr;
      p.ldy2 = gc.ldy2;
      p.y2_bf16 = g.bf ? 1 : 0;
      p.zgain = gc.zgain;
      p.z = gc.z;
      p.zlo = gc.zlo;
      p.ldz = gc.ldz;
      p.zper = gc.zper;
      p.zrow0 = r0;
    }
    const bool timed = gc.epi == EPI_ARGMAX && ctx->tev_active && r0 == 0;
    if (timed && hipEventRecord(ctx->tev_start, st) != hipSuccess) return dev(ctx, hipGetLastError(), "timing event");
    const int xsrc_launch = xsrc_for(rc);
    const hipError_t le = launch_gemm(wt, gc.epi, xsrc_launch, pl, p, st);
    if (timed && le == hipSuccess && hipEventRecord(ctx->tev_end, st) != hipSuccess)
      return dev(ctx, hipGetLastError(), "timing event");
    if (le != hipSuccess)
      return fail(ctx, DFLASH_E_DEVICE,
                  "gemm launch (epi %d, xsrc %d, K %d, rows %d, tiles %d, waves %d, ch %d x %d, tiles/wg %d, grid %d): %s",
                  gc.epi, xsrc_launch, gc.K, rc, p.ntiles, waves, pl.ch, pl.nch, pl.tiles_per_wg, pl.grid,
                  hipGetErrorString(le));
    if (gc.epi == EPI_ARGMAX && gc.idx) {  // no index output: the logits were the point
      const hipError_t fe = launch_argmax_finalize(p.part, pl.grid, rc, gc.idx + r0, st);
      if (fe != hipSuccess) return dev(ctx, fe, "argmax finalize");
    }
    r0 += rc;
  }
  return DFLASH_OK;
}

GemmSeg seg(const Lin& l, int col0, int rows) { return GemmSeg{l.w, l.s, l.b, col0, rows}; }

// A DFlash draft ranks rows 1..B of each run of B + 1 (per = B + 1), a target forward every
// row (per = 0), through the final RMSNorm and the lm_head. The norm's per-row factor 1/rms
// is positive, so it leaves each row's argmax as it is: the last down launch stores its
// finished rows times the norm's gain alone as the lm_head's operand rows, in place of a
// separate norm pass over them.
void gain_rows_for_argmax(const dflash_ctx* ctx, GemmCall& dn, void* z, void* zlo, int per) {
  dn.zgain = ctx->final_norm;
  dn.z = z;
  dn.zlo = zlo;
  dn.ldz = ctx->cfg.c.hidden;
  dn.zper = per;
}

// Rows of a QKV launch that may carry committed rows beside the draft rows (0: none): bf16
// activations on the MFMA attention (which forms and writes those rows), and a normed
// launch that stages its raw rows through LDS: two row tiles in two phases where that
// fits, else one.
int fold_rows_of(const Cfg& g) {
  const dflash_config& c = g.c;
  if (!g.bf || !attention_forms_committed_rows(g.bf, g.a)) return 0;
  GemmPlan pl;
  if (!plan_gemm(g.wt, EPI_STORE, XSRC_NORM, c.hidden, &pl) || pl.nch != 1) return 0;
  const int tiles = (c.q_heads + 2 * c.kv_heads) * c.head_dim / 16;
  const int tpw = tiles % 2 == 0 ? 2 : 1;
  for (const int rows : {FOLD_ROWS_TWO, FOLD_ROWS}) {
    const int xs = rows > 16 ? XSRC_NORM2P : XSRC_NORM2;
    if (gemm_lds_layout(g.wt, xs, 1, rows, pl.waves, 1, c.hidden, tpw).stage == 2 &&
        gemm_lds_bytes(g.wt, xs, 1, rows, pl.waves, 1, c.hidden, tpw) <= (size_t)LDS_BYTES)
      return rows;
  }
  return 0;
}

// K/V of rc encoder rows (the fc output in the append buffer) at positions pos.. into the
// ring: the per-layer k/v projections with the encoder norm fused as the operand norm, six
// layers per launch, then the ring write (k RMSNorm, RoPE, cache dtype)
// the raw per-layer K/V (app_kv, f32 [rc][layers * 2 * kvd]) of the rc encoder rows in app_fc
dflash_status kv_gemms(dflash_ctx* ctx, int rc, hipStream_t st) {
  const Cfg& g = ctx->cfg;
  const dflash_config& c = g.c;
  const int kvd = c.kv_heads * c.head_dim;
  const int kv_cols = c.layers * 2 * kvd;
  const float* fc_out = (const float*)(ctx->ws + ctx->lay.app_fc);
  float* kv = (float*)(ctx->ws + ctx->lay.app_kv);
  for (int l0 = 0; l0 < c.layers; l0 += GEMM_MAXSEG / 2) {
    const int l1 = std::min(c.layers, l0 + GEMM_MAXSEG / 2);
    GemmCall kvc{EPI_STORE, XSRC_NORM, {}, c.hidden, fc_out, c.hidden, ctx->enc_norm,
                 kv + (size_t)l0 * 2 * kvd, kv_cols, nullptr};
    kvc.split = g.bf;
    for (int l = l0; l < l1; ++l) {
      kvc.segs.push_back(seg(ctx->layers[l].k, (l - l0) * 2 * kvd, kvd));
      kvc.segs.push_back(seg(ctx->layers[l].v, (l - l0) * 2 * kvd + kvd, kvd));
    }
    const dflash_status s = run_gemm(ctx, kvc, rc, st);
    if (s != DFLASH_OK) return s;
  }
  return DFLASH_OK;
}

// k_norm, RoPE and the cache-dtype cast of n rows of app_kv starting at row r0, at positions
// pos.., into `ring`
dflash_status ring_write_rows(dflash_ctx* ctx, int r0, int n, int64_t pos, unsigned char* ring, hipStream_t st) {
  const Cfg& g = ctx->cfg;
  const size_t kv_cols = (size_t)g.c.layers * 2 * g.c.kv_heads * g.c.head_dim;
  const float* kv = (const float*)(ctx->ws + ctx->lay.app_kv) + (size_t)r0 * kv_cols;
  return dev(ctx, launch_ring_write(g.bf, g.a, kv, (const void* const*)(ctx->ws + ctx->lay.knorm_ptrs), n, pos, ring,
                                    st),
             "ring write");
}

dflash_status project_kv(dflash_ctx* ctx, int rc, int64_t pos, hipStream_t st) {
  const dflash_status s = kv_gemms(ctx, rc, st);
  return s != DFLASH_OK ? s : ring_write_rows(ctx, 0, rc, pos, ctx->ring, st);
}

// the deferred rows' K/V into the ring now
dflash_status flush_kv(dflash_ctx* ctx, hipStream_t st) {
  if (ctx->kv_rows <= 0) return DFLASH_OK;
  const dflash_status s = project_kv(ctx, ctx->kv_rows, ctx->kv_pos, st);
  if (s == DFLASH_OK) ctx->kv_rows = 0;
  return s;
}

// Bound on the per-work-group key bytes of one vocabulary argmax launch over rows given in
// the activation dtype (at most 48 rows per launch over bf16 or 4-bit weights, 32 over f32;
// fewer tiles per work-group, so more work-groups, at fewer rows).
size_t argmax_key_bytes(const Cfg& g, int n) {
  const int ntiles = g.c.vocab / 16;
  size_t most = 0;
  // the largest launch of n rows, and the largest of 16 rows or fewer (more work-groups)
  for (const int rc : {std::min(n, g.bf ? GEMM_MAX_ROWS : 32), std::min(n, 16)}) {
    const int tpw = argmax_tiles_per_wg(g.wt, 0, ntiles, rc);
    most = std::max(most, (size_t)rc * (size_t)((ntiles + tpw - 1) / tpw) * sizeof(unsigned long long));
  }
  return most;
}

}  // namespace

namespace dflash {

// dflash_lm_head_argmax with the per-work-group argmax keys in `keys` (keys_bytes long) in
// place of the context's workspace; nothing is enqueued unless every launch fits.
dflash_status lm_head_argmax_into(dflash_ctx* ctx, const void* rows, int32_t n, int32_t* d_idx,
                                  unsigned long long* keys, size_t keys_bytes, hipStream_t st) {
  if (!ctx) return DFLASH_E_ARG;
  if (!rows || !d_idx) return fail(ctx, DFLASH_E_ARG, "NULL rows or output");
  if (n < 1 || n > 4096) return fail(ctx, DFLASH_E_RANGE, "row count %d outside 1..4096", n);
  if (!keys) return fail(ctx, DFLASH_E_DEVICE, "no argmax key scratch on this device");
  const size_t need = argmax_key_bytes(ctx->cfg, n);
  if (need > keys_bytes)
    return fail(ctx, DFLASH_E_SHAPE, "vocabulary %d needs %zu bytes of argmax keys, above the %zu-byte scratch",
                ctx->cfg.c.vocab, need, keys_bytes);
  const dflash_config& c = ctx->cfg.c;
  GemmCall lm{EPI_ARGMAX, XSRC_LDS, {seg(ctx->lm_head, 0, c.vocab)}, c.hidden, rows, c.hidden, nullptr, nullptr, 0,
              d_idx};
  lm.part = keys;
  lm.part_bytes = keys_bytes;
  return run_gemm(ctx, lm, n, st);
}

dflash_status noalloc_keys_for_call(dflash_ctx* ctx, unsigned long long** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != ctx->device)
    return fail(ctx, DFLASH_E_ARG, "the context's device %d is not current", ctx->device);
  if (!ctx->noalloc_keys) return fail(ctx, DFLASH_E_DEVICE, "no argmax key array on device %d", ctx->device);
  *out = ctx->noalloc_keys;
  return DFLASH_OK;
}

}  // namespace dflash

// ======================================================================================
extern "C" {

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_E_ARG: return "bad argument";
    case DFLASH_E_SHAPE: return "bad shape";
    case DFLASH_E_RANGE: return "value out of range";
    case DFLASH_E_NO_CONTEXT: return "no committed context";
    case DFLASH_E_REWIND: return "illegal rewind";
    case DFLASH_E_STATE: return "uncommitted rows pending";
    case DFLASH_E_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* dflash_last_error(const dflash_ctx* ctx) { return ctx ? ctx->err : g_create_err; }

dflash_status dflash_query_sizes(const dflash_config* cfg, size_t* ring_bytes, size_t* workspace_bytes,
                                 size_t* packed_bytes) {
  Cfg g;
  dflash_status s = check_cfg(cfg, &g, g_create_err);
  if (s != DFLASH_OK) return s;
  if (!ring_bytes || !workspace_bytes || !packed_bytes) return cfg_fail(g_create_err, DFLASH_E_ARG, "NULL size output");
  *ring_bytes = ring_bytes_of(g);
  *workspace_bytes = make_layout(g).total;
  *packed_bytes = make_packed_layout(g).total;
  return DFLASH_OK;
}

}  // extern "C"

namespace {

// Binds a context to validated buffers and weights and initialises it on `st` (the body of
// dflash_create, shared with the batch context): packs every linear, fills the k_norm
// table, zero-fills the first ring_need ring bytes and synchronises the stream. fold_rows:
// whether committed rows' K/V may travel with the next draft.
dflash_status init_engine(dflash_ctx* ctx, const Cfg& g, const dflash_weights* wts, void* ring, size_t ring_need,
                          size_t ring_bytes, void* workspace, size_t workspace_bytes, void* packed,
                          size_t packed_bytes, bool fold_rows, hipStream_t st) {
  if (!wts || !wts->layers) return cfg_fail(g_create_err, DFLASH_E_ARG, "weights or layer array is NULL");
  if (!ring || !workspace || !packed) return cfg_fail(g_create_err, DFLASH_E_ARG, "ring, workspace or packed is NULL");
  if (((uintptr_t)ring & 255u) || ((uintptr_t)workspace & 255u) || ((uintptr_t)packed & 255u))
    return cfg_fail(g_create_err, DFLASH_E_ARG, "ring, workspace and packed must be 256-byte aligned");
  const Layout lay = make_layout(g);
  const PackedLayout pk = make_packed_layout(g);
  if (ring_bytes < ring_need || workspace_bytes < lay.total || packed_bytes < pk.total)
    return cfg_fail(g_create_err, DFLASH_E_SHAPE, "ring, workspace or packed smaller than the queried sizes");
  auto lin_ok = [&](const dflash_linear& l) {
    if (!l.w || !aligned16(l.w)) return false;
    if (g.wt == WT_Q4) return l.scales && l.biases && ((uintptr_t)l.scales & 1u) == 0 && ((uintptr_t)l.biases & 1u) == 0;
    return true;
  };
  // norm gains are read 16 bytes at a time
  auto gain_ok = [&](const void* p) { return p && aligned16(p); };
  if (!wts->embed || !gain_ok(wts->enc_norm) || !gain_ok(wts->final_norm) || !lin_ok(wts->lm_head) || !lin_ok(wts->fc))
    return cfg_fail(g_create_err, DFLASH_E_ARG, "a top-level weight is NULL or not 16-byte aligned");
  for (int l = 0; l < g.c.layers; ++l) {
    const dflash_layer& L = wts->layers[l];
    if (!lin_ok(L.q) || !lin_ok(L.k) || !lin_ok(L.v) || !lin_ok(L.o) || !lin_ok(L.gate) || !lin_ok(L.up) ||
        !lin_ok(L.down) || !gain_ok(L.in_norm) || !gain_ok(L.post_norm) || !gain_ok(L.q_norm) || !gain_ok(L.k_norm))
      return cfg_fail(g_create_err, DFLASH_E_ARG, "layer %d has a NULL or misaligned weight", l);
  }
  // the Markov factors are read 16 bytes per lane in place
  if (g.dspark ? !gain_ok(wts->markov_w1) || !gain_ok(wts->markov_w2) : wts->markov_w1 || wts->markov_w2)
    return cfg_fail(g_create_err, DFLASH_E_ARG,
                    g.dspark ? "the Markov factors are NULL or not 16-byte aligned"
                             : "Markov factors given to a DFlash context");
  ctx->cfg = g;
  ctx->lay = lay;
  ctx->fold_rows = fold_rows ? fold_rows_of(g) : 0;
  auto cv = [](const dflash_linear& l) { return Lin{l.w, l.scales, l.biases}; };
  ctx->lm_head = cv(wts->lm_head);
  ctx->fc = cv(wts->fc);
  ctx->embed = wts->embed;
  ctx->enc_norm = wts->enc_norm;
  ctx->final_norm = wts->final_norm;
  ctx->markov_w1 = wts->markov_w1;
  ctx->markov_w2 = wts->markov_w2;
  ctx->layers.resize(g.c.layers);
  std::vector<const void*> knorms(g.c.layers);
  for (int l = 0; l < g.c.layers; ++l) {
    const dflash_layer& L = wts->layers[l];
    ctx->layers[l] = Layer{cv(L.q), cv(L.k), cv(L.v), cv(L.o), cv(L.gate), cv(L.up), cv(L.down),
                           L.in_norm, L.post_norm, L.q_norm, L.k_norm};
    knorms[l] = L.k_norm;
  }
  ctx->ring = (unsigned char*)ring;
  ctx->ws = (unsigned char*)workspace;
  hipError_t e = hipGetDevice(&ctx->device);
  {
    int cus = 0;
    if (e == hipSuccess && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, ctx->device) == hipSuccess &&
        cus > 0)
      ctx->cus = cus;
  }
  if (g.dspark) ctx->mk_groups = markov_step_groups(g.c.vocab, g.c.markov_rank, g.bf, ctx->cus);
  // the device address of this device's fixed argmax key array, for the allocation-free argmax
  if (e == hipSuccess) {
    void* keys = nullptr;
    e = noalloc_scratch_address(ctx->device, &keys);
    ctx->noalloc_keys = (unsigned long long*)keys;
  }
  // repack every linear into fragment-major blocks; the context reads only the packed copies
  {
    const dflash_config& c = g.c;
    const int H = c.hidden, qd = c.q_heads * c.head_dim, kvd = c.kv_heads * c.head_dim;
    const int F = c.target_streams * c.target_width, I = c.intermediate;
    unsigned char* base = (unsigned char*)packed;
    size_t idx = 0;
    // adjacent-pair RoPE: q and k rows (and their norm gains) in deinterleaved order per head
    auto pack = [&](Lin& l, int N, int K, int perm_hd = 0) {
      unsigned char* dst = base + pk.off[idx++];
      if (g.wt == WT_Q4) {
        unsigned char* sdst = dst + q4_code_bytes(N, K);
        if (e == hipSuccess) e = launch_pack_q4(l.w, l.s, l.b, N, K, dst, sdst, st, perm_hd);
        l.s = sdst;
        l.b = nullptr;
      } else if (e == hipSuccess) {
        e = launch_pack(g.wt, l.w, N, K, dst, st, perm_hd);
      }
      l.w = dst;
    };
    const int perm = g.trad ? c.head_dim : 0;
    pack(ctx->fc, H, F);
    pack(ctx->lm_head, c.vocab, H);
    for (int l = 0; l < c.layers; ++l) {
      Layer& L = ctx->layers[l];
      pack(L.q, qd, H, perm);
      pack(L.k, kvd, H, perm);
      pack(L.v, kvd, H);
      pack(L.o, H, qd);
      pack(L.gate, I, H);
      pack(L.up, I, H);
      pack(L.down, H, I);
      if (g.trad) {
        unsigned char* qn = base + pk.gains + pk.gain_stride * 2 * l;
        unsigned char* kn = qn + pk.gain_stride;
        const int gelt = g.wt == WT_F32 ? 4 : 2;
        if (e == hipSuccess) e = launch_deinterleave(L.q_norm, qn, c.head_dim, gelt, st);
        if (e == hipSuccess) e = launch_deinterleave(L.k_norm, kn, c.head_dim, gelt, st);
        L.q_norm = qn;
        L.k_norm = kn;
        knorms[l] = kn;
      }
    }
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(ctx->ws + lay.knorm_ptrs, knorms.data(), sizeof(void*) * knorms.size(),
                       hipMemcpyHostToDevice, st);
  // every slot starts finite (zero): attention reads whole aligned runs of slots, including
  // keys outside a query's window that then get weight 0
  if (e == hipSuccess) e = hipMemsetAsync(ring, 0, ring_need, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host copy source dies with this call
  if (e != hipSuccess) return cfg_fail(g_create_err, DFLASH_E_DEVICE, "workspace init: %s", hipGetErrorString(e));
  return DFLASH_OK;
}


}  // namespace

extern "C" {

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* wts, void* ring, size_t ring_bytes,
                            void* workspace, size_t workspace_bytes, void* packed, size_t packed_bytes, void* stream,
                            dflash_ctx** out) {
  g_create_err[0] = 0;
  if (!out) return cfg_fail(g_create_err, DFLASH_E_ARG, "NULL output handle");
  *out = nullptr;
  Cfg g;
  dflash_status s = check_cfg(cfg, &g, g_create_err);
  if (s != DFLASH_OK) return s;
  dflash_ctx* ctx = new (std::nothrow) dflash_ctx();
  if (!ctx) return cfg_fail(g_create_err, DFLASH_E_ARG, "out of host memory");
  s = init_engine(ctx, g, wts, ring, ring_bytes_of(g), ring_bytes, workspace, workspace_bytes, packed, packed_bytes,
                  true, (hipStream_t)stream);
  if (s != DFLASH_OK) {
    delete ctx;
    return s;
  }
  *out = ctx;
  return DFLASH_OK;
}

void dflash_destroy(dflash_ctx* ctx) { delete ctx; }

dflash_status dflash_cache_state(const dflash_ctx* ctx, int64_t* e, int32_t* pending, int32_t* slack,
                                 int32_t* capacity) {
  if (!ctx) return DFLASH_E_ARG;
  if (e) *e = ctx->e;
  if (pending) *pending = (int32_t)ctx->pending;
  if (slack) *slack = (int32_t)ctx->cfg.S;
  if (capacity) *capacity = (int32_t)ctx->cfg.C;
  return DFLASH_OK;
}

dflash_status dflash_cache_trim(dflash_ctx* ctx, int32_t m) {
  if (!ctx) return DFLASH_E_ARG;
  if (m < 0 || m > ctx->pending || m > ctx->cfg.S)
    return fail(ctx, DFLASH_E_REWIND, "rewind of %d rows with %lld pending and slack %lld", m,
                (long long)ctx->pending, (long long)ctx->cfg.S);
  ctx->e += ctx->pending - m;
  ctx->pending = 0;
  // deferred rows past the new end are dropped with the rest
  if (ctx->kv_rows > 0)
    ctx->kv_rows = (int32_t)std::max<int64_t>(0, std::min<int64_t>(ctx->kv_rows, ctx->e - ctx->kv_pos));
  return DFLASH_OK;
}

dflash_status dflash_cache_append(dflash_ctx* ctx, const void* resid, int32_t n, int32_t commit, void* stream) {
  if (!ctx) return DFLASH_E_ARG;
  if (!resid || n <= 0) return fail(ctx, DFLASH_E_ARG, "append of %d rows: no residual stream captured", n);
  const Cfg& g = ctx->cfg;
  const dflash_config& c = g.c;
  hipStream_t st = (hipStream_t)stream;
  dflash_status s = flush_kv(ctx, st);
  if (s != DFLASH_OK) return s;
  const int64_t start = ctx->e + ctx->pending, end = start + n;
  const int64_t keep_from = commit ? end - c.window : end - g.C;
  const int64_t first = std::max<int64_t>(0, keep_from - start);
  const int64_t F = (int64_t)c.target_streams * c.target_width;
  // a few uncommitted rows (the verified rows of a round) are deferred: encoder rows now,
  // their K/V with the next draft's QKV launches (at least two draft rows beside them)
  const bool defer = !commit && first == 0 && n + 2 <= ctx->fold_rows && n <= c.window;
  for (int64_t r0 = first; r0 < n; r0 += GEMM_MAX_ROWS) {
    const int rc = (int)std::min<int64_t>(GEMM_MAX_ROWS, n - r0);
    float* fc_out = (float*)(ctx->ws + ctx->lay.app_fc);
    GemmCall f{EPI_STORE, XSRC_GLOBAL, {seg(ctx->fc, 0, c.hidden)}, (int)F,
               (const unsigned char*)resid + (size_t)r0 * F * g.act_elt, F, nullptr, fc_out, c.hidden, nullptr};
    s = run_gemm(ctx, f, rc, st);
    if (s != DFLASH_OK) return s;
    if (!defer) {
      s = project_kv(ctx, rc, start + r0, st);
      if (s != DFLASH_OK) return s;
    }
  }
  if (defer) {
    ctx->kv_pos = start;
    ctx->kv_rows = n;
  }
  if (commit) {
    ctx->e = end;
    ctx->pending = 0;
  } else {
    ctx->pending += n;
  }
  return DFLASH_OK;
}

dflash_status dflash_draft_block(dflash_ctx* ctx, int32_t anchor, int32_t block, int32_t* d_tokens, float* d_hidden,
                                 void* stream) {
  if (!ctx) return DFLASH_E_ARG;
  const Cfg& g = ctx->cfg;
  const dflash_config& c = g.c;
  if (block < 1 || block > c.max_block) return fail(ctx, DFLASH_E_RANGE, "block %d outside 1..%d", block, c.max_block);
  if (anchor < 0 || anchor >= c.vocab) return fail(ctx, DFLASH_E_RANGE, "anchor %d outside [0, %d)", anchor, c.vocab);
  if (!d_tokens) return fail(ctx, DFLASH_E_ARG, "NULL token output");
  if (ctx->e <= 0) return fail(ctx, DFLASH_E_NO_CONTEXT, "draft with an empty context");
  if (ctx->pending) return fail(ctx, DFLASH_E_STATE, "%lld appended rows are not committed", (long long)ctx->pending);
  // DSpark attends to every context row; the window rule agrees while it cuts nothing
  if (g.dspark && ctx->e + block - 1 > c.window)
    return fail(ctx, DFLASH_E_RANGE, "DSpark block at context %lld + %d rows reaches past the window %d",
                (long long)ctx->e, block, c.window);
  hipStream_t st = (hipStream_t)stream;
  const int R = g.dspark ? block : block + 1;  // DSpark: [anchor, mask x (gamma-1)]
  const int H = c.hidden;
  // committed rows whose K/V are deferred: projected with this draft's QKV launches (rows
  // R..R+nf-1) and written into the ring by its attention, or first on their own
  int nf = ctx->kv_rows;
  if (nf > 0 && (R + nf > ctx->fold_rows || ctx->kv_pos + nf != ctx->e)) {
    const dflash_status s0 = flush_kv(ctx, st);
    if (s0 != DFLASH_OK) return s0;
    nf = 0;
  }
  const int qd = c.q_heads * c.head_dim, kvd = c.kv_heads * c.head_dim;
  float* x = (float*)(ctx->ws + ctx->lay.x);
  float* qkv = (float*)(ctx->ws + ctx->lay.qkv);
  void* qb = ctx->ws + ctx->lay.qb;
  void* attn = ctx->ws + ctx->lay.attn;
  void* mlp = ctx->ws + ctx->lay.mlp;
  void* qb_lo = lo_plane(g, qb, g.R, qd);
  void* attn_lo = lo_plane(g, attn, g.R, qd);
  void* mlp_lo = lo_plane(g, mlp, g.R, c.intermediate);
  float* part = (float*)(ctx->ws + ctx->lay.part);
  const size_t ring_layer = (size_t)g.act_elt * 2 * c.kv_heads * (size_t)g.Cs * c.head_dim;

  // the proposing rows' operands of the lm_head (DFlash: rows 1..B; DSpark: all gamma rows)
  void* zrows = ctx->ws + ctx->lay.zrows;
  void* zrows_lo = lo_plane(g, zrows, block, H);
  float2* rope = (float2*)(ctx->ws + ctx->lay.rope);
  dflash_status s = dev(ctx,
                        launch_embed(g.bf, ctx->embed, H, c.vocab, anchor, c.mask_token_id, nullptr, R, nf,
                                     (const float*)(ctx->ws + ctx->lay.app_fc), x, rope, ctx->e, c.rope_theta,
                                     c.head_dim, st),
                        "embed");
  if (s != DFLASH_OK) return s;
  for (int l = 0; l < c.layers; ++l) {
    const Layer& L = ctx->layers[l];
    GemmCall q{EPI_STORE, XSRC_NORM, {seg(L.q, 0, qd), seg(L.k, qd, kvd), seg(L.v, qd + kvd, kvd)}, H, x, H,
               L.in_norm, qkv, qd + 2 * kvd, nullptr};
    q.split = g.bf;
    if (nf > 0) {  // the committed encoder rows behind the draft rows (copied by the embedding)
      q.gain2 = ctx->enc_norm;
      q.r2 = R;
    }
    if ((s = run_gemm(ctx, q, R + nf, st)) != DFLASH_OK) return s;
    s = dev(ctx,
            launch_block_attention(g.bf, g.a, qkv, L.q_norm, L.k_norm, rope, ctx->ring + l * ring_layer, R, nf,
                                   ctx->e, qb, qb_lo, part, attn, attn_lo, st),
            "attention");
    if (s != DFLASH_OK) return s;
    GemmCall o{EPI_RESID, XSRC_GLOBAL, {seg(L.o, 0, H)}, qd, attn, qd, nullptr, x, H, nullptr};
    o.split = g.bf;
    o.xlo = attn_lo;
    if ((s = run_gemm(ctx, o, R, st)) != DFLASH_OK) return s;
    GemmCall gu{EPI_SWIGLU, XSRC_NORM, {seg(L.gate, 0, c.intermediate), seg(L.up, 0, c.intermediate)}, H, x, H,
                L.post_norm, mlp, c.intermediate, nullptr};
    gu.split = g.bf;
    gu.ylo = mlp_lo;
    if ((s = run_gemm(ctx, gu, R, st)) != DFLASH_OK) return s;
    GemmCall dn{EPI_RESID, XSRC_GLOBAL, {seg(L.down, 0, H)}, c.intermediate, mlp, c.intermediate, nullptr, x, H,
                nullptr};
    dn.split = g.bf;
    dn.xlo = mlp_lo;
    if (!g.dspark && l == c.layers - 1) gain_rows_for_argmax(ctx, dn, zrows, zrows_lo, R);
    if ((s = run_gemm(ctx, dn, R, st)) != DFLASH_OK) return s;
  }
  ctx->kv_rows = 0;  // every layer's ring now holds them
  if (d_hidden) {
    s = dev(ctx, hipMemcpyAsync(d_hidden, x, sizeof(float) * R * H, hipMemcpyDeviceToDevice, st), "hidden copy");
    if (s != DFLASH_OK) return s;
  }
  if (!g.dspark) {  // the last down launch left rows 1..B times the final norm's gain
    GemmCall lm{EPI_ARGMAX, XSRC_LDS, {seg(ctx->lm_head, 0, c.vocab)}, H, zrows, H, nullptr, nullptr, 0, d_tokens};
    lm.split = g.bf;
    lm.xlo = zrows_lo;
    return run_gemm(ctx, lm, block, st);
  }
  // DSpark: the final RMSNorm of all gamma rows (their logits are scored, not only ranked),
  // every row's f32 logits, then the Markov chain: one launch per step, each taking
  // its token from the keys the previous step left (the anchor first) and storing it as the
  // previous step's output, then the reduction of the last step's keys
  // (the vocabulary argmax GEMM with its logit store: the store GEMM's folded 8-column
  // tiles measured 192 / 317 us against 122 us at 7 / 9 rows)
  s = dev(ctx, launch_rownorm(g.bf, x, ctx->final_norm, c.rms_eps, block, H, zrows, zrows_lo, st), "final norm");
  if (s != DFLASH_OK) return s;
  float* logits = (float*)(ctx->ws + ctx->lay.logits);
  GemmCall lm{EPI_ARGMAX, XSRC_LDS, {seg(ctx->lm_head, 0, c.vocab)}, H, zrows, H, nullptr, logits, c.vocab, nullptr};
  lm.split = g.bf;
  lm.xlo = zrows_lo;
  if ((s = run_gemm(ctx, lm, block, st)) != DFLASH_OK) return s;
  unsigned long long* keys[2] = {(unsigned long long*)(ctx->ws + ctx->lay.mk_part),
                                 (unsigned long long*)(ctx->ws + ctx->lay.mk_part) + MK_MAX_GROUPS};
  const int ng = ctx->mk_groups;
  hipEvent_t cs = ctx->cev_start, ce = ctx->cev_end;
  ctx->cev_start = ctx->cev_end = nullptr;
  if (cs && (s = dev(ctx, hipEventRecord(cs, st), "timing event")) != DFLASH_OK) return s;
  for (int i = 0; i < block; ++i) {
    s = dev(ctx,
            launch_markov_step(g.bf, c.markov_rank, ctx->markov_w1, ctx->markov_w2, c.vocab,
                               logits + (size_t)i * c.vocab, i ? keys[(i - 1) & 1] : nullptr, ng, anchor,
                               i ? d_tokens + i - 1 : nullptr, keys[i & 1], ng, st),
            "markov step");
    if (s != DFLASH_OK) return s;
  }
  s = dev(ctx, launch_argmax_finalize(keys[(block - 1) & 1], ng, 1, d_tokens + block - 1, st), "markov finish");
  if (s != DFLASH_OK) return s;
  if (ce) return dev(ctx, hipEventRecord(ce, st), "timing event");
  return DFLASH_OK;
}

dflash_status dflash_lm_head_argmax(dflash_ctx* ctx, const void* rows, int32_t n, int32_t* d_idx, void* stream) {
  if (!ctx) return DFLASH_E_ARG;
  if (!rows || !d_idx) return fail(ctx, DFLASH_E_ARG, "NULL rows or output");
  if (n < 1 || n > 4096) return fail(ctx, DFLASH_E_RANGE, "row count %d outside 1..4096", n);
  const dflash_config& c = ctx->cfg.c;
  GemmCall lm{EPI_ARGMAX, XSRC_LDS, {seg(ctx->lm_head, 0, c.vocab)}, c.hidden, rows, c.hidden, nullptr, nullptr, 0,
              d_idx};
  ctx->tev_active = ctx->tev_start != nullptr;
  const dflash_status s = run_gemm(ctx, lm, n, (hipStream_t)stream);
  ctx->tev_active = false;
  ctx->tev_start = ctx->tev_end = nullptr;
  return s;
}

dflash_status dflash_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t groups, void* stream) {
  if (!src || !sink || groups < 1 || ((uintptr_t)src & 15u) || bytes % 16 || bytes / 16 < (size_t)groups * 256)
    return cfg_fail(g_create_err, DFLASH_E_ARG, "probe needs a 16-byte aligned source of at least groups * 4096 bytes");
  const hipError_t e = launch_hbm_read_probe(src, bytes, sink, groups, (hipStream_t)stream);
  if (e != hipSuccess) return cfg_fail(g_create_err, DFLASH_E_DEVICE, "probe launch: %s", hipGetErrorString(e));
  return DFLASH_OK;
}

dflash_status dflash_time_next_argmax(dflash_ctx* ctx, void* start, void* end) {
  if (!ctx) return DFLASH_E_ARG;
  if ((start == nullptr) != (end == nullptr)) return fail(ctx, DFLASH_E_ARG, "give both timing events or neither");
  ctx->tev_start = (hipEvent_t)start;
  ctx->tev_end = (hipEvent_t)end;
  return DFLASH_OK;
}

dflash_status dflash_time_next_chain(dflash_ctx* ctx, void* start, void* end) {
  if (!ctx) return DFLASH_E_ARG;
  if ((start == nullptr) != (end == nullptr)) return fail(ctx, DFLASH_E_ARG, "give both timing events or neither");
  if (!ctx->cfg.dspark) return fail(ctx, DFLASH_E_ARG, "a DFlash context has no Markov chain");
  ctx->cev_start = (hipEvent_t)start;
  ctx->cev_end = (hipEvent_t)end;
  return DFLASH_OK;
}

dflash_status dflash_verify_greedy(dflash_ctx* ctx, const int32_t* d_draft, const int32_t* d_target, int32_t block,
                                   int32_t* d_out, void* stream) {
  if (!ctx) return DFLASH_E_ARG;
  if (!d_draft || !d_target || !d_out) return fail(ctx, DFLASH_E_ARG, "NULL verify buffer");
  if (block < 1 || block > ctx->cfg.c.max_block)
    return fail(ctx, DFLASH_E_RANGE, "block %d outside 1..%d", block, ctx->cfg.c.max_block);
  return dev(ctx, launch_verify(d_draft, d_target, block, ctx->cfg.c.vocab, d_out, (hipStream_t)stream), "verify");
}

dflash_status dflash_cache_read(dflash_ctx* ctx, int32_t layer, void* k_out, void* v_out, int32_t* n_out,
                                void* stream) {
  if (!ctx) return DFLASH_E_ARG;
  const Cfg& g = ctx->cfg;
  if (layer < 0 || layer >= g.c.layers) return fail(ctx, DFLASH_E_RANGE, "layer %d outside 0..%d", layer, g.c.layers - 1);
  if (!n_out || !k_out || !v_out) return fail(ctx, DFLASH_E_ARG, "NULL count or window output");
  const int64_t lo = std::max<int64_t>(0, ctx->e - g.c.window);
  const int n = (int)(ctx->e - lo);
  if (n == 0) {
    *n_out = 0;
    return DFLASH_OK;
  }
  const dflash_status s = flush_kv(ctx, (hipStream_t)stream);
  if (s != DFLASH_OK) return s;
  *n_out = n;
  const size_t ring_layer = (size_t)g.act_elt * 2 * g.c.kv_heads * (size_t)g.Cs * g.c.head_dim;
  return dev(ctx,
             launch_cache_read(g.bf, g.a, ctx->ring + layer * ring_layer, lo, n, k_out, v_out, (hipStream_t)stream,
                               g.trad ? 1 : 0),
             "cache read");
}

}  // extern "C"

// ======================================================================================
// The target's verify forward (dflash_target_*). A target context embeds a drafter-style
// engine (`core`): the same GEMM driver, packed-weight layout, workspace layout and launch
// plans, with the target's layers in place of the drafter's; per layer its own cache (a
// sliding ring of window + slack slots, or a full-attention buffer of max_context slots) and
// attention shape (causal: the block's own keys and values become cache rows).
// ======================================================================================

struct dflash_target {
  dflash_ctx core;
  dflash_target_config tc;
  int R = 0;                      // rows per forward at most
  std::vector<AttnShape> shape;   // per layer
  std::vector<size_t> cache_off;  // per layer byte offset of its K [nkv][cap][hd] and V^T [nkv][hd][cap]
  std::vector<int> capture_slot;  // per layer: its place in the captured row, or -1
  size_t cache_total = 0;
  bool has_full = false;
};

namespace {

constexpr int TARGET_MAX_BLOCK = 64;
constexpr int TARGET_CHUNK_ROWS = 32;  // rows of a prompt chunk a forward may take

bool target_full(const dflash_target_config& c, int l) { return l < 64 && ((c.full_mask >> l) & 1ull); }

// Validate the target config and derive the engine's Cfg plus per-layer shapes and offsets.
dflash_status check_target(const dflash_target_config* c, dflash_target* t, char* err) {
  if (!c) return cfg_fail(err, DFLASH_E_ARG, "target config is NULL");
  if (c->layers < 1 || c->layers > 64) return cfg_fail(err, DFLASH_E_SHAPE, "target layers must be 1..64");
  if (c->window < 1 || c->window > MAX_WINDOW) return cfg_fail(err, DFLASH_E_SHAPE, "window must be 1..%d", MAX_WINDOW);
  if (c->max_context < 64 || c->max_context > MAX_WINDOW)
    return cfg_fail(err, DFLASH_E_SHAPE, "max_context must be 64..%d", MAX_WINDOW);
  if (c->max_block < 1 || c->max_block > TARGET_MAX_BLOCK)
    return cfg_fail(err, DFLASH_E_RANGE, "target max_block must be 1..%d", TARGET_MAX_BLOCK);
  if (c->n_capture < 1 || c->n_capture > 8) return cfg_fail(err, DFLASH_E_SHAPE, "1..8 capture layers");
  for (int i = 0; i < c->n_capture; ++i)
    if (c->capture_layers[i] < 0 || c->capture_layers[i] >= c->layers || (i && c->capture_layers[i] <= c->capture_layers[i - 1]))
      return cfg_fail(err, DFLASH_E_SHAPE, "capture layers must be strictly increasing layer ids");
  const int R = std::max(c->max_block + 1, TARGET_CHUNK_ROWS);
  // the engine's shape: the drafter checks with fc = one stream of hidden (unused), the
  // widest attention span, and the rows of a forward
  dflash_config d{};
  d.hidden = c->hidden;
  d.layers = c->layers;
  d.q_heads = c->q_heads;
  d.kv_heads = c->kv_heads;
  d.head_dim = c->head_dim;
  d.intermediate = c->intermediate;
  d.vocab = c->vocab;
  d.target_streams = 1;
  d.target_width = c->hidden;
  d.window = std::max(c->window, c->max_context);
  d.max_block = R - 1;
  d.mask_token_id = 0;
  d.ring_phase = 0;
  d.rms_eps = c->rms_eps;
  d.rope_theta = c->rope_theta;
  d.weight_dtype = c->weight_dtype;
  d.act_dtype = c->act_dtype;
  Cfg g;
  const dflash_status s = check_cfg(&d, &g, err);
  if (s != DFLASH_OK) return s;
  g.S = slack_rows(c->max_block);  // the sliding caches' slack follows the verify block
  t->core.cfg = g;
  t->tc = *c;
  t->R = R;
  t->shape.assign(c->layers, g.a);
  t->cache_off.assign(c->layers, 0);
  t->capture_slot.assign(c->layers, -1);
  for (int i = 0; i < c->n_capture; ++i) t->capture_slot[c->capture_layers[i]] = i;
  size_t off = 0;
  for (int l = 0; l < c->layers; ++l) {
    AttnShape& a = t->shape[l];
    a.causal = 1;
    a.phase = 0;
    int64_t cap;
    if (target_full(*c, l)) {
      t->has_full = true;
      a.window = 1 << 30;  // past every distance
      cap = c->max_context;
    } else {
      a.window = c->window;
      cap = std::max<int64_t>({(int64_t)c->window + g.S, (int64_t)c->window + R, (int64_t)64});
    }
    a.cap = (int32_t)((cap + 7) & ~(int64_t)7);
    t->cache_off[l] = off;
    off = align256(off + (size_t)g.act_elt * 2 * c->kv_heads * (size_t)a.cap * c->head_dim);
  }
  t->cache_total = off;
  return DFLASH_OK;
}

Layout target_layout(const dflash_target* t) {
  Layout L = make_layout(t->core.cfg);
  // attention partials for the widest span: a full layer's whole context
  const Cfg& g = t->core.cfg;
  const size_t need = 4 * attention_partial_floats_span(g.a, t->R, t->tc.max_context);
  if (need > L.total - L.part) {
    L.part = L.total;
    L.total = align256(L.total + need);
  }
  return L;
}

size_t target_packed_bytes(const dflash_target* t, std::vector<size_t>* offs) {
  const Cfg& g = t->core.cfg;
  const dflash_target_config& c = t->tc;
  const int64_t H = c.hidden, qd = (int64_t)c.q_heads * c.head_dim, kvd = (int64_t)c.kv_heads * c.head_dim;
  size_t total = 0;
  auto add = [&](int64_t N, int64_t K) {
    if (offs) offs->push_back(total);
    total = align256(total + linear_bytes(g, N, K));
  };
  add(c.vocab, H);
  for (int l = 0; l < c.layers; ++l) {
    add(qd, H);
    add(kvd, H);
    add(kvd, H);
    add(H, qd);
    add(c.intermediate, H);
    add(c.intermediate, H);
    add(H, c.intermediate);
  }
  return total;
}

}  // namespace

extern "C" {

dflash_status dflash_target_query_sizes(const dflash_target_config* cfg, size_t* cache_bytes, size_t* workspace_bytes,
                                        size_t* packed_bytes) {
  dflash_target t;
  const dflash_status s = check_target(cfg, &t, g_create_err);
  if (s != DFLASH_OK) return s;
  if (!cache_bytes || !workspace_bytes || !packed_bytes) return cfg_fail(g_create_err, DFLASH_E_ARG, "NULL size output");
  *cache_bytes = t.cache_total;
  *workspace_bytes = target_layout(&t).total;
  *packed_bytes = target_packed_bytes(&t, nullptr);
  return DFLASH_OK;
}

dflash_status dflash_target_create(const dflash_target_config* cfg, const dflash_target_weights* wts, void* cache,
                                   size_t cache_bytes, void* workspace, size_t workspace_bytes, void* packed,
                                   size_t packed_bytes, void* stream, dflash_target** out) {
  g_create_err[0] = 0;
  if (!out) return cfg_fail(g_create_err, DFLASH_E_ARG, "NULL output handle");
  *out = nullptr;
  dflash_target* t = new (std::nothrow) dflash_target();
  if (!t) return cfg_fail(g_create_err, DFLASH_E_ARG, "out of host memory");
  auto bail = [&](dflash_status st) {
    delete t;
    return st;
  };
  dflash_status s = check_target(cfg, t, g_create_err);
  if (s != DFLASH_OK) return bail(s);
  if (!wts || !wts->layers || !wts->embed) return bail(cfg_fail(g_create_err, DFLASH_E_ARG, "weights, layers or embed NULL"));
  if (!cache || !workspace || !packed) return bail(cfg_fail(g_create_err, DFLASH_E_ARG, "cache, workspace or packed is NULL"));
  if (((uintptr_t)cache & 255u) || ((uintptr_t)workspace & 255u) || ((uintptr_t)packed & 255u))
    return bail(cfg_fail(g_create_err, DFLASH_E_ARG, "cache, workspace and packed must be 256-byte aligned"));
  const Layout lay = target_layout(t);
  std::vector<size_t> poff;
  const size_t pk = target_packed_bytes(t, &poff);
  if (cache_bytes < t->cache_total || workspace_bytes < lay.total || packed_bytes < pk)
    return bail(cfg_fail(g_create_err, DFLASH_E_SHAPE, "cache, workspace or packed smaller than the queried sizes"));
  const Cfg& g = t->core.cfg;
  auto lin_ok = [&](const dflash_linear& l) {
    if (!l.w || !aligned16(l.w)) return false;
    if (g.wt == WT_Q4) return l.scales && l.biases;
    return true;
  };
  auto gain_ok = [&](const void* p) { return p && aligned16(p); };
  if (!lin_ok(wts->lm_head) || !gain_ok(wts->final_norm))
    return bail(cfg_fail(g_create_err, DFLASH_E_ARG, "lm_head or final_norm NULL or misaligned"));
  for (int l = 0; l < g.c.layers; ++l) {
    const dflash_layer& L = wts->layers[l];
    if (!lin_ok(L.q) || !lin_ok(L.k) || !lin_ok(L.v) || !lin_ok(L.o) || !lin_ok(L.gate) || !lin_ok(L.up) ||
        !lin_ok(L.down) || !gain_ok(L.in_norm) || !gain_ok(L.post_norm) || !gain_ok(L.q_norm) || !gain_ok(L.k_norm))
      return bail(cfg_fail(g_create_err, DFLASH_E_ARG, "target layer %d has a NULL or misaligned weight", l));
  }
  dflash_ctx& ctx = t->core;
  ctx.lay = lay;
  ctx.ws = (unsigned char*)workspace;
  ctx.ring = (unsigned char*)cache;
  ctx.embed = wts->embed;
  ctx.final_norm = wts->final_norm;
  auto cv = [](const dflash_linear& l) { return Lin{l.w, l.scales, l.biases}; };
  ctx.lm_head = cv(wts->lm_head);
  ctx.layers.resize(g.c.layers);
  for (int l = 0; l < g.c.layers; ++l) {
    const dflash_layer& L = wts->layers[l];
    ctx.layers[l] = Layer{cv(L.q), cv(L.k), cv(L.v), cv(L.o), cv(L.gate), cv(L.up), cv(L.down),
                          L.in_norm, L.post_norm, L.q_norm, L.k_norm};
  }
  hipError_t e = hipGetDevice(&ctx.device);
  hipStream_t st = (hipStream_t)stream;
  {
    const dflash_config& c = g.c;
    const int H = c.hidden, qd = c.q_heads * c.head_dim, kvd = c.kv_heads * c.head_dim, I = c.intermediate;
    unsigned char* base = (unsigned char*)packed;
    size_t idx = 0;
    auto pack = [&](Lin& l, int N, int K) {
      unsigned char* dst = base + poff[idx++];
      if (g.wt == WT_Q4) {
        unsigned char* sdst = dst + q4_code_bytes(N, K);
        if (e == hipSuccess) e = launch_pack_q4(l.w, l.s, l.b, N, K, dst, sdst, st);
        l.s = sdst;
        l.b = nullptr;
      } else if (e == hipSuccess) {
        e = launch_pack(g.wt, l.w, N, K, dst, st);
      }
      l.w = dst;
    };
    pack(ctx.lm_head, c.vocab, H);
    for (int l = 0; l < c.layers; ++l) {
      Layer& L = ctx.layers[l];
      pack(L.q, qd, H);
      pack(L.k, kvd, H);
      pack(L.v, kvd, H);
      pack(L.o, H, qd);
      pack(L.gate, I, H);
      pack(L.up, I, H);
      pack(L.down, H, I);
    }
  }
  // every slot starts finite (zero): attention reads whole aligned runs of slots
  if (e == hipSuccess) e = hipMemsetAsync(cache, 0, t->cache_total, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return bail(cfg_fail(g_create_err, DFLASH_E_DEVICE, "target init: %s", hipGetErrorString(e)));
  *out = t;
  return DFLASH_OK;
}

void dflash_target_destroy(dflash_target* t) { delete t; }

const char* dflash_target_last_error(const dflash_target* t) { return t ? t->core.err : g_create_err; }

dflash_status dflash_target_forward(dflash_target* t, int32_t anchor, const int32_t* d_tokens, int32_t n,
                                    int32_t* d_argmax, void* d_capture, void* stream) {
  if (!t) return DFLASH_E_ARG;
  dflash_ctx* ctx = &t->core;
  const Cfg& g = ctx->cfg;
  const dflash_config& c = g.c;
  const dflash_target_config& tc = t->tc;
  if (n < 1 || n > t->R) return fail(ctx, DFLASH_E_RANGE, "forward of %d rows outside 1..%d", n, t->R);
  if (anchor < 0 || anchor >= c.vocab) return fail(ctx, DFLASH_E_RANGE, "anchor %d outside [0, %d)", anchor, c.vocab);
  if (!d_argmax || (n > 1 && !d_tokens)) return fail(ctx, DFLASH_E_ARG, "NULL argmax output or block tokens");
  if (ctx->pending) return fail(ctx, DFLASH_E_STATE, "%lld rows pending: trim first", (long long)ctx->pending);
  if (t->has_full && ctx->e + n > tc.max_context)
    return fail(ctx, DFLASH_E_RANGE, "positions past max_context %d", tc.max_context);
  hipStream_t st = (hipStream_t)stream;
  const int R = n, H = c.hidden;
  const int qd = c.q_heads * c.head_dim, kvd = c.kv_heads * c.head_dim;
  float* x = (float*)(ctx->ws + ctx->lay.x);
  float* qkv = (float*)(ctx->ws + ctx->lay.qkv);
  void* qb = ctx->ws + ctx->lay.qb;
  void* attn = ctx->ws + ctx->lay.attn;
  void* mlp = ctx->ws + ctx->lay.mlp;
  void* qb_lo = lo_plane(g, qb, g.R, qd);
  void* attn_lo = lo_plane(g, attn, g.R, qd);
  void* mlp_lo = lo_plane(g, mlp, g.R, c.intermediate);
  float* part = (float*)(ctx->ws + ctx->lay.part);
  float2* rope = (float2*)(ctx->ws + ctx->lay.rope);
  const int64_t ldcap = (int64_t)tc.n_capture * H;
  void* zrows = ctx->ws + ctx->lay.zrows;  // the lm_head's operand rows
  void* zrows_lo = lo_plane(g, zrows, R, H);
  dflash_status s = dev(ctx,
                        launch_embed(g.bf, ctx->embed, H, c.vocab, anchor, 0, d_tokens, R, 0, nullptr, x, rope, ctx->e,
                                     c.rope_theta, c.head_dim, st),
                        "embed");
  if (s != DFLASH_OK) return s;
  for (int l = 0; l < c.layers; ++l) {
    const Layer& L = ctx->layers[l];
    GemmCall q{EPI_STORE, XSRC_NORM, {seg(L.q, 0, qd), seg(L.k, qd, kvd), seg(L.v, qd + kvd, kvd)}, H, x, H,
               L.in_norm, qkv, qd + 2 * kvd, nullptr};
    q.split = g.bf;
    if ((s = run_gemm(ctx, q, R, st)) != DFLASH_OK) return s;
    s = dev(ctx,
            launch_block_attention(g.bf, t->shape[l], qkv, L.q_norm, L.k_norm, rope, ctx->ring + t->cache_off[l], R, 0,
                                   ctx->e, qb, qb_lo, part, attn, attn_lo, st),
            "attention");
    if (s != DFLASH_OK) return s;
    GemmCall o{EPI_RESID, XSRC_GLOBAL, {seg(L.o, 0, H)}, qd, attn, qd, nullptr, x, H, nullptr};
    o.split = g.bf;
    o.xlo = attn_lo;
    if ((s = run_gemm(ctx, o, R, st)) != DFLASH_OK) return s;
    GemmCall gu{EPI_SWIGLU, XSRC_NORM, {seg(L.gate, 0, c.intermediate), seg(L.up, 0, c.intermediate)}, H, x, H,
                L.post_norm, mlp, c.intermediate, nullptr};
    gu.split = g.bf;
    gu.ylo = mlp_lo;
    if ((s = run_gemm(ctx, gu, R, st)) != DFLASH_OK) return s;
    GemmCall dn{EPI_RESID, XSRC_GLOBAL, {seg(L.down, 0, H)}, c.intermediate, mlp, c.intermediate, nullptr, x, H,
                nullptr};
    dn.split = g.bf;
    dn.xlo = mlp_lo;
    if (d_capture && t->capture_slot[l] >= 0) {  // the residual stream after this layer
      dn.y2 = (unsigned char*)d_capture + (size_t)t->capture_slot[l] * H * g.act_elt;
      dn.ldy2 = ldcap;
    }
    if (l == c.layers - 1) gain_rows_for_argmax(ctx, dn, zrows, zrows_lo, 0);
    if ((s = run_gemm(ctx, dn, R, st)) != DFLASH_OK) return s;
  }
  // the last down launch left every row times the final norm's gain: the lm_head argmax
  GemmCall lm{EPI_ARGMAX, XSRC_LDS, {seg(ctx->lm_head, 0, c.vocab)}, H, zrows, H, nullptr, nullptr, 0, d_argmax};
  lm.split = g.bf;
  lm.xlo = zrows_lo;
  s = run_gemm(ctx, lm, R, st);
  if (s != DFLASH_OK) return s;
  ctx->pending = R;
  return DFLASH_OK;
}

dflash_status dflash_target_trim(dflash_target* t, int32_t m) {
  if (!t) return DFLASH_E_ARG;
  dflash_ctx* ctx = &t->core;
  if (m < 0 || m > ctx->pending || m > ctx->cfg.S)
    return fail(ctx, DFLASH_E_REWIND, "rewind of %d rows with %lld pending and slack %lld", m, (long long)ctx->pending,
                (long long)ctx->cfg.S);
  ctx->e += ctx->pending - m;
  ctx->pending = 0;
  return DFLASH_OK;
}

dflash_status dflash_target_state(const dflash_target* t, int64_t* e, int32_t* pending, int32_t* slack) {
  if (!t) return DFLASH_E_ARG;
  if (e) *e = t->core.e;
  if (pending) *pending = (int32_t)t->core.pending;
  if (slack) *slack = (int32_t)t->core.cfg.S;
  return DFLASH_OK;
}

dflash_status dflash_target_cache_read(dflash_target* t, int32_t layer, void* k_out, void* v_out, int32_t* n_out,
                                       void* stream) {
  if (!t) return DFLASH_E_ARG;
  dflash_ctx* ctx = &t->core;
  if (layer < 0 || layer >= ctx->cfg.c.layers) return fail(ctx, DFLASH_E_RANGE, "layer %d out of range", layer);
  if (!n_out || !k_out || !v_out) return fail(ctx, DFLASH_E_ARG, "NULL count or window output");
  const AttnShape& a = t->shape[layer];
  const int64_t e = ctx->e;
  const int64_t lo = target_full(t->tc, layer) ? 0 : std::max<int64_t>(0, e - (a.window - 1));
  const int n = (int)(e - lo);
  *n_out = n;
  if (n == 0) return DFLASH_OK;
  return dev(ctx,
             launch_cache_read(ctx->cfg.bf, a, ctx->ring + t->cache_off[layer], lo, n, k_out, v_out,
                               (hipStream_t)stream),
             "cache read");
}

}  // extern "C"

// ======================================================================================
// Independent sequences drafted together (dflash_batch_*): one engine (packed weights,
// workspace sized for every sequence's block) and one ring per sequence. Every GEMM of a
// round runs once over the rows of all sequences, so each weight byte is read once per
// round for the whole batch; the embedding, attention (bf16 MFMA shapes), final norm and
// verify also take every sequence in one launch, each on its own positions and ring; the
// ring writes of appended rows run per sequence.
// ======================================================================================
struct dflash_batch {
  dflash_ctx core;  // the engine; core.ring is sequence 0's ring, core.e/pending are unused
  int n_seq = 0;
  size_t ring_seq = 0;  // bytes of one sequence's ring
  std::vector<int64_t> e, pending;
};

namespace {

constexpr int BATCH_MAX_SEQ = 64;
constexpr int BATCH_MAX_ROWS = 512;  // n_seq * (max_block + 1)

dflash_status check_batch(const dflash_config* c, int32_t n_seq, Cfg* g, char* err) {
  dflash_status s = check_cfg(c, g, err);
  if (s != DFLASH_OK) return s;
  if (n_seq < 1 || n_seq > BATCH_MAX_SEQ) return cfg_fail(err, DFLASH_E_RANGE, "n_seq %d outside 1..%d", n_seq, BATCH_MAX_SEQ);
  if (g->dspark) return cfg_fail(err, DFLASH_E_ARG, "a batch drafts in the DFlash form only");
  if ((int64_t)n_seq * (c->max_block + 1) > BATCH_MAX_ROWS)
    return cfg_fail(err, DFLASH_E_RANGE, "n_seq * (max_block + 1) = %lld rows above %d",
                    (long long)n_seq * (c->max_block + 1), BATCH_MAX_ROWS);
  // buffers of a round hold every sequence's block rows; the ring geometry (Cs) stays the
  // one of a single sequence, computed by check_cfg above
  g->R = n_seq * (c->max_block + 1);
  return DFLASH_OK;
}

unsigned char* seq_ring(dflash_batch* b, int s) { return b->core.ring + (size_t)s * b->ring_seq; }

// Runs f with the engine's committed state set to sequence s's (the single-sequence paths
// read ctx->ring, ctx->e and ctx->pending), then stores that state back.
template <class F>
dflash_status as_sequence(dflash_batch* b, int s, F&& f) {
  dflash_ctx& c = b->core;
  unsigned char* ring0 = c.ring;
  c.ring = seq_ring(b, s);
  c.e = b->e[s];
  c.pending = b->pending[s];
  const dflash_status st = f();
  b->e[s] = c.e;
  b->pending[s] = c.pending;
  c.ring = ring0;
  c.e = c.pending = 0;
  return st;
}

}  // namespace

extern "C" {

dflash_status dflash_batch_query_sizes(const dflash_config* cfg, int32_t n_seq, size_t* ring_bytes,
                                       size_t* workspace_bytes, size_t* packed_bytes) {
  Cfg g;
  dflash_status s = check_batch(cfg, n_seq, &g, g_create_err);
  if (s != DFLASH_OK) return s;
  if (!ring_bytes || !workspace_bytes || !packed_bytes) return cfg_fail(g_create_err, DFLASH_E_ARG, "NULL size output");
  *ring_bytes = (size_t)n_seq * ring_bytes_of(g);
  *workspace_bytes = make_layout(g).total;
  *packed_bytes = make_packed_layout(g).total;
  return DFLASH_OK;
}

dflash_status dflash_batch_create(const dflash_config* cfg, int32_t n_seq, const dflash_weights* wts, void* ring,
                                  size_t ring_bytes, void* workspace, size_t workspace_bytes, void* packed,
                                  size_t packed_bytes, void* stream, dflash_batch** out) {
  g_create_err[0] = 0;
  if (!out) return cfg_fail(g_create_err, DFLASH_E_ARG, "NULL output handle");
  *out = nullptr;
  Cfg g;
  dflash_status s = check_batch(cfg, n_seq, &g, g_create_err);
  if (s != DFLASH_OK) return s;
  dflash_batch* b = new (std::nothrow) dflash_batch();
  if (!b) return cfg_fail(g_create_err, DFLASH_E_ARG, "out of host memory");
  b->n_seq = n_seq;
  b->ring_seq = ring_bytes_of(g);
  b->e.assign(n_seq, 0);
  b->pending.assign(n_seq, 0);
  // no deferred K/V: an append projects its rows at once, so a draft never carries
  // committed rows beside the block rows of several sequences
  s = init_engine(&b->core, g, wts, ring, (size_t)n_seq * b->ring_seq, ring_bytes, workspace, workspace_bytes, packed,
                  packed_bytes, false, (hipStream_t)stream);
  if (s != DFLASH_OK) {
    delete b;
    return s;
  }
  *out = b;
  return DFLASH_OK;
}

void dflash_batch_destroy(dflash_batch* b) { delete b; }

const char* dflash_batch_last_error(const dflash_batch* b) { return b ? b->core.err : g_create_err; }

dflash_status dflash_batch_state(const dflash_batch* b, int32_t seq, int64_t* e, int32_t* pending) {
  if (!b) return DFLASH_E_ARG;
  if (seq < 0 || seq >= b->n_seq) return DFLASH_E_RANGE;
  if (e) *e = b->e[seq];
  if (pending) *pending = (int32_t)b->pending[seq];
  return DFLASH_OK;
}

dflash_status dflash_batch_append(dflash_batch* b, const void* resid, const int32_t* counts, int32_t commit,
                                  void* stream) {
  if (!b) return DFLASH_E_ARG;
  dflash_ctx* ctx = &b->core;
  if (!resid || !counts) return fail(ctx, DFLASH_E_ARG, "NULL residual rows or counts: no residual stream captured");
  int64_t total = 0;
  bool fits = !commit;  // rows of one call all land in the ring: every sequence's count <= C
  for (int s = 0; s < b->n_seq; ++s) {
    if (counts[s] < 0) return fail(ctx, DFLASH_E_ARG, "sequence %d: negative row count %d", s, counts[s]);
    total += counts[s];
    fits = fits && counts[s] <= ctx->cfg.C;
  }
  if (total <= 0) return fail(ctx, DFLASH_E_ARG, "append of zero rows: no residual stream captured");
  if (total > INT32_MAX) return fail(ctx, DFLASH_E_RANGE, "append of %lld rows", (long long)total);
  const Cfg& g = ctx->cfg;
  const dflash_config& c = g.c;
  const int64_t F = (int64_t)c.target_streams * c.target_width;
  hipStream_t st = (hipStream_t)stream;
  const unsigned char* base = (const unsigned char*)resid;
  if (!fits) {
    // committing appends (prompts) go sequence by sequence: each drops the rows its window
    // can no longer see before the encoder
    int64_t r = 0;
    for (int s = 0; s < b->n_seq; ++s) {
      const int n = counts[s];
      if (n > 0) {
        const unsigned char* rows = base + (size_t)r * F * g.act_elt;
        const dflash_status st_s =
            as_sequence(b, s, [&] { return dflash_cache_append(ctx, rows, n, commit, stream); });
        if (st_s != DFLASH_OK) return st_s;
      }
      r += n;
    }
    return DFLASH_OK;
  }
  // pending rows of every sequence (a round's verify rows): the encoder, the K/V
  // projections and the ring writes run over all sequences' rows at once (the ring writes
  // per sequence where the attention does not form keys itself)
  std::vector<int64_t> start(b->n_seq), first(b->n_seq + 1, 0);
  for (int s = 0; s < b->n_seq; ++s) {
    start[s] = b->e[s] + b->pending[s];
    first[s + 1] = first[s] + counts[s];
  }
  float* fc_out = (float*)(ctx->ws + ctx->lay.app_fc);
  for (int64_t r0 = 0; r0 < total; r0 += GEMM_MAX_ROWS) {
    const int rc = (int)std::min<int64_t>(GEMM_MAX_ROWS, total - r0);
    GemmCall f{EPI_STORE, XSRC_GLOBAL, {seg(ctx->fc, 0, c.hidden)}, (int)F, base + (size_t)r0 * F * g.act_elt, F,
               nullptr, fc_out, c.hidden, nullptr};
    dflash_status s = run_gemm(ctx, f, rc, st);
    if (s == DFLASH_OK) s = kv_gemms(ctx, rc, st);
    if (s == DFLASH_OK && attention_forms_committed_rows(g.bf, g.a)) {
      // rows r0..r0+rc-1 of the call: sequence q's share is [max(first[q], r0), first[q+1])
      RingSeqs rs{};
      rs.n = b->n_seq;
      for (int q = 0; q <= b->n_seq; ++q) rs.first[q] = (int)std::clamp<int64_t>(first[q] - r0, 0, rc);
      for (int q = 0; q < b->n_seq; ++q) rs.start[q] = start[q] + std::max<int64_t>(r0 - first[q], 0);
      s = dev(ctx,
              launch_ring_write_batch(g.bf, g.a, (const float*)(ctx->ws + ctx->lay.app_kv),
                                      (const void* const*)(ctx->ws + ctx->lay.knorm_ptrs), rs, seq_ring(b, 0),
                                      b->ring_seq, st),
              "ring write");
    } else {
      for (int q = 0; q < b->n_seq && s == DFLASH_OK; ++q) {
        const int64_t lo = std::max<int64_t>(first[q], r0), hi = std::min<int64_t>(first[q + 1], r0 + rc);
        if (lo < hi)
          s = ring_write_rows(ctx, (int)(lo - r0), (int)(hi - lo), start[q] + (lo - first[q]), seq_ring(b, q), st);
      }
    }
    if (s != DFLASH_OK) return s;
  }
  for (int s = 0; s < b->n_seq; ++s) b->pending[s] += counts[s];
  return DFLASH_OK;
}

dflash_status dflash_batch_trim(dflash_batch* b, const int32_t* m) {
  if (!b) return DFLASH_E_ARG;
  if (!m) return fail(&b->core, DFLASH_E_ARG, "NULL rewind counts");
  for (int s = 0; s < b->n_seq; ++s)
    if (m[s] < 0 || m[s] > b->pending[s] || m[s] > b->core.cfg.S)
      return fail(&b->core, DFLASH_E_REWIND, "sequence %d: rewind of %d rows with %lld pending and slack %lld", s,
                  m[s], (long long)b->pending[s], (long long)b->core.cfg.S);
  for (int s = 0; s < b->n_seq; ++s) {
    b->e[s] += b->pending[s] - m[s];
    b->pending[s] = 0;
  }
  return DFLASH_OK;
}

dflash_status dflash_batch_draft(dflash_batch* b, const int32_t* anchors, int32_t block, int32_t* d_tokens,
                                 float* d_hidden, void* stream) {
  if (!b) return DFLASH_E_ARG;
  dflash_ctx* ctx = &b->core;
  const Cfg& g = ctx->cfg;
  const dflash_config& c = g.c;
  if (!anchors || !d_tokens) return fail(ctx, DFLASH_E_ARG, "NULL anchors or token output");
  if (block < 1 || block > c.max_block) return fail(ctx, DFLASH_E_RANGE, "block %d outside 1..%d", block, c.max_block);
  for (int s = 0; s < b->n_seq; ++s) {
    if (anchors[s] < 0 || anchors[s] >= c.vocab)
      return fail(ctx, DFLASH_E_RANGE, "sequence %d: anchor %d outside [0, %d)", s, anchors[s], c.vocab);
    if (b->e[s] <= 0) return fail(ctx, DFLASH_E_NO_CONTEXT, "sequence %d: draft with an empty context", s);
    if (b->pending[s])
      return fail(ctx, DFLASH_E_STATE, "sequence %d: %lld appended rows are not committed", s, (long long)b->pending[s]);
  }
  hipStream_t st = (hipStream_t)stream;
  const int S = b->n_seq, R1 = block + 1, rows = S * R1;
  const int H = c.hidden, hd = c.head_dim;
  const int qd = c.q_heads * hd, kvd = c.kv_heads * hd;
  float* x = (float*)(ctx->ws + ctx->lay.x);
  float* qkv = (float*)(ctx->ws + ctx->lay.qkv);
  unsigned char* qb = ctx->ws + ctx->lay.qb;
  unsigned char* attn = ctx->ws + ctx->lay.attn;
  void* mlp = ctx->ws + ctx->lay.mlp;
  unsigned char* qb_lo = (unsigned char*)lo_plane(g, qb, g.R, qd);
  unsigned char* attn_lo = (unsigned char*)lo_plane(g, attn, g.R, qd);
  void* mlp_lo = lo_plane(g, mlp, g.R, c.intermediate);
  float* part = (float*)(ctx->ws + ctx->lay.part);
  float2* rope = (float2*)(ctx->ws + ctx->lay.rope);
  const size_t ring_layer = (size_t)g.act_elt * 2 * c.kv_heads * (size_t)g.Cs * hd;
  void* zrows = ctx->ws + ctx->lay.zrows;  // each sequence's rows 1..B, consecutive
  void* zrows_lo = lo_plane(g, zrows, S * block, H);
  EmbedSeqs es{};
  AttnSeqs as{};
  es.n = as.n = S;
  for (int q = 0; q < S; ++q) {
    es.anchor[q] = anchors[q];
    es.pos0[q] = as.e[q] = b->e[q];
  }
  dflash_status s = dev(ctx,
                        launch_embed_batch(g.bf, ctx->embed, H, es, R1, c.mask_token_id, x, rope, c.rope_theta, hd, st),
                        "embed");
  for (int l = 0; l < c.layers && s == DFLASH_OK; ++l) {
    const Layer& L = ctx->layers[l];
    GemmCall qc{EPI_STORE, XSRC_NORM, {seg(L.q, 0, qd), seg(L.k, qd, kvd), seg(L.v, qd + kvd, kvd)}, H, x, H,
                L.in_norm, qkv, qd + 2 * kvd, nullptr};
    qc.split = g.bf;
    if ((s = run_gemm(ctx, qc, rows, st)) != DFLASH_OK) return s;
    s = dev(ctx,
            launch_block_attention_batch(g.bf, g.a, as, qkv, L.q_norm, L.k_norm, rope, ctx->ring + l * ring_layer,
                                         b->ring_seq, R1, qb, g.bf ? qb_lo : nullptr, part, attn,
                                         g.bf ? attn_lo : nullptr, st),
            "attention");
    if (s != DFLASH_OK) return s;
    GemmCall o{EPI_RESID, XSRC_GLOBAL, {seg(L.o, 0, H)}, qd, attn, qd, nullptr, x, H, nullptr};
    o.split = g.bf;
    o.xlo = attn_lo;
    if ((s = run_gemm(ctx, o, rows, st)) != DFLASH_OK) return s;
    GemmCall gu{EPI_SWIGLU, XSRC_NORM, {seg(L.gate, 0, c.intermediate), seg(L.up, 0, c.intermediate)}, H, x, H,
                L.post_norm, mlp, c.intermediate, nullptr};
    gu.split = g.bf;
    gu.ylo = mlp_lo;
    if ((s = run_gemm(ctx, gu, rows, st)) != DFLASH_OK) return s;
    GemmCall dn{EPI_RESID, XSRC_GLOBAL, {seg(L.down, 0, H)}, c.intermediate, mlp, c.intermediate, nullptr, x, H,
                nullptr};
    dn.split = g.bf;
    dn.xlo = mlp_lo;
    if (l == c.layers - 1) gain_rows_for_argmax(ctx, dn, zrows, zrows_lo, R1);
    if ((s = run_gemm(ctx, dn, rows, st)) != DFLASH_OK) return s;
  }
  if (s != DFLASH_OK) return s;
  if (d_hidden) {
    s = dev(ctx, hipMemcpyAsync(d_hidden, x, sizeof(float) * rows * H, hipMemcpyDeviceToDevice, st), "hidden copy");
    if (s != DFLASH_OK) return s;
  }
  // the last down launch left each sequence's rows 1..B times the final norm's gain in
  // consecutive operand rows; one lm_head argmax over all of them: d_tokens [n_seq][block]
  GemmCall lm{EPI_ARGMAX, XSRC_LDS, {seg(ctx->lm_head, 0, c.vocab)}, H, zrows, H, nullptr, nullptr, 0, d_tokens};
  lm.split = g.bf;
  lm.xlo = zrows_lo;
  return run_gemm(ctx, lm, S * block, st);
}

dflash_status dflash_batch_lm_head_argmax(dflash_batch* b, const void* rows, int32_t n, int32_t* d_idx, void* stream) {
  if (!b) return DFLASH_E_ARG;
  return dflash_lm_head_argmax(&b->core, rows, n, d_idx, stream);
}

dflash_status dflash_batch_verify_greedy(dflash_batch* b, const int32_t* d_draft, const int32_t* d_target,
                                         int32_t block, int32_t* d_out, void* stream) {
  if (!b) return DFLASH_E_ARG;
  dflash_ctx* ctx = &b->core;
  if (!d_draft || !d_target || !d_out) return fail(ctx, DFLASH_E_ARG, "NULL verify buffer");
  if (block < 1 || block > ctx->cfg.c.max_block)
    return fail(ctx, DFLASH_E_RANGE, "block %d outside 1..%d", block, ctx->cfg.c.max_block);
  return dev(ctx, launch_verify(d_draft, d_target, block, ctx->cfg.c.vocab, d_out, (hipStream_t)stream, b->n_seq),
             "verify");
}

dflash_status dflash_batch_cache_read(dflash_batch* b, int32_t seq, int32_t layer, void* k_out, void* v_out,
                                      int32_t* n_out, void* stream) {
  if (!b) return DFLASH_E_ARG;
  if (seq < 0 || seq >= b->n_seq) return fail(&b->core, DFLASH_E_RANGE, "sequence %d outside 0..%d", seq, b->n_seq - 1);
  return as_sequence(b, seq, [&] { return dflash_cache_read(&b->core, layer, k_out, v_out, n_out, stream); });
}

}  // extern "C"
