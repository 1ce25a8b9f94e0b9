// Host-side checks of the C-ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// over the runtime's own sources (dflash.cpp, controller.cpp); the kernels are linked as they
// are built for the library, and no call here reaches the device.
//
// It drives every entry point down the paths that end before a device call:
//   - the shape validation of dflash_query_sizes, dflash_batch_query_sizes and
//     dflash_target_query_sizes over seeded mutations of valid configs (edge values of every
//     field: zero, negative, the int32 limits, off-by-one around each bound), with the ring
//     and cache sizes an accepted config reports checked against the slack rule restated
//     here (S = max(clamp(8 * block, 32, 128), block), capacity W + S; lablup/mlxcel #1762,
//     What changed; Pre-merge review round, second finding);
//   - the refusals of dflash_create, dflash_batch_create and dflash_target_create, one
//     defect at a time (NULL or misaligned buffers and weights, buffers below the queried
//     sizes, Markov factors on the wrong variant), each leaving *out NULL;
//   - every call on a NULL handle;
//   - the width controller (lablup/mlxcel #1762, Round loop; Pre-merge review round, first
//     finding) over long seeded schedules, its refusals leaving its state unchanged, and a
//     transcript of every round that the test replays through the oracle's controller.
//
// Output: lines "C case depth ceiling window challenge_every", "T case block committed ms"
// and "F case incumbent challenger challenges adoptions" for the transcript, then "checks N
// failures F". Exit status 1 on a failure.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "dflash.h"

namespace {

long g_checks = 0, g_failures = 0;

#define CHECK(cond, ...)                                                     \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      if (++g_failures <= 40) {                                              \
        std::fprintf(stderr, "FAIL line %d: %s: ", __LINE__, #cond);         \
        std::fprintf(stderr, __VA_ARGS__);                                   \
        std::fputc('\n', stderr);                                            \
      }                                                                      \
    }                                                                        \
  } while (0)

struct SplitMix64 {  // Steele, Lea and Flood, "Fast splittable pseudorandom number generators"
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int32_t below(int32_t n) { return (int32_t)(next() % (uint64_t)n); }
  double unit() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
};

const int32_t EDGES[] = {std::numeric_limits<int32_t>::min(), -4096, -1, 0, 1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32,
                         33, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 511, 512, 1024, 2048, 4095, 4096,
                         4097, 8192, 65536, 202048, 1 << 20, 1 << 24, std::numeric_limits<int32_t>::max() - 15,
                         std::numeric_limits<int32_t>::max()};
const float FEDGES[] = {0.f, -1.f, 1e-30f, 1e-6f, 1.f, 1e6f, std::numeric_limits<float>::infinity(),
                        -std::numeric_limits<float>::infinity(), std::numeric_limits<float>::quiet_NaN(),
                        std::numeric_limits<float>::denorm_min()};

int32_t pick_edge(SplitMix64& r) {
  const int n = (int)(sizeof(EDGES) / sizeof(EDGES[0]));
  return r.below(4) == 0 ? (int32_t)r.next() : EDGES[r.below(n)];
}

// ---------------------------------------------------------------- drafter configs

dflash_config tiny_f32() {
  dflash_config c{};
  c.hidden = 256, c.layers = 2, c.q_heads = 4, c.kv_heads = 2, c.head_dim = 64, c.intermediate = 512;
  c.vocab = 4096, c.target_streams = 3, c.target_width = 256, c.window = 32, c.max_block = 4;
  c.mask_token_id = 4095, c.ring_phase = 0, c.rms_eps = 1e-6f, c.rope_theta = 1e6f;
  c.weight_dtype = DFLASH_F32, c.act_dtype = DFLASH_F32;
  return c;
}

dflash_config muse_bf16() {
  dflash_config c{};
  c.hidden = 2048, c.layers = 5, c.q_heads = 32, c.kv_heads = 4, c.head_dim = 128, c.intermediate = 6144;
  c.vocab = 202048, c.target_streams = 5, c.target_width = 4096, c.window = 2048, c.max_block = 16;
  c.mask_token_id = 202047, c.ring_phase = 40, c.rms_eps = 1e-6f, c.rope_theta = 1e6f;
  c.weight_dtype = DFLASH_BF16, c.act_dtype = DFLASH_BF16;
  return c;
}

dflash_config muse_q4() {
  dflash_config c = muse_bf16();
  c.weight_dtype = DFLASH_Q4G64;
  return c;
}

dflash_config muse_dspark() {
  dflash_config c = muse_bf16();
  c.variant = DFLASH_VARIANT_DSPARK, c.rope_traditional = 1, c.markov_rank = 256, c.window = 4096, c.max_block = 9;
  return c;
}

dflash_config tiny_dspark() {
  dflash_config c = tiny_f32();
  c.variant = DFLASH_VARIANT_DSPARK, c.rope_traditional = 1, c.markov_rank = 64, c.window = 256, c.max_block = 31;
  return c;
}

int64_t slack_rows(int64_t b) {
  const int64_t s = b * 8 < 32 ? 32 : (b * 8 > 128 ? 128 : b * 8);
  return s > b ? s : b;
}

// layers * 2 (K and V) * kv_heads * Cs * head_dim * element size, Cs = the capacity W + S
// raised to W + block + 1 and to 64, rounded up to a multiple of 8
uint64_t ring_formula(const dflash_config& c) {
  int64_t cs = c.window + slack_rows(c.max_block);
  if (cs < (int64_t)c.window + c.max_block + 1) cs = (int64_t)c.window + c.max_block + 1;
  if (cs < 64) cs = 64;
  cs = (cs + 7) / 8 * 8;
  const uint64_t elt = c.act_dtype == DFLASH_F32 ? 4 : 2;
  return (uint64_t)c.layers * 2 * (uint64_t)c.kv_heads * (uint64_t)cs * (uint64_t)c.head_dim * elt;
}

int32_t* int_field(dflash_config& c, int i) {
  int32_t* f[] = {&c.hidden, &c.layers, &c.q_heads, &c.kv_heads, &c.head_dim, &c.intermediate, &c.vocab,
                  &c.target_streams, &c.target_width, &c.window, &c.max_block, &c.mask_token_id, &c.ring_phase,
                  &c.weight_dtype, &c.act_dtype, &c.variant, &c.rope_traditional, &c.markov_rank};
  return f[i];
}
constexpr int N_INT_FIELDS = 18;

void mutate(dflash_config& c, SplitMix64& r) {
  const int k = 1 + r.below(3);
  for (int i = 0; i < k; ++i) {
    const int f = r.below(N_INT_FIELDS + 2);
    if (f == N_INT_FIELDS) c.rms_eps = FEDGES[r.below((int)(sizeof(FEDGES) / sizeof(FEDGES[0])))];
    else if (f == N_INT_FIELDS + 1) c.rope_theta = FEDGES[r.below((int)(sizeof(FEDGES) / sizeof(FEDGES[0])))];
    else if (f >= 13 && r.below(2)) *int_field(c, f) = r.below(4) - 1;  // enum fields: mostly near the valid codes
    else *int_field(c, f) = pick_edge(r);
  }
}

bool valid_status(dflash_status s) { return s >= DFLASH_OK && s <= DFLASH_E_DEVICE; }

void check_drafter_sizes(SplitMix64& r) {
  const dflash_config bases[] = {tiny_f32(), muse_bf16(), muse_q4(), muse_dspark(), tiny_dspark()};
  for (const dflash_config& b : bases) {
    size_t rb = 0, wb = 0, pb = 0;
    CHECK(dflash_query_sizes(&b, &rb, &wb, &pb) == DFLASH_OK, "base config refused: %s", dflash_last_error(nullptr));
    CHECK(rb == ring_formula(b), "ring %zu, slack rule %llu", rb, (unsigned long long)ring_formula(b));
    CHECK(wb > 0 && pb > 0 && wb % 256 == 0 && pb % 256 == 0, "workspace %zu packed %zu", wb, pb);
    CHECK(dflash_query_sizes(&b, nullptr, &wb, &pb) == DFLASH_E_ARG, "NULL ring output");
    CHECK(dflash_query_sizes(&b, &rb, &wb, nullptr) == DFLASH_E_ARG, "NULL packed output");
  }
  CHECK(dflash_query_sizes(nullptr, nullptr, nullptr, nullptr) == DFLASH_E_ARG, "NULL config");
  long accepted = 0;
  for (int it = 0; it < 60000; ++it) {
    dflash_config c = bases[r.below(5)];
    mutate(c, r);
    size_t rb = 7, wb = 7, pb = 7;
    const dflash_status s = dflash_query_sizes(&c, &rb, &wb, &pb);
    CHECK(valid_status(s), "status %d", (int)s);
    if (s != DFLASH_OK) {
      const char* e = dflash_last_error(nullptr);
      CHECK(e && e[0], "no message for status %d", (int)s);
      CHECK(rb == 7 && wb == 7 && pb == 7, "a refused query wrote its outputs");
      continue;
    }
    ++accepted;
    CHECK(rb == ring_formula(c), "ring %zu vs %llu (window %d block %d)", rb, (unsigned long long)ring_formula(c),
          c.window, c.max_block);
    CHECK(wb > 0 && pb > 0 && wb % 256 == 0 && pb % 256 == 0, "workspace %zu packed %zu", wb, pb);
    CHECK(c.hidden > 0 && c.vocab % 16 == 0 && c.mask_token_id >= 0 && c.mask_token_id < c.vocab &&
              c.max_block >= 1 && c.max_block <= 256 && c.window >= 1 && c.window <= 4096 && c.head_dim % 16 == 0 &&
              c.head_dim <= 128 && c.q_heads % c.kv_heads == 0 && c.ring_phase >= 0,
          "accepted an out-of-range config");
    CHECK(c.variant == DFLASH_VARIANT_DSPARK ? c.max_block <= 31 && c.markov_rank >= 64 : c.markov_rank == 0,
          "variant %d block %d rank %d", c.variant, c.max_block, c.markov_rank);
    // the sizes depend on the config alone
    size_t rb2 = 0, wb2 = 0, pb2 = 0;
    CHECK(dflash_query_sizes(&c, &rb2, &wb2, &pb2) == DFLASH_OK && rb2 == rb && wb2 == wb && pb2 == pb,
          "a second query differs");
    // a batch of n: n rings of that size, the same packed weights, a workspace for n blocks
    const int32_t ns[] = {std::numeric_limits<int32_t>::min(), -1, 0, 1, 2, 63, 64, 65,
                          std::numeric_limits<int32_t>::max()};
    const int32_t n = ns[r.below(9)];
    size_t brb = 0, bwb = 0, bpb = 0;
    const dflash_status bs = dflash_batch_query_sizes(&c, n, &brb, &bwb, &bpb);
    CHECK(valid_status(bs), "batch status %d", (int)bs);
    if (bs == DFLASH_OK) {
      CHECK(n >= 1 && n <= 64 && (int64_t)n * (c.max_block + 1) <= 512 && c.variant == DFLASH_VARIANT_DFLASH,
            "batch of %d at block %d accepted", n, c.max_block);
      CHECK(brb == (size_t)n * rb && bpb == pb && bwb >= wb, "batch sizes %zu %zu %zu", brb, bwb, bpb);
    }
  }
  CHECK(accepted > 200, "only %ld mutated configs accepted: the sweep is too narrow", accepted);
  std::fprintf(stderr, "drafter configs: %ld of 60000 mutations accepted\n", accepted);
}

// ---------------------------------------------------------------- target configs

dflash_target_config tiny_target() {
  dflash_target_config c{};
  c.hidden = 256, c.layers = 6, c.q_heads = 4, c.kv_heads = 2, c.head_dim = 64, c.intermediate = 512;
  c.vocab = 4096, c.window = 32, c.max_context = 512, c.max_block = 16;
  c.full_mask = (1ull << 2) | (1ull << 5);
  c.n_capture = 3, c.capture_layers[0] = 1, c.capture_layers[1] = 3, c.capture_layers[2] = 5;
  c.rms_eps = 1e-6f, c.rope_theta = 1e6f, c.weight_dtype = DFLASH_F32, c.act_dtype = DFLASH_F32;
  return c;
}

dflash_target_config muse_target() {
  dflash_target_config c{};
  c.hidden = 2048, c.layers = 10, c.q_heads = 32, c.kv_heads = 4, c.head_dim = 128, c.intermediate = 6144;
  c.vocab = 202048, c.window = 2048, c.max_context = 4096, c.max_block = 16;
  c.full_mask = (1ull << 4) | (1ull << 9);
  c.n_capture = 5;
  for (int i = 0; i < 5; ++i) c.capture_layers[i] = 2 * i + 1;
  c.rms_eps = 1e-6f, c.rope_theta = 1e6f, c.weight_dtype = DFLASH_BF16, c.act_dtype = DFLASH_BF16;
  return c;
}

// sliding layers hold round8(max(W + S, W + R, 64)) slots with R = max(block + 1, 32), full
// layers round8(max_context); each layer's K and V start 256-byte aligned
uint64_t cache_formula(const dflash_target_config& c) {
  const int64_t R = c.max_block + 1 > 32 ? c.max_block + 1 : 32;
  const uint64_t elt = c.act_dtype == DFLASH_F32 ? 4 : 2;
  uint64_t off = 0;
  for (int l = 0; l < c.layers; ++l) {
    int64_t cap;
    if (l < 64 && ((c.full_mask >> l) & 1ull)) {
      cap = c.max_context;
    } else {
      cap = c.window + slack_rows(c.max_block);
      if (cap < c.window + R) cap = c.window + R;
      if (cap < 64) cap = 64;
    }
    cap = (cap + 7) / 8 * 8;
    off += elt * 2 * (uint64_t)c.kv_heads * (uint64_t)cap * (uint64_t)c.head_dim;
    off = (off + 255) / 256 * 256;
  }
  return off;
}

void check_target_sizes(SplitMix64& r) {
  const dflash_target_config bases[] = {tiny_target(), muse_target()};
  for (const dflash_target_config& b : bases) {
    size_t cb = 0, wb = 0, pb = 0;
    CHECK(dflash_target_query_sizes(&b, &cb, &wb, &pb) == DFLASH_OK, "base target refused: %s",
          dflash_last_error(nullptr));
    CHECK(cb == cache_formula(b), "cache %zu vs %llu", cb, (unsigned long long)cache_formula(b));
    CHECK(dflash_target_query_sizes(&b, &cb, nullptr, &pb) == DFLASH_E_ARG, "NULL workspace output");
  }
  CHECK(dflash_target_query_sizes(nullptr, nullptr, nullptr, nullptr) == DFLASH_E_ARG, "NULL target config");
  long accepted = 0;
  for (int it = 0; it < 30000; ++it) {
    dflash_target_config c = bases[r.below(2)];
    const int k = 1 + r.below(3);
    for (int i = 0; i < k; ++i) {
      switch (r.below(16)) {
        case 0: c.hidden = pick_edge(r); break;
        case 1: c.layers = r.below(2) ? pick_edge(r) : r.below(70); break;
        case 2: c.q_heads = pick_edge(r); break;
        case 3: c.kv_heads = pick_edge(r); break;
        case 4: c.head_dim = pick_edge(r); break;
        case 5: c.intermediate = pick_edge(r); break;
        case 6: c.vocab = pick_edge(r); break;
        case 7: c.window = pick_edge(r); break;
        case 8: c.max_context = pick_edge(r); break;
        case 9: c.max_block = r.below(2) ? pick_edge(r) : r.below(70); break;
        case 10: c.full_mask = r.next() & r.next(); break;
        case 11: c.n_capture = r.below(2) ? pick_edge(r) : r.below(10); break;
        case 12: c.capture_layers[r.below(8)] = r.below(2) ? pick_edge(r) : r.below(12); break;
        case 13: c.rms_eps = FEDGES[r.below((int)(sizeof(FEDGES) / sizeof(FEDGES[0])))]; break;
        case 14: c.weight_dtype = r.below(4) - 1; break;
        default: c.act_dtype = r.below(4) - 1; break;
      }
    }
    size_t cb = 7, wb = 7, pb = 7;
    const dflash_status s = dflash_target_query_sizes(&c, &cb, &wb, &pb);
    CHECK(valid_status(s), "target status %d", (int)s);
    if (s != DFLASH_OK) {
      CHECK(cb == 7 && wb == 7 && pb == 7, "a refused target query wrote its outputs");
      continue;
    }
    ++accepted;
    CHECK(c.layers >= 1 && c.layers <= 64 && c.n_capture >= 1 && c.n_capture <= 8 && c.max_block >= 1 &&
              c.max_block <= 64 && c.max_context >= 64 && c.max_context <= 4096,
          "accepted an out-of-range target");
    for (int i = 0; i < c.n_capture; ++i)
      CHECK(c.capture_layers[i] >= 0 && c.capture_layers[i] < c.layers && (i == 0 || c.capture_layers[i] > c.capture_layers[i - 1]),
            "capture layer %d = %d", i, c.capture_layers[i]);
    CHECK(cb == cache_formula(c), "cache %zu vs %llu", cb, (unsigned long long)cache_formula(c));
    CHECK(wb > 0 && pb > 0, "workspace %zu packed %zu", wb, pb);
  }
  CHECK(accepted > 100, "only %ld mutated targets accepted", accepted);
  std::fprintf(stderr, "target configs: %ld of 30000 mutations accepted\n", accepted);
}

// ---------------------------------------------------------------- create refusals

alignas(256) unsigned char g_blob[8192];

struct Weights {
  std::vector<dflash_layer> layers;
  dflash_weights w{};
  explicit Weights(const dflash_config& c) : layers(c.layers) {
    const void* p = g_blob;
    const bool q4 = c.weight_dtype == DFLASH_Q4G64;
    auto lin = [&]() { return dflash_linear{p, q4 ? p : nullptr, q4 ? p : nullptr}; };
    for (dflash_layer& L : layers)
      L = dflash_layer{lin(), lin(), lin(), lin(), lin(), lin(), lin(), p, p, p, p};
    w.embed = p, w.lm_head = lin(), w.fc = lin(), w.enc_norm = p, w.final_norm = p;
    w.layers = layers.data();
    if (c.variant == DFLASH_VARIANT_DSPARK) w.markov_w1 = p, w.markov_w2 = p;
  }
};

// every weight pointer slot of one drafter, in turn: set it to `v` and expect a refusal
std::vector<const void**> weight_slots(Weights& W) {
  std::vector<const void**> s = {&W.w.embed, &W.w.lm_head.w, &W.w.fc.w, &W.w.enc_norm, &W.w.final_norm};
  for (dflash_layer& L : W.layers) {
    for (dflash_linear* l : {&L.q, &L.k, &L.v, &L.o, &L.gate, &L.up, &L.down}) s.push_back(&l->w);
    for (const void** g : {&L.in_norm, &L.post_norm, &L.q_norm, &L.k_norm}) s.push_back(g);
  }
  return s;
}

void check_create_refusals() {
  const dflash_config cfgs[] = {tiny_f32(), muse_bf16(), muse_q4(), tiny_dspark(), muse_dspark()};
  void* buf = g_blob;
  void* odd = g_blob + 64;  // 64-byte aligned, not 256
  for (const dflash_config& c : cfgs) {
    size_t rb = 0, wb = 0, pb = 0;
    CHECK(dflash_query_sizes(&c, &rb, &wb, &pb) == DFLASH_OK, "base");
    auto create = [&](const dflash_weights* w, void* ring, size_t rbytes, void* ws, size_t wbytes, void* pk,
                      size_t pbytes) {
      dflash_ctx* out = reinterpret_cast<dflash_ctx*>(g_blob + 1);  // stale value, must come back NULL
      const dflash_status s = dflash_create(&c, w, ring, rbytes, ws, wbytes, pk, pbytes, nullptr, &out);
      CHECK(out == nullptr, "create left a handle behind (status %d)", (int)s);
      CHECK(dflash_last_error(nullptr)[0] != 0, "create refusal without a message");
      return s;
    };
    Weights W(c);
    CHECK(dflash_create(&c, &W.w, buf, rb, buf, wb, buf, pb, nullptr, nullptr) == DFLASH_E_ARG, "NULL out");
    CHECK(create(nullptr, buf, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "NULL weights");
    {
      dflash_ctx* out = nullptr;
      CHECK(dflash_create(nullptr, &W.w, buf, rb, buf, wb, buf, pb, nullptr, &out) == DFLASH_E_ARG && !out,
            "NULL config");
    }
    CHECK(create(&W.w, nullptr, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "NULL ring");
    CHECK(create(&W.w, buf, rb, nullptr, wb, buf, pb) == DFLASH_E_ARG, "NULL workspace");
    CHECK(create(&W.w, buf, rb, buf, wb, nullptr, pb) == DFLASH_E_ARG, "NULL packed");
    CHECK(create(&W.w, odd, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "misaligned ring");
    CHECK(create(&W.w, buf, rb, odd, wb, buf, pb) == DFLASH_E_ARG, "misaligned workspace");
    CHECK(create(&W.w, buf, rb, buf, wb, odd, pb) == DFLASH_E_ARG, "misaligned packed");
    CHECK(create(&W.w, buf, rb - 1, buf, wb, buf, pb) == DFLASH_E_SHAPE, "short ring");
    CHECK(create(&W.w, buf, rb, buf, wb - 1, buf, pb) == DFLASH_E_SHAPE, "short workspace");
    CHECK(create(&W.w, buf, rb, buf, wb, buf, pb - 1) == DFLASH_E_SHAPE, "short packed");
    {
      const dflash_layer* keep = W.w.layers;
      W.w.layers = nullptr;
      CHECK(create(&W.w, buf, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "NULL layer array");
      W.w.layers = keep;
    }
    for (const void** slot : weight_slots(W)) {
      const void* keep = *slot;
      for (const void* bad : {(const void*)nullptr, (const void*)(g_blob + 8)}) {
        if (bad && slot == &W.w.embed) continue;  // the table is read in place, any alignment of rows
        *slot = bad;
        CHECK(create(&W.w, buf, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "weight slot %p refused", (void*)slot);
      }
      *slot = keep;
    }
    if (c.weight_dtype == DFLASH_Q4G64) {
      W.layers[c.layers - 1].down.scales = nullptr;
      CHECK(create(&W.w, buf, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "q4 linear without scales");
      W.layers[c.layers - 1].down.scales = g_blob;
    }
    if (c.variant == DFLASH_VARIANT_DSPARK) {
      W.w.markov_w2 = nullptr;
      CHECK(create(&W.w, buf, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "DSpark without its second factor");
      W.w.markov_w2 = g_blob + 4;
      CHECK(create(&W.w, buf, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "misaligned Markov factor");
    } else {
      W.w.markov_w1 = g_blob;
      CHECK(create(&W.w, buf, rb, buf, wb, buf, pb) == DFLASH_E_ARG, "Markov factor on a DFlash context");
      W.w.markov_w1 = nullptr;
      // the batch: the same refusals behind its own validation
      size_t brb = 0, bwb = 0, bpb = 0;
      CHECK(dflash_batch_query_sizes(&c, 3, &brb, &bwb, &bpb) == DFLASH_OK, "batch of 3");
      dflash_batch* bo = reinterpret_cast<dflash_batch*>(g_blob + 1);
      CHECK(dflash_batch_create(&c, 3, &W.w, buf, brb - 1, buf, bwb, buf, bpb, nullptr, &bo) == DFLASH_E_SHAPE && !bo,
            "batch with a short ring");
      bo = reinterpret_cast<dflash_batch*>(g_blob + 1);
      CHECK(dflash_batch_create(&c, 0, &W.w, buf, brb, buf, bwb, buf, bpb, nullptr, &bo) == DFLASH_E_RANGE && !bo,
            "batch of 0");
      bo = reinterpret_cast<dflash_batch*>(g_blob + 1);
      CHECK(dflash_batch_create(&c, 3, nullptr, buf, brb, buf, bwb, buf, bpb, nullptr, &bo) == DFLASH_E_ARG && !bo,
            "batch without weights");
      CHECK(dflash_batch_create(&c, 3, &W.w, buf, brb, buf, bwb, buf, bpb, nullptr, nullptr) == DFLASH_E_ARG,
            "batch NULL out");
    }
  }
  // the target: its config, then one defect at a time
  for (const dflash_target_config& c : {tiny_target(), muse_target()}) {
    size_t cb = 0, wb = 0, pb = 0;
    CHECK(dflash_target_query_sizes(&c, &cb, &wb, &pb) == DFLASH_OK, "target base");
    std::vector<dflash_layer> layers(c.layers);
    const void* p = g_blob;
    auto lin = [&]() { return dflash_linear{p, nullptr, nullptr}; };
    for (dflash_layer& L : layers) L = dflash_layer{lin(), lin(), lin(), lin(), lin(), lin(), lin(), p, p, p, p};
    dflash_target_weights w{p, lin(), p, layers.data()};
    auto create = [&](void* cache, size_t cbytes, void* ws, size_t wbytes) {
      dflash_target* out = reinterpret_cast<dflash_target*>(g_blob + 1);
      const dflash_status s = dflash_target_create(&c, &w, cache, cbytes, ws, wbytes, buf, pb, nullptr, &out);
      CHECK(out == nullptr, "target create left a handle behind (status %d)", (int)s);
      return s;
    };
    CHECK(create(nullptr, cb, buf, wb) == DFLASH_E_ARG, "NULL cache");
    CHECK(create(odd, cb, buf, wb) == DFLASH_E_ARG, "misaligned cache");
    CHECK(create(buf, cb - 1, buf, wb) == DFLASH_E_SHAPE, "short cache");
    CHECK(create(buf, cb, buf, wb - 1) == DFLASH_E_SHAPE, "short target workspace");
    w.lm_head.w = g_blob + 8;
    CHECK(create(buf, cb, buf, wb) == DFLASH_E_ARG, "misaligned lm_head");
    w.lm_head.w = p;
    layers[c.layers - 1].k_norm = nullptr;
    CHECK(create(buf, cb, buf, wb) == DFLASH_E_ARG, "NULL k_norm");
    layers[c.layers - 1].k_norm = p;
    w.embed = nullptr;
    CHECK(create(buf, cb, buf, wb) == DFLASH_E_ARG, "NULL embed");
    w.embed = p;
    CHECK(dflash_target_create(&c, &w, buf, cb, buf, wb, buf, pb, nullptr, nullptr) == DFLASH_E_ARG, "NULL out");
  }
}

// ---------------------------------------------------------------- NULL handles

void check_null_handles() {
  int32_t i32 = 0, i32b = 0;
  int64_t i64 = 0;
  int32_t dev_tokens[4] = {0, 0, 0, 0};
  const int32_t anchors[2] = {1, 2}, counts[2] = {1, 1}, ms[2] = {0, 0};
  for (int s = -3; s < 12; ++s) {
    const char* t = dflash_status_string((dflash_status)s);
    CHECK(t && t[0], "status string %d", s);
  }
  CHECK(dflash_last_error(nullptr) && dflash_batch_last_error(nullptr) && dflash_target_last_error(nullptr),
        "last error of a NULL handle");
  dflash_destroy(nullptr);
  dflash_batch_destroy(nullptr);
  dflash_target_destroy(nullptr);
  dflash_width_ctl_destroy(nullptr);
  const dflash_status E = DFLASH_E_ARG;
  CHECK(dflash_cache_append(nullptr, g_blob, 1, 1, nullptr) == E, "append");
  CHECK(dflash_cache_trim(nullptr, 0) == E, "trim");
  CHECK(dflash_draft_block(nullptr, 0, 1, dev_tokens, nullptr, nullptr) == E, "draft");
  CHECK(dflash_lm_head_argmax(nullptr, g_blob, 1, dev_tokens, nullptr) == E, "argmax");
  CHECK(dflash_lm_head_argmax_noalloc(nullptr, g_blob, 1, dev_tokens, nullptr) == E, "argmax noalloc");
  CHECK(dflash_time_next_argmax(nullptr, nullptr, nullptr) == E, "time argmax");
  CHECK(dflash_time_next_chain(nullptr, nullptr, nullptr) == E, "time chain");
  CHECK(dflash_verify_greedy(nullptr, dev_tokens, dev_tokens, 1, dev_tokens, nullptr) == E, "verify");
  CHECK(dflash_cache_state(nullptr, &i64, &i32, &i32b, &i32b) == E, "state");
  CHECK(dflash_cache_read(nullptr, 0, g_blob, g_blob, &i32, nullptr) == E, "cache read");
  CHECK(dflash_hbm_read_probe(nullptr, 4096, (uint32_t*)dev_tokens, 1, nullptr) == E, "probe source");
  CHECK(dflash_hbm_read_probe(g_blob, 4096, nullptr, 1, nullptr) == E, "probe sink");
  CHECK(dflash_hbm_read_probe(g_blob, 4096, (uint32_t*)dev_tokens, 2, nullptr) == E, "probe short source");
  CHECK(dflash_hbm_read_probe(g_blob + 4, 8192, (uint32_t*)dev_tokens, 1, nullptr) == E, "probe misaligned");
  CHECK(dflash_target_forward(nullptr, 0, dev_tokens, 1, dev_tokens, nullptr, nullptr) == E, "target forward");
  CHECK(dflash_target_trim(nullptr, 0) == E, "target trim");
  CHECK(dflash_target_state(nullptr, &i64, &i32, &i32b) == E, "target state");
  CHECK(dflash_target_cache_read(nullptr, 0, g_blob, g_blob, &i32, nullptr) == E, "target cache read");
  CHECK(dflash_batch_append(nullptr, g_blob, counts, 1, nullptr) == E, "batch append");
  CHECK(dflash_batch_trim(nullptr, ms) == E, "batch trim");
  CHECK(dflash_batch_draft(nullptr, anchors, 1, dev_tokens, nullptr, nullptr) == E, "batch draft");
  CHECK(dflash_batch_lm_head_argmax(nullptr, g_blob, 1, dev_tokens, nullptr) == E, "batch argmax");
  CHECK(dflash_batch_verify_greedy(nullptr, dev_tokens, dev_tokens, 1, dev_tokens, nullptr) == E, "batch verify");
  CHECK(dflash_batch_state(nullptr, 0, &i64, &i32) == E, "batch state");
  CHECK(dflash_batch_cache_read(nullptr, 0, 0, g_blob, g_blob, &i32, nullptr) == E, "batch cache read");
  CHECK(dflash_width_ctl_width(nullptr) == 0, "controller width");
  CHECK(dflash_width_ctl_record(nullptr, 1, 1, 1.0) == E, "controller record");
  CHECK(dflash_width_ctl_state(nullptr, &i32, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == E,
        "controller state");
}

// ---------------------------------------------------------------- width controller

struct CtlState {
  int32_t inc, chal, challenging;
  double inc_rate, chal_rate;
  int64_t challenges, adoptions;
  bool operator==(const CtlState& o) const {
    auto same = [](double a, double b) { return a == b || (std::isnan(a) && std::isnan(b)); };
    return inc == o.inc && chal == o.chal && challenging == o.challenging && same(inc_rate, o.inc_rate) &&
           same(chal_rate, o.chal_rate) && challenges == o.challenges && adoptions == o.adoptions;
  }
};

CtlState ctl_state(const dflash_width_ctl* c) {
  CtlState s{};
  CHECK(dflash_width_ctl_state(c, &s.inc, &s.chal, &s.challenging, &s.inc_rate, &s.chal_rate, &s.challenges,
                               &s.adoptions) == DFLASH_OK,
        "state");
  return s;
}

void check_controller(SplitMix64& r) {
  dflash_width_ctl* c = reinterpret_cast<dflash_width_ctl*>(g_blob + 1);
  CHECK(dflash_width_ctl_create(0, 4, 1, 1, &c) == DFLASH_E_RANGE && !c, "depth 0");
  CHECK(dflash_width_ctl_create(5, 4, 1, 1, &c) == DFLASH_E_RANGE && !c, "depth above ceiling");
  CHECK(dflash_width_ctl_create(4, 16, 0, 1, &c) == DFLASH_E_RANGE && !c, "window 0");
  CHECK(dflash_width_ctl_create(4, 16, 1, 0, &c) == DFLASH_E_RANGE && !c, "challenge_every 0");
  CHECK(dflash_width_ctl_create(4, 16, 1, 1, nullptr) == DFLASH_E_ARG, "NULL out");
  CHECK(dflash_width_ctl_create(std::numeric_limits<int32_t>::min(), std::numeric_limits<int32_t>::max(), 1, 1, &c) ==
            DFLASH_E_RANGE,
        "negative depth");

  struct Case {
    int32_t depth, ceiling, window, every, rounds;
  };
  const Case cases[] = {{4, 16, 5, 3, 4000}, {2, 8, 1, 1, 3000}, {5, 5, 3, 2, 500}, {1, 32, 7, 4, 4000},
                        {16, 16, 1, 1, 200}, {3, 31, 2, 5, 3000}};
  int idx = 0;
  for (const Case& k : cases) {
    CHECK(dflash_width_ctl_create(k.depth, k.ceiling, k.window, k.every, &c) == DFLASH_OK && c, "create");
    std::printf("C %d %d %d %d %d\n", idx, k.depth, k.ceiling, k.window, k.every);
    CHECK(dflash_width_ctl_width(c) == k.depth, "starts at the depth");
    // a rate that favours the wider block in some stretches and the narrower in others
    for (int i = 0; i < k.rounds; ++i) {
      const int32_t b = dflash_width_ctl_width(c);
      CHECK(b == k.depth || b == k.ceiling, "width %d outside {%d, %d}", b, k.depth, k.ceiling);
      const bool wide_pays = (i / 600) % 2 == 0;
      const double p = wide_pays ? 0.9 : 0.35;
      int32_t committed = 1;
      while (committed < b + 1 && r.unit() < p) ++committed;
      const double ms = (0.2 + 0.02 * b) * (0.8 + 0.4 * r.unit());
      if (r.below(50) == 0) {  // a refused record leaves the controller as it was
        const CtlState before = ctl_state(c);
        CHECK(dflash_width_ctl_record(c, b == k.depth ? k.ceiling + 1 : k.depth - 1, committed, ms) ==
                  DFLASH_E_STATE,
              "record at another width");
        CHECK(dflash_width_ctl_record(c, b, 0, ms) == DFLASH_E_RANGE, "no committed token");
        CHECK(dflash_width_ctl_record(c, b, committed, 0.0) == DFLASH_E_RANGE, "zero time");
        CHECK(dflash_width_ctl_record(c, b, committed, -1.0) == DFLASH_E_RANGE, "negative time");
        CHECK(dflash_width_ctl_record(c, b, committed, std::nan("")) == DFLASH_E_RANGE, "NaN time");
        CHECK(ctl_state(c) == before, "a refused record changed the state");
      }
      CHECK(dflash_width_ctl_record(c, b, committed, ms) == DFLASH_OK, "record");
      std::printf("T %d %d %d %.17g\n", idx, b, committed, ms);
    }
    const CtlState s = ctl_state(c);
    std::printf("F %d %d %d %lld %lld\n", idx, s.inc, s.chal, (long long)s.challenges, (long long)s.adoptions);
    CHECK(s.adoptions <= s.challenges, "adoptions %lld of %lld", (long long)s.adoptions, (long long)s.challenges);
    if (k.depth == k.ceiling) CHECK(s.challenges == 0, "a single width never challenges");
    dflash_width_ctl_destroy(c);
    ++idx;
  }
  // extreme inputs: the largest commits over long windows, the shortest times
  CHECK(dflash_width_ctl_create(1, std::numeric_limits<int32_t>::max(), 1000, 1, &c) == DFLASH_OK, "wide create");
  for (int i = 0; i < 20000; ++i) {
    const int32_t b = dflash_width_ctl_width(c);
    const double ms = r.below(2) ? std::numeric_limits<double>::denorm_min() : 1e300;
    CHECK(dflash_width_ctl_record(c, b, std::numeric_limits<int32_t>::max(), ms) == DFLASH_OK, "extreme record");
  }
  const CtlState s = ctl_state(c);
  CHECK(s.inc == 1 || s.inc == std::numeric_limits<int32_t>::max(), "incumbent %d", s.inc);
  dflash_width_ctl_destroy(c);
}

}  // namespace

int main() {
  SplitMix64 r{0x5eed5eedull};
  check_null_handles();
  check_drafter_sizes(r);
  check_target_sizes(r);
  check_create_refusals();
  check_controller(r);
  std::printf("checks %ld failures %ld\n", g_checks, g_failures);
  return g_failures ? 1 : 0;
}
