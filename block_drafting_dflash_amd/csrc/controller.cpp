// Adaptive verify width of the round loop (host only): the C-ABI declared in
// include/dflash.h under dflash_width_ctl_*.
//
// A drafter that declares a depth below the requested width runs a throughput controller
// between the two: it warms up at the depth and widens to the ceiling only when a measured
// window pays for it (lablup/mlxcel #1762 "Muse Glimmer DFlash assistant drafter on the round
// loop", What changed, "Round loop"; Pre-merge review round, first finding). The measure is
// committed tokens per millisecond (same page, Real-checkpoint validation, item 5). The
// schedule: measure the incumbent (first the depth) over windows; after every
// `challenge_every` of them run one window at the other width and adopt it only if its rate is
// strictly above the incumbent's rate over its whole measurement period since the last
// challenge. A new period then starts from the adopted challenge window, or empty.
#include <new>

#include "../../include/dflash.h"

struct dflash_width_ctl {
  int32_t depth, ceiling, window, challenge_every;
  int32_t incumbent, challenger;
  bool challenging = false;
  bool have_rate = false;
  double incumbent_rate = 0.0;  // tokens per ms of the incumbent over its current period
  double last_challenge_rate = 0.0;
  int32_t windows_since_challenge = 0;
  int32_t rounds = 0;  // of the current window
  int64_t tokens = 0;
  double ms = 0.0;
  int64_t period_tokens = 0;  // of the incumbent's windows since the last challenge
  double period_ms = 0.0;
  int64_t challenges = 0, adoptions = 0;
};

extern "C" {

dflash_status dflash_width_ctl_create(int32_t depth, int32_t ceiling, int32_t window, int32_t challenge_every,
                                      dflash_width_ctl** out) {
  if (!out) return DFLASH_E_ARG;
  *out = nullptr;
  if (depth < 1 || ceiling < depth || window < 1 || challenge_every < 1) return DFLASH_E_RANGE;
  dflash_width_ctl* c = new (std::nothrow) dflash_width_ctl();
  if (!c) return DFLASH_E_ARG;
  c->depth = depth;
  c->ceiling = ceiling;
  c->window = window;
  c->challenge_every = challenge_every;
  c->incumbent = depth;
  c->challenger = ceiling;
  *out = c;
  return DFLASH_OK;
}

void dflash_width_ctl_destroy(dflash_width_ctl* c) { delete c; }

int32_t dflash_width_ctl_width(const dflash_width_ctl* c) {
  if (!c) return 0;
  return c->challenging ? c->challenger : c->incumbent;
}

dflash_status dflash_width_ctl_record(dflash_width_ctl* c, int32_t block, int32_t committed, double ms) {
  if (!c) return DFLASH_E_ARG;
  if (block != dflash_width_ctl_width(c)) return DFLASH_E_STATE;
  if (committed < 1 || !(ms > 0.0)) return DFLASH_E_RANGE;
  c->tokens += committed;
  c->ms += ms;
  if (++c->rounds < c->window) return DFLASH_OK;
  const int64_t w_tokens = c->tokens;
  const double w_ms = c->ms;
  c->rounds = 0;
  c->tokens = 0;
  c->ms = 0.0;
  if (!c->challenging) {
    c->period_tokens += w_tokens;
    c->period_ms += w_ms;
    c->incumbent_rate = (double)c->period_tokens / c->period_ms;
    c->have_rate = true;
    if (c->depth != c->ceiling && ++c->windows_since_challenge >= c->challenge_every) {
      c->challenging = true;
      c->windows_since_challenge = 0;
    }
    return DFLASH_OK;
  }
  const double rate = (double)w_tokens / w_ms;
  ++c->challenges;
  c->last_challenge_rate = rate;
  if (rate > c->incumbent_rate) {
    const int32_t w = c->incumbent;
    c->incumbent = c->challenger;
    c->challenger = w;
    c->incumbent_rate = rate;
    c->period_tokens = w_tokens;
    c->period_ms = w_ms;
    ++c->adoptions;
  } else {
    c->period_tokens = 0;
    c->period_ms = 0.0;
  }
  c->challenging = false;
  return DFLASH_OK;
}

dflash_status dflash_width_ctl_state(const dflash_width_ctl* c, int32_t* incumbent, int32_t* challenger,
                                     int32_t* challenging, double* incumbent_rate, double* challenge_rate,
                                     int64_t* challenges, int64_t* adoptions) {
  if (!c) return DFLASH_E_ARG;
  if (incumbent) *incumbent = c->incumbent;
  if (challenger) *challenger = c->challenger;
  if (challenging) *challenging = c->challenging ? 1 : 0;
  if (incumbent_rate) *incumbent_rate = c->have_rate ? c->incumbent_rate : -1.0;
  if (challenge_rate) *challenge_rate = c->challenges ? c->last_challenge_rate : -1.0;
  if (challenges) *challenges = c->challenges;
  if (adoptions) *adoptions = c->adoptions;
  return DFLASH_OK;
}

}  // extern "C"
