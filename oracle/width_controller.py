"""CPU oracle of the adaptive verify-width controller.  TEST INFRASTRUCTURE ONLY.

Only tests/ and bench.py's cpu_baseline leg may import this module; the product path never
calls it, and it shares no code with the library's controller (csrc/controller.cpp).

Source: lablup/mlxcel #1762 "feat(speculative): Muse Glimmer DFlash assistant drafter on the
round loop":
  * What changed, "Round loop": for a drafter that declares a depth below the requested width
    without insisting on it, the round loop runs a throughput controller between the two; the
    Muse assistant starts at 4 rows under a 16-row ceiling;
  * Pre-merge review round, first finding: a run warms up at the declared depth and widens to
    the requested ceiling only when a measurement window pays for it; the widths a run can
    settle on are the depth and the ceiling;
  * Real-checkpoint validation, item 5: the comparator's measure is tokens per ms over a
    window (16-row challenge windows at 0.012-0.024 tokens/ms against 0.030-0.037 at 4 rows
    were not adopted).

READING (the pages give the behaviour, not the schedule): the controller holds an incumbent
width (first the depth) and a challenger (the other of depth and ceiling). It measures the
incumbent over windows of `window` rounds; after every `challenge_every` incumbent windows it
runs one window at the challenger. A rate is committed tokens divided by summed round times
(tokens per ms). The incumbent's rate is taken over its whole measurement period since the
last challenge (the sums of its windows' tokens and times); the challenger is adopted (the
two swap roles) only if its window's rate is strictly greater. A new period then starts: from
the adopted challenge window, or empty if the incumbent stays. With depth == ceiling nothing
is ever challenged.
"""
from __future__ import annotations

from typing import List, Optional, Tuple


class WidthController:
    def __init__(self, depth: int, ceiling: int, window: int, challenge_every: int):
        if not (1 <= depth <= ceiling) or window < 1 or challenge_every < 1:
            raise ValueError("need 1 <= depth <= ceiling, window >= 1, challenge_every >= 1")
        self.depth, self.ceiling = depth, ceiling
        self.window, self.challenge_every = window, challenge_every
        self.incumbent, self.challenger = depth, ceiling
        self.challenging = False
        self.incumbent_rate: Optional[float] = None
        self.windows_since_challenge = 0
        self.rounds = 0
        self.tokens = 0  # of the current window
        self.ms = 0.0
        self.period_tokens = 0  # of the incumbent's windows since the last challenge
        self.period_ms = 0.0
        self.decisions: List[Tuple[int, float, float, bool]] = []  # (challenger, its rate, incumbent rate, adopted)

    def probed_widths(self) -> Tuple[int, ...]:
        """The widths a run can settle on: the warm-up depth and the ceiling."""
        return (self.depth,) if self.depth == self.ceiling else (self.depth, self.ceiling)

    def width(self) -> int:
        """Block width of the next round."""
        return self.challenger if self.challenging else self.incumbent

    def record(self, block: int, committed: int, ms: float) -> None:
        """One finished round at width `block`: `committed` tokens (accepted + bonus) in `ms`."""
        if block != self.width():
            raise ValueError(f"round ran at {block}, the controller asked for {self.width()}")
        if committed < 1 or not ms > 0.0:
            raise ValueError("a round commits at least one token and takes positive time")
        self.tokens += committed
        self.ms += ms
        self.rounds += 1
        if self.rounds < self.window:
            return
        w_tokens, w_ms = self.tokens, self.ms
        self.rounds, self.tokens, self.ms = 0, 0, 0.0
        if not self.challenging:
            self.period_tokens += w_tokens
            self.period_ms += w_ms
            self.incumbent_rate = self.period_tokens / self.period_ms
            self.windows_since_challenge += 1
            if self.depth != self.ceiling and self.windows_since_challenge >= self.challenge_every:
                self.challenging = True
                self.windows_since_challenge = 0
            return
        rate = w_tokens / w_ms
        adopted = rate > self.incumbent_rate
        self.decisions.append((self.challenger, rate, self.incumbent_rate, adopted))
        if adopted:
            self.incumbent, self.challenger = self.challenger, self.incumbent
            self.incumbent_rate = rate
            self.period_tokens, self.period_ms = w_tokens, w_ms
        else:
            self.period_tokens, self.period_ms = 0, 0.0
        self.challenging = False
