"""Round counters of a speculative run, with the definitions the pages print.

draft_rounds / draft_n / draft_n_accepted follow the response timings of the Muse
assistant run (lablup/mlxcel #1762, Real-checkpoint validation, item 4). Mean accepted
length is reported both ways the pages use it: without the bonus token (the Muse
cross-window run: 209 accepted over 47 rounds reads 4.45) and with it (the LFM2.5
DSpark runs in lablup/mlxcel #1751: 184 over 71 rounds reads 3.59). Every round
emits its accepted tokens plus one bonus token.
"""
from __future__ import annotations

import dataclasses
from typing import Dict


@dataclasses.dataclass
class RoundCounters:
    rounds: int = 0
    proposed: int = 0
    accepted: int = 0
    hist: Dict[int, int] = dataclasses.field(default_factory=dict)

    def record(self, block: int, k: int) -> None:
        if not (0 <= k <= block):
            raise ValueError("accepted length outside 0..block")
        self.rounds += 1
        self.proposed += block
        self.accepted += k
        self.hist[k] = self.hist.get(k, 0) + 1

    @property
    def emitted(self) -> int:
        """Tokens committed by the rounds: accepted drafts plus one bonus per round."""
        return self.accepted + self.rounds

    def mean_accepted(self) -> float:
        return self.accepted / self.rounds

    def mean_accepted_with_bonus(self) -> float:
        return self.accepted / self.rounds + 1.0

    def acceptance(self) -> float:
        return self.accepted / self.proposed

    @staticmethod
    def emitted_per_verify(tokens: int, rounds: int) -> float:
        """(generated tokens - 1) / rounds: the first token comes from the prefill."""
        return (tokens - 1) / rounds

    def as_dict(self) -> Dict[str, object]:
        return {"draft_rounds": self.rounds, "draft_n": self.proposed,
                "draft_n_accepted": self.accepted,
                "mean_accepted": self.mean_accepted() if self.rounds else None,
                "mean_accepted_with_bonus": self.mean_accepted_with_bonus() if self.rounds else None,
                "accept_hist": {str(k): v for k, v in sorted(self.hist.items())}}
