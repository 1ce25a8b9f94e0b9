"""CPU oracle of independent sequences drafted together.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module.

READING: the pages serve one sequence per round loop and decline batched windows (lablup/
mlxcel #1762 "Muse Glimmer DFlash assistant drafter on the round loop", Not in this PR;
lablup/mlxcel #1751 "LFM2 / LFM2.5 DSpark drafter on the DFlash loop", Review fixes: the LFM2
pairing stays at one sequence too). A batch of n sequences is therefore read as n
independent round loops that happen to run at the same block width: each sequence has its
own ring, committed end and pending rows, and nothing one sequence appends, drafts or trims
changes another's results. The batch is n copies of the single-sequence oracle
(dflash_oracle.OracleDrafter) driven in lock-step; ragged rows are split by per-sequence
counts, and a trim applies to every sequence or, if any rewind is illegal, to none.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from oracle.dflash_oracle import DraftResult, OracleDrafter, OracleError


class OracleBatch:
    def __init__(self, shape, weights, n_seq: int, max_block: int, phase: int = 0):
        if n_seq < 1:
            raise OracleError("a batch needs at least one sequence")
        self.n_seq = n_seq
        self.seqs = [OracleDrafter(shape, weights, max_block, phase) for _ in range(n_seq)]

    def append(self, resid: np.ndarray, counts: Sequence[int], commit: bool = False) -> None:
        """resid holds sequence 0's counts[0] rows, then sequence 1's, ..."""
        counts = [int(c) for c in counts]
        if len(counts) != self.n_seq or any(c < 0 for c in counts) or sum(counts) < 1:
            raise OracleError("one non-negative count per sequence, at least one row in all")
        if resid.shape[0] != sum(counts):
            raise OracleError("rows do not match the counts")
        r = 0
        for s, n in enumerate(counts):
            if n:
                self.seqs[s].append(resid[r:r + n], commit=commit)
            r += n

    def trim(self, m: Sequence[int]) -> None:
        m = [int(x) for x in m]
        for od, mm in zip(self.seqs, m):
            e, span, S, _ = od.state()
            if mm < 0 or mm > min(span, S):
                raise OracleError(f"illegal rewind of {mm} rows (span {span}, slack {S})")
        for od, mm in zip(self.seqs, m):
            od.trim(mm)

    def draft(self, anchors: Sequence[int], block: int) -> List[DraftResult]:
        if len(anchors) != self.n_seq:
            raise OracleError("one anchor per sequence")
        for od, a in zip(self.seqs, anchors):  # every check before any sequence drafts
            od._check_draft(int(a), block)
        return [od.draft(int(a), block) for od, a in zip(self.seqs, anchors)]

    def state(self, s: int):
        return self.seqs[s].state()
