"""Lock-step driver for the GPU parity tests: the HIP path (through the C-ABI) and the CPU
oracle advance on identical seeded inputs and are compared after every call.

Acceptance rule (exact vs tolerance):
  * drafted tokens and target argmaxes: exact wherever the oracle's top-2 logit margin
    exceeds 1e-2; a row at or below that margin is a near tie where either index is
    correct, so both sides continue with the oracle's value;
  * accepted length k, bonus token, cache offsets: exact;
  * hidden rows and live ring K/V: per-vector relative L2 error <= 1e-4 (f32 shapes) or
    2e-2 (bf16 shapes), and element by element |gpu - oracle| <= tol * rms(oracle row), plus
    one bf16 rounding step of the oracle's value where both sides store bf16 (the ring of
    bf16 shapes: values a hair apart before the cast may round to neighbouring bf16 values).

The near-tie margin is 1e-2 for bf16 shapes; f32 shapes, whose logits agree with the
oracle's to about 1e-6, use 1e-4.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np
import torch

from block_drafting_dflash_amd import binding, synth
from oracle import dflash_oracle as O

MARGIN = 1e-2
MARGIN_F32 = 1e-4


def rel_rows(g: np.ndarray, o: np.ndarray) -> np.ndarray:
    g = g.reshape(-1, g.shape[-1]).astype(np.float64)
    o = o.reshape(-1, o.shape[-1]).astype(np.float64)
    den = np.maximum(np.linalg.norm(o, axis=1), 1e-30)
    return np.linalg.norm(g - o, axis=1) / den


def bf16_step(o: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |o| (8 significant bits; 2^-133 below the normal range)."""
    _, ex = np.frexp(np.abs(o))
    return np.ldexp(1.0, np.maximum(ex, -125) - 8)


def elem_excess(g: np.ndarray, o: np.ndarray, tol: float, bf16_storage: bool) -> float:
    """max over elements of |g - o| / (tol * rms(o's row) [+ one bf16 step of o]); <= 1 passes."""
    g = g.reshape(-1, g.shape[-1]).astype(np.float64)
    o = o.reshape(-1, o.shape[-1]).astype(np.float64)
    bound = tol * np.sqrt(np.mean(o * o, axis=1, keepdims=True))
    if bf16_storage:
        bound = bound + bf16_step(o)
    bound = np.maximum(bound, 1e-30)
    return float((np.abs(g - o) / bound).max(initial=0.0))


@dataclasses.dataclass
class Stats:
    rows_checked: int = 0
    near_ties: int = 0
    near_tie_flips: int = 0
    max_hidden_rel: float = 0.0
    max_window_rel: float = 0.0
    # largest element error as a fraction of its bound (<= 1)
    max_hidden_elem: float = 0.0
    max_window_elem: float = 0.0


class LockStep:
    def __init__(self, shape, weights_np, max_block: int, phase: int = 0, dev_weights=None,
                 check_windows: bool = True, window_period: int = 1):
        self.sh = shape
        self.dev = dev_weights if dev_weights is not None else binding.to_device(shape, weights_np)
        self.gpu = binding.Drafter(shape, self.dev, max_block, phase)
        self.orc = O.OracleDrafter(shape, weights_np, max_block, phase)
        self.tol = 1e-4 if shape.act_dtype == "f32" else 2e-2
        self.margin = MARGIN_F32 if shape.act_dtype == "f32" else MARGIN
        self.bf16 = shape.act_dtype == "bf16"
        self.dt = binding.act_torch_dtype(shape)
        self.stats = Stats()
        self.check_windows = check_windows
        # the live window is read back after every window_period-th trim; between reads the
        # verified rows' K/V travel with the next draft (read-back projects them first)
        self.window_period = window_period
        self.trims = 0

    def _t(self, a: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.dt).to(self.gpu.device)

    def _agree(self, got: np.ndarray, want: np.ndarray, margins: np.ndarray, what: str) -> None:
        for i in range(len(want)):
            self.stats.rows_checked += 1
            if margins[i] <= self.margin:
                self.stats.near_ties += 1
                self.stats.near_tie_flips += int(got[i] != want[i])
                continue
            assert got[i] == want[i], f"{what} row {i}: gpu {got[i]} oracle {want[i]} (margin {margins[i]:.4g})"

    def check_state(self) -> None:
        e, pend, S, C = self.gpu.cache_state()
        oe, ospan, oS, oC = self.orc.state()
        assert (e, pend, S, C) == (oe, ospan, oS, oC), ((e, pend, S, C), (oe, ospan, oS, oC))

    def check_window(self) -> None:
        for l in range(self.sh.layers):
            k, v = self.gpu.cache_read(l)
            pos, ok, ov = self.orc.live_window(l)
            assert k.shape[1] == len(pos)
            kg, vg = k.float().cpu().numpy(), v.float().cpu().numpy()
            kr = rel_rows(kg, ok)
            vr = rel_rows(vg, ov)
            m = float(max(kr.max(initial=0), vr.max(initial=0)))
            self.stats.max_window_rel = max(self.stats.max_window_rel, m)
            assert m <= self.tol, f"layer {l} window rel err {m}"
            x = max(elem_excess(kg, ok, self.tol, self.bf16), elem_excess(vg, ov, self.tol, self.bf16))
            self.stats.max_window_elem = max(self.stats.max_window_elem, x)
            assert x <= 1.0, f"layer {l} window element error {x:.3g} x its bound"

    def append(self, rows: np.ndarray, commit: bool = False) -> None:
        self.gpu.cache_append(self._t(rows), commit=commit)
        self.orc.append(rows, commit=commit)
        self.check_state()

    def trim(self, m: int) -> None:
        self.gpu.cache_trim(m)
        self.orc.trim(m)
        self.check_state()
        self.trims += 1
        if self.check_windows and self.trims % self.window_period == 0:
            torch.cuda.synchronize()
            self.check_window()

    def draft(self, anchor: int, block: int) -> np.ndarray:
        dspark = getattr(self.sh, "variant", "dflash") == "dspark"
        rows = block if dspark else block + 1
        hidden = torch.empty((rows, self.sh.hidden), dtype=torch.float32, device=self.gpu.device)
        toks = self.gpu.draft_block(anchor, block, hidden=hidden)
        res = self.orc.draft(anchor, block)
        torch.cuda.synchronize()
        hg = hidden.cpu().numpy()
        rel = rel_rows(hg, res.hidden)
        self.stats.max_hidden_rel = max(self.stats.max_hidden_rel, float(rel.max()))
        assert rel.max() <= self.tol, f"hidden rel err {rel.max()} > {self.tol}"
        x = elem_excess(hg, res.hidden, self.tol, False)
        self.stats.max_hidden_elem = max(self.stats.max_hidden_elem, x)
        assert x <= 1.0, f"hidden element error {x:.3g} x its bound"
        if dspark:
            return self._agree_chain(toks.cpu().numpy(), res, anchor)
        self._agree(toks.cpu().numpy(), res.tokens, res.margins, "draft token")
        return res.tokens

    def _agree_chain(self, got: np.ndarray, res, anchor: int) -> np.ndarray:
        """DSpark chain: each step's token against the oracle's step taken from the GPU's own
        previous token (the anchor first), exact above the near-tie margin, so a near tie the
        two sides break differently still leaves every later step checked."""
        w1, w2 = self.orc.w["markov_w1"], self.orc.w["markov_w2"]
        prev = int(anchor)
        for i in range(len(got)):
            score = res.logits[i] + O.markov_transition(w1, w2, prev)
            idx, margin = O.argmax_with_margin(score[None, :])
            self.stats.rows_checked += 1
            if margin[0] <= self.margin:
                self.stats.near_ties += 1
                self.stats.near_tie_flips += int(got[i] != idx[0])
            else:
                assert got[i] == idx[0], f"chain step {i}: gpu {got[i]} oracle {idx[0]} (margin {margin[0]:.4g})"
            prev = int(got[i])
        return got.astype(np.int64)

    def target_argmax(self, rows: np.ndarray) -> np.ndarray:
        idx = self.gpu.lm_head_argmax(self._t(rows))
        oi, om = self.orc.lm_head_argmax(rows)
        torch.cuda.synchronize()
        self._agree(idx.cpu().numpy(), oi, om, "target argmax")
        return oi

    def verify(self, d: np.ndarray, a: np.ndarray) -> tuple:
        B = len(d)
        dev = self.gpu.device
        out = self.gpu.verify_greedy(torch.tensor(d, dtype=torch.int32, device=dev),
                                     torch.tensor(a, dtype=torch.int32, device=dev), B)
        k, bonus = O.verify_greedy(d, a)
        got = out.cpu().tolist()
        assert got == [k, bonus, 0], (got, k, bonus)
        return k, bonus


def run_lm_head_rounds(ls: LockStep, context: int, block: int, rounds: int, anchor_tag: int = 0) -> List[int]:
    """Prefill + rounds whose verify rows go through the shared lm_head."""
    sh = ls.sh
    ls.append(synth.resid_rows(sh, context, 0), commit=True)
    if ls.check_windows:
        torch.cuda.synchronize()
        ls.check_window()
    anchor = synth.anchor_token(sh, tag=anchor_tag)
    ks = []
    for r in range(rounds):
        d = ls.draft(anchor, block)
        a = ls.target_argmax(synth.verify_hidden(sh, block + 1, r))
        k, bonus = ls.verify(d, a)
        ls.append(synth.resid_rows(sh, block + 1, r + 1))
        ls.trim(block - k)
        ks.append(k)
        anchor = bonus
    return ks


def _prefill(ls: LockStep, context: int) -> None:
    ls.append(synth.resid_rows(ls.sh, context, 0), commit=True)
    if ls.check_windows:
        torch.cuda.synchronize()
        ls.check_window()


def run_synthetic_rounds(ls: LockStep, context: int, block: int, rounds: int, p: float, tag: int = 0,
                         prefill: bool = True) -> List[int]:
    """Rounds whose target argmaxes come from the p-accept stand-in target."""
    sh = ls.sh
    if prefill:
        _prefill(ls, context)
    anchor = synth.anchor_token(sh, tag=tag)
    ks = []
    for r in range(rounds):
        d = ls.draft(anchor, block)
        a = synth.synthetic_target_argmax(d, synth.accept_draws(block, r, tag), p, sh.vocab)
        k, bonus = ls.verify(d, a)
        ls.append(synth.resid_rows(sh, block + 1, 1000 * tag + r + 1))
        ls.trim(block - k)
        ks.append(k)
        anchor = bonus
    return ks


def target_with_accept_length(d: np.ndarray, k: int, vocab: int, tail: int) -> np.ndarray:
    """Verify-row argmaxes that accept exactly k of the drafted tokens d."""
    B = len(d)
    a = np.empty(B + 1, dtype=np.int64)
    a[:k] = d[:k]
    if k < B:
        a[k] = (int(d[k]) + 1) % vocab
        a[k + 1:] = tail % vocab
    else:
        a[B] = tail % vocab
    return a


def run_random_depth_rounds(ls: LockStep, context: int, block: int, rounds: int, tag: int = 0,
                            prefill: bool = True) -> List[int]:
    """Rounds whose accepted length is drawn uniformly from 0..block (trims of random depth)."""
    sh = ls.sh
    if prefill:
        _prefill(ls, context)
    anchor = synth.anchor_token(sh, tag=tag)
    ks = []
    for r in range(rounds):
        d = ls.draft(anchor, block)
        kk = synth.random_depth_k(block, r, tag)
        a = target_with_accept_length(d, kk, sh.vocab, tail=anchor + 7 * r)
        k, bonus = ls.verify(d, a)
        assert k == kk
        ls.append(synth.resid_rows(sh, block + 1, 1000 * tag + r + 1))
        ls.trim(block - k)
        ks.append(k)
        anchor = bonus
    return ks
