"""CPU oracle of the target side of a DFlash round: the target's verify forward.  TEST
INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module.
It shares no code with the HIP library; it reuses the drafter oracle's plain definitions
(RMSNorm, SiLU, neox RoPE, bf16 rounding, first-max argmax, the slack rule).

Source: lablup/mlxcel #1762 "feat(speculative): Muse Glimmer DFlash assistant drafter on the
round loop", What changed, "Muse target": residual-stream capture before the final norm, trim
rollback over the mixed caches, sliding caches armed with clamp(block * 8, 32, 128) rows of
speculative buffer floored at the block size; the target hands out its raw embedding table
and its lm_head (no softcap), which the drafter binds. lablup/mlxcel #1751 "LFM2 / LFM2.5
DSpark drafter on the DFlash loop", opening paragraph (the verify forward with residual-stream
capture; a drafter fed five of the target's residual streams) and Implementation Review
Summary (attention layers trim their KV cache by trim(block_size - n), n = accepted + 1; the
output is token-identical to classic decode).

READINGS (the pages describe a real checkpoint; the target here is synthetic):
  * a causal decoder of Qwen3 shape: per layer RMSNorm -> q/k/v -> per-head q/k RMSNorm ->
    neox RoPE at the absolute position -> causal attention -> o + residual -> RMSNorm ->
    SwiGLU -> down + residual; a final RMSNorm and the shared lm_head after the last layer;
  * layers are sliding or full: a query at position q sees keys p <= q, and on a sliding
    layer only q - W < p (the last W positions, itself included; a rotating cache of W rows);
  * the captured residual streams are the residual stream after each capture layer (before
    the final norm), concatenated in capture order: [rows, streams * hidden];
  * the verify forward runs rows [anchor, d_1..d_B] at positions e..e+B, appends their K/V
    to every layer's cache as pending rows and returns a_i = argmax(lm_head(final_norm(x_i)));
    trim(m) commits the pending rows except the last m (legal iff m <= min(pending, S));
  * precision as in the drafter oracle: f64 activations; bf16 shapes round cached K/V and
    the captured streams (handed to the drafter in its activation dtype) to bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

from oracle.dflash_oracle import (F64, OracleError, argmax_with_margin, cast, rms_norm, rope_neox, silu,
                                  speculative_slack)


@dataclasses.dataclass
class VerifyResult:
    argmax: np.ndarray  # [R] int64: a_0..a_{R-1}
    margins: np.ndarray  # [R] top-1 minus top-2 logit
    capture: np.ndarray  # [R, streams * hidden]: residual streams (storage dtype values)
    hidden: np.ndarray  # [R, hidden]: residual stream after the last layer


class OracleTarget:
    """Synthetic target with per-layer caches keyed by absolute position (no ring)."""

    def __init__(self, shape, weights: Dict[str, object], max_block: int):
        self.sh = shape
        self.w = weights
        self.S = speculative_slack(max_block)
        self.max_block = max_block
        self.e = 0
        self.pending = 0
        # K[l][p], V[l][p]: [nkv, hd] of absolute position p (positions past e + pending are
        # stale or unwritten and never read: a query's keys are positions <= itself)
        self.K = [np.zeros((0, shape.kv_heads, shape.head_dim)) for _ in range(shape.layers)]
        self.V = [np.zeros((0, shape.kv_heads, shape.head_dim)) for _ in range(shape.layers)]

    def _grow(self, n: int) -> None:
        for l in range(self.sh.layers):
            if self.K[l].shape[0] < n:
                extra = max(n, 2 * self.K[l].shape[0]) - self.K[l].shape[0]
                pad = np.zeros((extra, self.sh.kv_heads, self.sh.head_dim))
                self.K[l] = np.concatenate([self.K[l], pad])
                self.V[l] = np.concatenate([self.V[l], pad])

    def first_key(self, layer: int, q: int) -> int:
        """Oldest position a query at q sees on this layer."""
        return 0 if self.sh.layer_kind(layer) == "full" else max(0, q - self.sh.window + 1)

    def _lin(self, name):
        return np.asarray(self.w[name], dtype=F64)

    def _act(self, x):
        return cast(x, self.sh.act_dtype)

    def forward(self, tokens) -> VerifyResult:
        """Rows `tokens` at positions e.. appended to every cache as pending rows."""
        sh = self.sh
        tokens = [int(t) for t in tokens]
        R = len(tokens)
        if R < 1:
            raise OracleError("no rows")
        if self.pending:
            raise OracleError("pending rows: trim first")
        if any(not (0 <= t < sh.vocab) for t in tokens):
            raise OracleError("token id out of range")
        pos = self.e + np.arange(R)
        self._grow(self.e + R)
        x = np.asarray(self.w["embed"], dtype=F64)[tokens]
        nq, nkv, hd = sh.q_heads, sh.kv_heads, sh.head_dim
        group = nq // nkv
        caps = []
        for l in range(sh.layers):
            p = f"layers.{l}."
            h = rms_norm(x, self._lin(p + "in_norm"), sh.rms_eps)
            q = (h @ self._lin(p + "q").T).reshape(R, nq, hd)
            k = (h @ self._lin(p + "k").T).reshape(R, nkv, hd)
            v = (h @ self._lin(p + "v").T).reshape(R, nkv, hd)
            q = rope_neox(rms_norm(q, self._lin(p + "q_norm"), sh.rms_eps), pos, sh.rope_theta)
            k = self._act(rope_neox(rms_norm(k, self._lin(p + "k_norm"), sh.rms_eps), pos, sh.rope_theta))
            v = self._act(v)
            self.K[l][self.e:self.e + R] = k
            self.V[l][self.e:self.e + R] = v
            o = np.zeros((R, nq, hd))
            for i in range(R):
                qp = int(pos[i])
                K = self.K[l][self.first_key(l, qp):qp + 1]  # [n, nkv, hd]: keys lo..qp
                V = self.V[l][self.first_key(l, qp):qp + 1]
                for hh in range(nq):
                    g = hh // group
                    s = K[:, g, :] @ q[i, hh] / np.sqrt(hd)
                    w = np.exp(s - s.max())
                    o[i, hh] = (w / w.sum()) @ V[:, g, :]
            x = x + o.reshape(R, nq * hd) @ self._lin(p + "o").T
            h2 = rms_norm(x, self._lin(p + "post_norm"), sh.rms_eps)
            x = x + (silu(h2 @ self._lin(p + "gate").T) * (h2 @ self._lin(p + "up").T)) @ self._lin(p + "down").T
            if l in sh.capture_layers:
                caps.append((sh.capture_layers.index(l), x.copy()))
        caps.sort(key=lambda c: c[0])
        capture = self._act(np.concatenate([c[1] for c in caps], axis=1))
        z = rms_norm(x, self._lin("final_norm"), sh.rms_eps)
        logits = z @ self._lin("lm_head").T
        idx, margins = argmax_with_margin(logits)
        self.pending = R
        return VerifyResult(argmax=idx.astype(np.int64), margins=margins, capture=capture, hidden=x)

    def trim(self, m: int) -> None:
        """Commit the pending rows except the last m (offsets rewind; nothing is restored)."""
        if m < 0 or m > min(self.pending, self.S):
            raise OracleError(f"illegal rewind of {m} rows (pending {self.pending}, slack {self.S})")
        self.e = self.e + self.pending - m
        self.pending = 0

    def prefill(self, tokens, chunk: int) -> VerifyResult:
        """The prompt in forwards of at most `chunk` rows, each committed; the captures and
        argmaxes of all rows, concatenated."""
        outs = []
        for s in range(0, len(tokens), chunk):
            outs.append(self.forward(tokens[s:s + chunk]))
            self.trim(0)
        return VerifyResult(argmax=np.concatenate([o.argmax for o in outs]),
                            margins=np.concatenate([o.margins for o in outs]),
                            capture=np.concatenate([o.capture for o in outs]),
                            hidden=np.concatenate([o.hidden for o in outs]))

    def window(self, layer: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Committed positions the next query (at e) can see on this layer, with K and V
        ([nkv, n, hd]) in position order."""
        lo = self.first_key(layer, self.e)
        return (np.arange(lo, self.e), self.K[layer][lo:self.e].transpose(1, 0, 2),
                self.V[layer][lo:self.e].transpose(1, 0, 2))

    def state(self):
        return self.e, self.pending, self.S
