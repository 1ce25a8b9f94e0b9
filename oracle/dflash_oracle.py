"""CPU oracle of one DFlash speculative round at batch 1.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
module. The product path never calls it, and it shares no code with the HIP library:
every definition below is written out plainly in numpy float64 from the pages, with no
blocking, fusion or reordering beyond splitting the vocabulary into chunks to bound
memory (each logit is still one independent f64 dot product).

Sources (page title, section):
  [muse]   lablup/mlxcel #1762 "feat(speculative): Muse Glimmer DFlash assistant drafter on
           the round loop" -- sections "What changed", "Pre-merge review round",
           "Reported and not fixed", "Real-checkpoint validation".
  [dflash] z-lab/dflash #168 "mlx: load Meta's Muse-Glimmer-30B-assistant DFlash head via a
           draft-adapter registry" -- sections "Why" (remap table), "How", "Measured".
  [dspark] lablup/mlxcel #1751 "LFM2 / LFM2.5 DSpark drafter on the DFlash loop" -- sections
           "Security fixes", "Implementation Review Summary" (Verified against the issue;
           Short-conv rollback).

What the round computes (readings where the pages are silent are marked READING):
  * context append: each captured target residual row R (the concatenated residual
    streams) goes through encoder.fc and encoder.output_norm_enc, both per row, so rows
    that can never be visible may be dropped before the encoder [muse, Pre-merge review
    round, third finding]. READING: each layer's K/V of a context row are
    k = RoPE(k_norm(c W_k^T), p), v = c W_v^T with c the encoder output, and are
    written to a ring slot (p + phase) mod C; the draft's own block K/V are transient
    and attended after the context K/V (the cache holds context rows only) [dspark,
    Implementation Review Summary, Verified against the issue].
  * draft: rows [anchor, mask x B] at absolute positions e..e+B embedded with the
    target's raw table [muse, What changed: raw table, not the embed_norm lookup], then
    five Qwen3-shaped layers [dflash, Why] with per-head q/k RMSNorm and bidirectional
    attention under the absolute-position mask |q - k| <= W [muse, What changed].
    READING: RMSNorm y = x (mean(x^2) + eps)^-1/2 g; neox RoPE with base theta at the
    absolute position, angles in f64; scale 1/sqrt(head_dim); contiguous GQA groups;
    no biases; SwiGLU MLP; a final RMSNorm before the shared untied lm_head (no softcap)
    [muse, What changed]; the drafted token of row j (j = 1..B) is the first index of
    the maximum logit.
  * verify: greedy exact match; k = longest prefix with d_{i+1} == a_i, bonus a_k,
    n = k + 1 rows committed and the attention caches rewound by block - n [dspark,
    Implementation Review Summary, Short-conv rollback].
  * ring slack S = max(clamp(8 B, 32, 128), B) and trim = offset rewind with no restore
    [muse, What changed; Pre-merge review round, second finding].
  * READING (precision): activations are real numbers (f64 here). bf16 shapes round to
    bf16 (nearest, ties to even) only where a value is stored in the cache dtype: the
    context K/V written to the ring and the block's own k/v, which are attended next to
    them. Inputs arrive in their storage dtype (the residual slab, the verify rows, the
    embedding table and the weights are bf16 values already). f32 shapes round nothing.
    Rounding computed activations to bf16 before every contraction would make any two
    correct implementations drift apart by about 1e-2 in the logits at the Muse-shaped
    sizes (each differently rounded operand flips further roundings downstream), so the
    argmax could not be compared exactly above a 1e-2 margin.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------------------
# scalar definitions
# ----------------------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each f64 (ties to even), returned as f64.

    bf16 keeps 8 significant bits: for |x| in [2^(e-1), 2^e) the spacing is 2^(e-8);
    below the smallest normal 2^-126 the spacing stays 2^-133. Values that round past
    the largest finite bf16 become +-inf.
    """
    x = np.asarray(x, dtype=F64)
    m, ex = np.frexp(x)
    ex = np.maximum(ex, -125)
    q = np.ldexp(np.ones_like(x), ex - 8)
    r = np.rint(x / q) * q
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > big, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def cast(x: np.ndarray, act_dtype: str) -> np.ndarray:
    """Operand cast of the activation dtype (identity for f32 shapes)."""
    return round_bf16(x) if act_dtype == "bf16" else np.asarray(x, dtype=F64)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x * (mean(x^2) + eps)^(-1/2) * g."""
    x = np.asarray(x, dtype=F64)
    return x * (np.mean(x * x, axis=-1, keepdims=True) + eps) ** -0.5 * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope_neox(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing (i, i + hd/2), at absolute positions.

    x: [n, heads, hd]; pos: [n]. Angle of pair i at position p is p * theta^(-2i/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=F64) / hd)
    ang = np.asarray(pos, dtype=F64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_traditional(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, adjacent pairing (2i, 2i + 1), at absolute positions.

    The DSpark checkpoint's pairing: its config turns the rotate-half form off, and every
    rotary call site of the backbone then pairs neighbouring elements [dspark, opening
    paragraph; Implementation Review Summary, Verified against the issue]. Pair i at
    position p turns by p * theta^(-2i/hd), the angle of pair i of the rotate-half form.
    x: [n, heads, hd]; pos: [n].
    """
    hd = x.shape[-1]
    inv = theta ** (-np.arange(0, hd, 2, dtype=F64) / hd)  # pair i: theta^(-2i/hd)
    ang = np.asarray(pos, dtype=F64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty(x.shape, dtype=F64)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xo * c + xe * s
    return out


def rope(x: np.ndarray, pos: np.ndarray, theta: float, style: str) -> np.ndarray:
    """RoPE in the named pairing: "neox" (rotate-half) or "traditional" (adjacent)."""
    if style == "neox":
        return rope_neox(x, pos, theta)
    if style == "traditional":
        return rope_traditional(x, pos, theta)
    raise ValueError(f"unknown rope style {style!r}")


def markov_transition(w1: np.ndarray, w2: np.ndarray, prev: int) -> np.ndarray:
    """Transition logits of the low-rank token-transition head after token `prev`.

    markov_w1 [vocab, rank] is gathered at the previous token and markov_w2 [vocab, rank]
    maps the rank-r row to a logit per vocabulary entry [dspark, opening paragraph: a
    rank-256 Markov token-transition head; Security fixes: markov_w1 is indexed by a token
    id once per chain step, rank lies along the last axis of both factors, the transition
    logits span the vocabulary].
    """
    return np.asarray(w2, dtype=F64) @ np.asarray(w1[int(prev)], dtype=F64)


def markov_chain(backbone_logits: np.ndarray, w1, w2, anchor: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """DSpark proposals d_1..d_gamma from the gamma backbone logit rows.

    The chain starts from the anchor and each step's argmax is the token the next step
    gathers [dspark, Implementation Review Summary, Verified against the issue]: step i
    scores row i of the backbone logits plus the transition logits of token t_i (t_0 =
    anchor, t_{i+1} = d_{i+1}) and proposes the first index of the maximum. READING: the
    pages do not spell out how the two logit vectors combine; they are added (both span
    the vocabulary, and the pages check one against the other's size), unscaled.
    Returns (tokens [gamma], margins [gamma], winning scores [gamma]).
    """
    L = np.asarray(backbone_logits, dtype=F64)
    prev = int(anchor)
    toks, margins, tops = [], [], []
    for i in range(L.shape[0]):
        score = L[i] + markov_transition(w1, w2, prev)
        idx, margin = argmax_with_margin(score[None, :])
        prev = int(idx[0])
        toks.append(prev)
        margins.append(float(margin[0]))
        tops.append(float(score[prev]))
    return np.array(toks, dtype=np.int64), np.array(margins), np.array(tops)


DSPARK_MAX_VERIFY_WIDTH = 32  # [dspark, Security fixes, the HIGH finding: verify width clamp]


def speculative_slack(block: int) -> int:
    """Rows of ring slack past the window: clamp(8 B, 32, 128), floored at B.

    [muse, What changed: eight rows per block, clamped to 32..128, never fewer than the
    block; Pre-merge review round, second finding: the floor].
    """
    return max(min(max(8 * block, 32), 128), block)


def dequant_q4(packed: np.ndarray, scales: np.ndarray, biases: np.ndarray, group: int) -> np.ndarray:
    """4-bit affine dequantization w = s * q + b, exact in f64.

    packed: uint32 [out, in/8], eight codes per word along the input dim, lowest nibble
    first, so the packed width is in * 4 / 32 [dspark, Security fixes: a packed factor's
    width is its unpacked width times the bit depth over 32]. scales/biases: [out, in/group].
    """
    out, words = packed.shape
    codes = np.empty((out, words * 8), dtype=F64)
    for j in range(8):
        codes[:, j::8] = (packed >> np.uint32(4 * j)) & np.uint32(0xF)
    s = np.repeat(np.asarray(scales, dtype=F64), group, axis=1)
    b = np.repeat(np.asarray(biases, dtype=F64), group, axis=1)
    return s * codes + b


def argmax_with_margin(logits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """First index of the row maximum, and the top-1 minus top-2 value per row."""
    idx = np.argmax(logits, axis=1)
    if logits.shape[1] < 2:
        return idx, np.full(logits.shape[0], np.inf)
    top2 = np.partition(logits, -2, axis=1)[:, -2:]
    return idx, top2[:, 1] - top2[:, 0]


def verify_greedy(draft, target) -> Tuple[int, int]:
    """Greedy exact-match verify of one block.

    draft = d_1..d_B (the drafter's tokens for positions e+1..e+B); target = a_0..a_B
    (the target's argmax at verify rows e..e+B). k counts the leading rows where
    d_{i+1} == a_i; the bonus token is a_k. [dspark, Implementation Review Summary:
    greedy exact-match verify rule, verify_width = block_size + 1, n = accepted + 1]
    """
    B = len(draft)
    if len(target) != B + 1:
        raise ValueError("target must have block + 1 rows")
    k = 0
    while k < B and int(draft[k]) == int(target[k]):
        k += 1
    return k, int(target[k])


# ----------------------------------------------------------------------------------------
# the drafter with its ring-buffer context cache
# ----------------------------------------------------------------------------------------

class OracleError(Exception):
    pass


@dataclasses.dataclass
class DraftResult:
    tokens: np.ndarray  # [B] int64: drafted d_1..d_B
    hidden: np.ndarray  # [B+1, H] f64: residual stream after the last layer
    margins: np.ndarray  # [B] f64: top-1 minus top-2 logit of rows 1..B
    logits_top: np.ndarray  # [B] f64: the winning logit
    logits: Optional[np.ndarray] = None  # DSpark: the backbone logits [gamma, V] the chain scores


class OracleDrafter:
    """Muse-assistant-shaped drafter plus its ring context cache, in f64.

    shape: any object with the drafter dimensions (hidden, layers, q_heads, kv_heads,
    head_dim, intermediate, vocab, target_streams, target_width, window, weight_dtype,
    act_dtype, rms_eps, rope_theta, group, mask_id). weights: name -> array in storage
    form (f32 arrays of exact values, or objects with packed/scales/biases for q4).
    """

    def __init__(self, shape, weights: Dict[str, object], max_block: int, phase: int = 0,
                 slack_override: Optional[int] = None, cache_f64: bool = True):
        self.sh = shape
        self.w = weights
        if max_block < 1:
            raise OracleError("max_block must be >= 1")
        self.max_block = max_block
        self.S = speculative_slack(max_block) if slack_override is None else slack_override
        self.W = shape.window
        self.C = self.W + self.S
        self.phase = phase % self.C
        self.e = 0  # committed context end (absolute position)
        self.span = 0  # rows appended since the last trim (speculative)
        L, nkv, hd = shape.layers, shape.kv_heads, shape.head_dim
        self.slot_pos = np.full(self.C, -1, dtype=np.int64)
        self.K = np.zeros((L, nkv, self.C, hd), dtype=F64)
        self.V = np.zeros((L, nkv, self.C, hd), dtype=F64)
        self._cache: Dict[str, np.ndarray] = {}
        self._cache_f64 = cache_f64
        self.variant = getattr(shape, "variant", "dflash")
        self.rope_style = getattr(shape, "rope_style", "neox")
        if self.variant == "dspark":
            if getattr(shape, "markov_rank", 0) < 1:
                raise OracleError("a DSpark drafter needs its Markov head")
            if max_block + 1 > DSPARK_MAX_VERIFY_WIDTH:
                raise OracleError(f"verify width {max_block + 1} above {DSPARK_MAX_VERIFY_WIDTH}")
        elif self.variant != "dflash":
            raise OracleError(f"unknown drafter variant {self.variant!r}")

    # -- weights -------------------------------------------------------------------------
    def _lin(self, name: str, rows: Optional[slice] = None) -> np.ndarray:
        if rows is None and name in self._cache:
            return self._cache[name]
        w = self.w[name]
        if hasattr(w, "packed"):
            sl = rows if rows is not None else slice(None)
            out = dequant_q4(w.packed[sl], w.scales[sl], w.biases[sl], w.group)
        else:
            out = np.asarray(w[rows] if rows is not None else w, dtype=F64)
        if rows is None and self._cache_f64:
            self._cache[name] = out
        return out

    def _gain(self, name: str) -> np.ndarray:
        return np.asarray(self.w[name], dtype=F64)

    def _act(self, x):
        """Rounding to the storage dtype (cache K/V; inputs given in that dtype)."""
        return cast(x, self.sh.act_dtype)

    # -- pieces --------------------------------------------------------------------------
    def encode(self, resid: np.ndarray) -> np.ndarray:
        """encoder.fc then encoder.output_norm_enc, per row (rows given in the storage dtype)."""
        r = self._act(np.asarray(resid, dtype=F64))
        h = r @ self._lin("fc").T
        return rms_norm(h, self._gain("enc_norm"), self.sh.rms_eps)

    def context_kv(self, c: np.ndarray, pos: np.ndarray, layer: int) -> Tuple[np.ndarray, np.ndarray]:
        """Per-layer context K/V of encoder rows c at absolute positions pos (ring dtype)."""
        sh = self.sh
        n = c.shape[0]
        k = (c @ self._lin(f"layers.{layer}.k").T).reshape(n, sh.kv_heads, sh.head_dim)
        v = (c @ self._lin(f"layers.{layer}.v").T).reshape(n, sh.kv_heads, sh.head_dim)
        k = rms_norm(k, self._gain(f"layers.{layer}.k_norm"), sh.rms_eps)
        k = rope(k, pos, sh.rope_theta, self.rope_style)
        return self._act(k), self._act(v)

    def lm_head_logits(self, rows: np.ndarray, chunk: int = 16384) -> np.ndarray:
        """f64 logits of rows through the untied lm_head (no softcap)."""
        z = np.asarray(rows, dtype=F64)
        V = self.sh.vocab
        out = np.empty((z.shape[0], V), dtype=F64)
        if "lm_head" in self._cache or V <= chunk or self._cache_f64:
            out[:] = z @ self._lin("lm_head").T
            return out
        for s in range(0, V, chunk):
            sl = slice(s, min(V, s + chunk))
            out[:, sl] = z @ self._lin("lm_head", sl).T
        return out

    def embed(self, ids) -> np.ndarray:
        return np.asarray(self.w["embed"][np.asarray(ids)], dtype=F64)

    # -- cache ---------------------------------------------------------------------------
    def append(self, resid: np.ndarray, commit: bool = False) -> None:
        """Append captured target residual rows at the next absolute positions.

        Rows are speculative (counted in span) until trim; with commit=True they are
        committed at once, and rows that the committed window can no longer see are
        dropped before the encoder runs [muse, Pre-merge review round, third finding].
        """
        resid = np.asarray(resid)
        n = resid.shape[0]
        if n <= 0:
            raise OracleError("append of zero rows: no residual stream captured")
        if resid.shape[1] != self.sh.fc_in:
            raise OracleError("residual width does not match encoder.fc")
        start = self.e + self.span
        end = start + n
        keep_from = end - self.W if commit else end - self.C
        first = max(0, keep_from - start)
        rows = resid[first:]
        pos = np.arange(start + first, end, dtype=np.int64)
        c = self.encode(rows)
        slots = (pos + self.phase) % self.C
        for l in range(self.sh.layers):
            k, v = self.context_kv(c, pos, l)
            # later rows overwrite earlier ones if an append wraps the whole ring
            for i, s in enumerate(slots):
                self.K[l, :, s, :] = k[i]
                self.V[l, :, s, :] = v[i]
        self.slot_pos[slots] = pos
        if commit:
            self.e = end
            self.span = 0
        else:
            self.span += n

    def trim(self, m: int) -> None:
        """Commit the speculative rows except the last m: e += span - m, span = 0.

        Legal iff 0 <= m <= min(span, S); nothing is restored [muse, Pre-merge review
        round: RotatingKVCache::trim rewinds the offsets without restoring them].
        """
        if m < 0 or m > min(self.span, self.S):
            raise OracleError(f"illegal rewind of {m} rows (span {self.span}, slack {self.S})")
        self.e += self.span - m
        self.span = 0

    def live_window(self, layer: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Positions [max(0,e-W), e) with their K, V ([nkv, n, hd]) in position order.

        Raises if a position of the window is not held by the ring (a hole).
        """
        lo = max(0, self.e - self.W)
        pos = np.arange(lo, self.e, dtype=np.int64)
        slots = (pos + self.phase) % self.C
        if np.any(self.slot_pos[slots] != pos):
            raise OracleError("window has holes: a visible position was overwritten")
        return pos, self.K[layer][:, slots, :], self.V[layer][:, slots, :]

    # -- draft ---------------------------------------------------------------------------
    def _attention(self, layer: int, q, kb, vb, qpos) -> np.ndarray:
        """Bidirectional attention of the block over ring context + block keys.

        Visible keys: ring slots holding a committed position p (0 <= p <= e-1) and the
        block's own rows, each visible to query position qp iff |qp - p| <= W.
        """
        sh = self.sh
        R = q.shape[0]
        group = sh.q_heads // sh.kv_heads
        ctx_slots = np.nonzero((self.slot_pos >= 0) & (self.slot_pos <= self.e - 1))[0]
        ctx_pos = self.slot_pos[ctx_slots]
        kpos = np.concatenate([ctx_pos, qpos])
        out = np.zeros((R, sh.q_heads, sh.head_dim), dtype=F64)
        scale = 1.0 / np.sqrt(sh.head_dim)
        # vis[j, i]: key i is visible to query row j; an invisible key gets weight exactly 0
        vis = np.abs(qpos[:, None] - kpos[None, :]) <= self.W
        for h in range(sh.q_heads):
            g = h // group
            keys = np.concatenate([self.K[layer, g, ctx_slots, :], kb[:, g, :]], axis=0)
            vals = np.concatenate([self.V[layer, g, ctx_slots, :], vb[:, g, :]], axis=0)
            s = np.where(vis, (q[:, h, :] @ keys.T) * scale, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[:, h] = (p / p.sum(axis=1, keepdims=True)) @ vals
        return out

    def _backbone(self, ids, qpos: np.ndarray) -> np.ndarray:
        """Rows `ids` at absolute positions qpos through every layer over the ring's
        committed context and their own keys: the residual stream after the last layer."""
        sh = self.sh
        R = len(ids)
        x = self.embed(ids)
        nq, nkv, hd = sh.q_heads, sh.kv_heads, sh.head_dim
        for l in range(sh.layers):
            p = f"layers.{l}."
            h = rms_norm(x, self._gain(p + "in_norm"), sh.rms_eps)
            q = (h @ self._lin(p + "q").T).reshape(R, nq, hd)
            kb = (h @ self._lin(p + "k").T).reshape(R, nkv, hd)
            vb = (h @ self._lin(p + "v").T).reshape(R, nkv, hd)
            q = rope(rms_norm(q, self._gain(p + "q_norm"), sh.rms_eps), qpos, sh.rope_theta, self.rope_style)
            kb = self._act(rope(rms_norm(kb, self._gain(p + "k_norm"), sh.rms_eps), qpos, sh.rope_theta,
                                self.rope_style))
            vb = self._act(vb)
            o = self._attention(l, q, kb, vb, qpos).reshape(R, nq * hd)
            x = x + o @ self._lin(p + "o").T
            h2 = rms_norm(x, self._gain(p + "post_norm"), sh.rms_eps)
            a = silu(h2 @ self._lin(p + "gate").T) * (h2 @ self._lin(p + "up").T)
            x = x + a @ self._lin(p + "down").T
        return x

    def _check_draft(self, anchor: int, block: int) -> None:
        sh = self.sh
        if not (1 <= block <= self.max_block):
            raise OracleError("block out of range")
        if not (0 <= anchor < sh.vocab) or not (0 <= sh.mask_id < sh.vocab):
            raise OracleError("token id out of range")
        if self.e <= 0:
            raise OracleError("empty context")
        if self.span != 0:
            raise OracleError("uncommitted rows pending: trim first")

    def draft(self, anchor: int, block: int) -> DraftResult:
        """One block forward: rows [anchor, mask x B] -> drafted tokens d_1..d_B (DFlash),
        or the DSpark form (draft_dspark) for a DSpark shape."""
        if self.variant == "dspark":
            return self.draft_dspark(anchor, block)
        sh = self.sh
        self._check_draft(anchor, block)
        qpos = self.e + np.arange(block + 1, dtype=np.int64)
        x = self._backbone([anchor] + [sh.mask_id] * block, qpos)
        z = rms_norm(x[1:], self._gain("final_norm"), sh.rms_eps)
        logits = self.lm_head_logits(z)
        idx, margin = argmax_with_margin(logits)
        return DraftResult(tokens=idx.astype(np.int64), hidden=x, margins=margin,
                           logits_top=logits[np.arange(block), idx])

    def draft_dspark(self, anchor: int, gamma: int) -> DraftResult:
        """DSpark block: gamma rows [anchor, mask x (gamma - 1)] at positions e..e+gamma-1,
        every row's logits consumed, position 0 included, then the Markov chain
        [dspark, Implementation Review Summary, Verified against the issue].

        The DSpark backbone attends without a mask (same section: context K/V in the
        cache, the proposal K/V after them, no mask). READING: with the window rule
        |q - p| <= W that is exact while every context row lies within W of every query,
        e + gamma - 1 <= W; longer contexts are refused rather than cut.
        """
        sh = self.sh
        self._check_draft(anchor, gamma)
        if self.e + gamma - 1 > self.W:
            raise OracleError("context past the window: the unmasked DSpark attention would be cut")
        qpos = self.e + np.arange(gamma, dtype=np.int64)
        x = self._backbone([anchor] + [sh.mask_id] * (gamma - 1), qpos)
        z = rms_norm(x, self._gain("final_norm"), sh.rms_eps)
        logits = self.lm_head_logits(z)
        toks, margins, tops = markov_chain(logits, self.w["markov_w1"], self.w["markov_w2"], anchor)
        return DraftResult(tokens=toks, hidden=x, margins=margins, logits_top=tops, logits=logits)

    def lm_head_argmax(self, rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """argmax over the vocabulary of rows (given in the storage dtype) through the shared
        lm_head, and margins."""
        logits = self.lm_head_logits(self._act(np.asarray(rows, dtype=F64)))
        idx, margin = argmax_with_margin(logits)
        return idx.astype(np.int64), margin

    def state(self) -> Tuple[int, int, int, int]:
        return self.e, self.span, self.S, self.C
