"""Seeded synthetic inputs for the DFlash round: shapes, weights, residual rows, verify rows.

This module is shared by the tests, the bench and the oracle runs. It holds random draws,
their storage encodings (bf16 rounding of the draws, the 4-bit affine packing) and the
workload shapes, and none of the method's arithmetic: no norm, projection, attention,
argmax, verify or cache rule lives here.

Shapes follow the Muse Glimmer assistant as the pages describe it: five Qwen3-shaped
sliding-attention layers fed by encoder.fc over concatenated target residual streams
(lablup/mlxcel #1762 "Muse Glimmer DFlash assistant drafter on the round loop", What
changed; z-lab/dflash #168 "load Meta's Muse-Glimmer-30B-assistant DFlash head", Why:
vocab 202048, bidirectional). The stand-in weights are N(0, 0.02); norm gains are
1 + 0.02 N(0, 1) so that the gain multiply is exercised.

Random streams are numpy PCG64 generators keyed by ``SeedSequence(seed, spawn_key=...)``
so every tensor (and every 2048-row block of a large tensor) has its own reproducible
stream and can be drawn in parallel or on its own.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import os
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

# Seeds of the independent input streams.
SEED_WEIGHTS = 0
SEED_RESID = 1
SEED_VERIFY = 2
SEED_ANCHOR = 3
SEED_ACCEPT = 4
SEED_WIDTH_P = 5
SEED_TRIM = 6
SEED_PHASE = 7
SEED_TARGET = 8  # the synthetic target's own layers (its embedding table and lm_head are the drafter's)
SEED_PROMPT = 9

ROW_BLOCK = 2048  # rows per independent RNG block of a weight tensor


@dataclasses.dataclass(frozen=True)
class Shape:
    """Drafter dimensions and storage types (a flat config, as on the Muse assistant)."""

    hidden: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    target_streams: int
    target_width: int
    window: int
    weight_dtype: str  # "f32" | "bf16" | "q4"
    act_dtype: str  # "f32" | "bf16": residual slab, GEMM operands, ring
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    group: int = 64  # q4 group size along the input dim
    mask_token_id: Optional[int] = None
    # the DSpark form of the drafter (lablup/mlxcel #1751 "LFM2 / LFM2.5 DSpark drafter on
    # the DFlash loop", opening paragraph): every block row proposes a token through a
    # low-rank Markov token-transition head, and RoPE may pair adjacent elements
    variant: str = "dflash"  # "dflash" | "dspark"
    rope_style: str = "neox"  # "neox" (rotate-half) | "traditional" (adjacent pairs)
    markov_rank: int = 0

    @property
    def mask_id(self) -> int:
        return self.vocab - 1 if self.mask_token_id is None else self.mask_token_id

    @property
    def fc_in(self) -> int:
        return self.target_streams * self.target_width

    def with_(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


TINY_F32 = Shape(hidden=256, layers=2, q_heads=4, kv_heads=2, head_dim=64, intermediate=512,
                 vocab=4096, target_streams=3, target_width=256, window=32,
                 weight_dtype="f32", act_dtype="f32")
MUSE_BF16 = Shape(hidden=2048, layers=5, q_heads=32, kv_heads=4, head_dim=128, intermediate=6144,
                  vocab=202048, target_streams=5, target_width=4096, window=2048,
                  weight_dtype="bf16", act_dtype="bf16")
MUSE_Q4 = MUSE_BF16.with_(weight_dtype="q4")
# The Muse-shaped backbone in the DSpark form: a rank-256 Markov head, adjacent-pair RoPE and
# a window as long as the longest context served (DSpark attends to every context row).
MUSE_DSPARK_BF16 = MUSE_BF16.with_(variant="dspark", rope_style="traditional", markov_rank=256, window=4096)
TINY_DSPARK_F32 = TINY_F32.with_(variant="dspark", rope_style="traditional", markov_rank=64, window=256)


@dataclasses.dataclass(frozen=True)
class TargetShape:
    """Synthetic causal target: Qwen3-shaped layers, each with a sliding window of `window`
    positions or full attention, and the layers whose residual stream is captured for the
    drafter (hidden = the drafter's hidden, so both share the embedding table and lm_head)."""

    hidden: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    window: int
    full_layers: Tuple[int, ...]
    capture_layers: Tuple[int, ...]
    weight_dtype: str
    act_dtype: str
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    max_context: int = 4096

    def layer_kind(self, l: int) -> str:
        return "full" if l in self.full_layers else "sliding"

    @property
    def streams(self) -> int:
        return len(self.capture_layers)

    def with_(self, **kw) -> "TargetShape":
        return dataclasses.replace(self, **kw)


def drafter_for(target: TargetShape, drafter: Shape) -> Shape:
    """The drafter paired with a target: fc takes the target's captured streams."""
    return drafter.with_(target_streams=target.streams, target_width=target.hidden)


# Targets of the two drafter sizes: hidden equal to the drafter's, mixed sliding/full layers
# (every fifth layer full), residual streams captured at every other layer.
TINY_F32_TARGET = TargetShape(hidden=256, layers=6, q_heads=4, kv_heads=2, head_dim=64, intermediate=512,
                              vocab=4096, window=32, full_layers=(2, 5), capture_layers=(1, 3, 5),
                              weight_dtype="f32", act_dtype="f32", max_context=512)
MUSE_BF16_TARGET = TargetShape(hidden=2048, layers=10, q_heads=32, kv_heads=4, head_dim=128, intermediate=6144,
                               vocab=202048, window=2048, full_layers=(4, 9), capture_layers=(1, 3, 5, 7, 9),
                               weight_dtype="bf16", act_dtype="bf16", max_context=4096)


def target_weight_names(t: TargetShape) -> List[str]:
    names = ["final_norm"]
    for l in range(t.layers):
        names += [f"layers.{l}.{n}" for n in
                  ("q", "k", "v", "o", "gate", "up", "down", "in_norm", "post_norm", "q_norm", "k_norm")]
    return names


def make_target_weights(t: TargetShape, drafter_weights: Dict[str, object], seed: int = SEED_TARGET,
                        threads: Optional[int] = None) -> Dict[str, object]:
    """The target's weights in storage form: its own layers and final norm drawn from their
    own stream (N(0, 0.02), gains 1 + 0.02 N(0, 1)), and the drafter's embedding table and
    lm_head (shared)."""
    proxy = Shape(hidden=t.hidden, layers=t.layers, q_heads=t.q_heads, kv_heads=t.kv_heads, head_dim=t.head_dim,
                  intermediate=t.intermediate, vocab=t.vocab, target_streams=1, target_width=t.hidden,
                  window=t.window, weight_dtype=t.weight_dtype, act_dtype=t.act_dtype)
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    out: Dict[str, object] = {"embed": drafter_weights["embed"], "lm_head": drafter_weights["lm_head"]}
    with _cf.ThreadPoolExecutor(max_workers=threads) as pool:
        for name in target_weight_names(t):
            w = draw_tensor(proxy, name, seed, pool)
            out[name] = w if t.weight_dtype == "f32" else _bf16_parallel(w, pool)
    return out


def prompt_tokens(vocab: int, n: int, tag: int = 0, seed: int = SEED_PROMPT) -> np.ndarray:
    """A prompt of uniform token ids."""
    return _rng(seed, tag).integers(0, vocab, n).astype(np.int64)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    context: int
    blocks: Tuple[int, ...]
    rounds: int
    verify: str  # "lm_head": verify rows N(0,1) through the shared lm_head; "synthetic": p-accept target
    accept_p: Optional[float] = None


# The round workloads (sizes as named; the bench times the Muse-shaped block-4 one).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny-f32-b4-ctx64", TINY_F32, 64, (4,), 32, "lm_head"),
        Workload("muse-bf16-b4-ctx1024", MUSE_BF16, 1024, (4,), 16, "lm_head"),
        Workload("muse-bf16-b16-ctx4096", MUSE_BF16, 4096, (16,), 64, "synthetic", 0.6),
        Workload("muse-bf16-ctx16384-wrap", MUSE_BF16, 16384, (8, 32), 128, "random_depth"),
        Workload("muse-q4-sweep-ctx2048", MUSE_Q4, 2048, (4, 5, 8, 16), 256, "synthetic"),
        # DSpark proposals per block at the pages' verify widths 8 and 10 (lablup/mlxcel
        # #1751, Real-checkpoint validation)
        Workload("muse-dspark-bf16-w8-w10-ctx1024", MUSE_DSPARK_BF16, 1024, (7, 9), 16, "lm_head"),
    ]
}


# --------------------------------------------------------------------------------------
# storage encodings of the draws
# --------------------------------------------------------------------------------------

def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to bf16 (nearest, ties to even) and return them as float32.

    Storage encoding of the synthetic draws only; the arithmetic's own cast points are
    implemented separately by each side.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16-exact float32 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert not np.any(u & np.uint32(0xFFFF)), "value is not bf16-exact"
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class Q4Tensor:
    """4-bit affine weight [out, in]: w = scale * q + bias per group of `group` inputs.

    ``packed`` is uint32 [out, in/8] with eight 4-bit codes per word along the input
    dim, lowest nibble first (packed width = in * 4 / 32). ``scales``/``biases`` are
    bf16-exact float32 [out, in/group].
    """

    packed: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    group: int

    @property
    def shape(self) -> Tuple[int, int]:
        return (self.packed.shape[0], self.packed.shape[1] * 8)


def quantize_q4(w: np.ndarray, group: int) -> Q4Tensor:
    """Synthetic affine quantizer: s = bf16((max-min)/15), b = bf16(min), q = clip(rne((w-b)/s))."""
    out, inn = w.shape
    assert inn % group == 0 and inn % 8 == 0
    g = w.astype(np.float32).reshape(out, inn // group, group)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    s = to_bf16_values((hi - lo) / np.float32(15.0))
    b = to_bf16_values(lo)
    s_safe = np.where(s == 0, np.float32(1.0), s)
    q = np.rint((g - b[:, :, None]) / s_safe[:, :, None])
    q = np.clip(q, 0, 15).astype(np.uint32).reshape(out, inn)
    q8 = q.reshape(out, inn // 8, 8)
    packed = np.zeros((out, inn // 8), dtype=np.uint32)
    for j in range(8):
        packed |= q8[:, :, j] << np.uint32(4 * j)
    return Q4Tensor(packed=packed, scales=s, biases=b, group=group)


# --------------------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------------------

def weight_names(shape: Shape) -> List[str]:
    """Fixed tensor order; the index of a name keys its random stream."""
    names = ["embed", "lm_head", "fc", "enc_norm", "final_norm"]
    for l in range(shape.layers):
        names += [f"layers.{l}.{t}" for t in
                  ("q", "k", "v", "o", "gate", "up", "down",
                   "in_norm", "post_norm", "q_norm", "k_norm")]
    if shape.markov_rank > 0:  # last, so that every other tensor keeps its stream
        names += ["markov_w1", "markov_w2"]
    return names


def weight_shape(shape: Shape, name: str) -> Tuple[int, ...]:
    H, hd = shape.hidden, shape.head_dim
    t = name.split(".")[-1]
    return {
        "embed": (shape.vocab, H),
        "lm_head": (shape.vocab, H),
        "fc": (H, shape.fc_in),
        "enc_norm": (H,), "final_norm": (H,), "in_norm": (H,), "post_norm": (H,),
        "q_norm": (hd,), "k_norm": (hd,),
        "q": (shape.q_heads * hd, H),
        "k": (shape.kv_heads * hd, H),
        "v": (shape.kv_heads * hd, H),
        "o": (H, shape.q_heads * hd),
        "gate": (shape.intermediate, H),
        "up": (shape.intermediate, H),
        "down": (H, shape.intermediate),
        "markov_w1": (shape.vocab, shape.markov_rank),
        "markov_w2": (shape.vocab, shape.markov_rank),
    }[t]


def is_gain(name: str) -> bool:
    return name.split(".")[-1] in ("enc_norm", "final_norm", "in_norm", "post_norm", "q_norm", "k_norm")


def is_markov(name: str) -> bool:
    return name.startswith("markov_")


def is_quantized(shape: Shape, name: str) -> bool:
    """q4 applies to fc, every layer linear and the lm_head; embed, gains and the Markov
    factors stay bf16."""
    return shape.weight_dtype == "q4" and not is_gain(name) and name != "embed" and not is_markov(name)


# Draw scale of the Markov factors: with rank r their transition logits have standard
# deviation 0.25^2 sqrt(r) (1.0 at rank 256), the size of the Muse-shaped backbone's logits
# (0.02 sqrt(2048) ~ 0.9), so both terms of a chain step move its argmax.
MARKOV_SCALE = 0.25


def _draw_block(seed: int, idx: int, blk: int, rows: int, cols: int, gain: bool, scale: float = 0.02) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(idx, blk))))
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    if gain:
        return np.float32(1.0) + np.float32(0.02) * z
    return np.float32(scale) * z


def _scale(name: str) -> float:
    return MARKOV_SCALE if is_markov(name) else 0.02


def draw_tensor(shape: Shape, name: str, seed: int = SEED_WEIGHTS,
                pool: Optional[_cf.Executor] = None) -> np.ndarray:
    """float32 draws of one tensor, before any storage rounding."""
    names = weight_names(shape)
    idx = names.index(name)
    shp = weight_shape(shape, name)
    gain = is_gain(name)
    if len(shp) == 1:
        return _draw_block(seed, idx, 0, 1, shp[0], gain).reshape(shp)
    rows, cols = shp
    out = np.empty((rows, cols), dtype=np.float32)
    blocks = [(b, b * ROW_BLOCK, min(rows, (b + 1) * ROW_BLOCK)) for b in range((rows + ROW_BLOCK - 1) // ROW_BLOCK)]

    def fill(item):
        b, r0, r1 = item
        out[r0:r1] = _draw_block(seed, idx, b, r1 - r0, cols, gain, _scale(name))

    if pool is None or len(blocks) == 1:
        for it in blocks:
            fill(it)
    else:
        list(pool.map(fill, blocks))
    return out


def draw_rows(shape: Shape, name: str, rows: Iterable[int], seed: int = SEED_WEIGHTS) -> np.ndarray:
    """float32 draws of selected rows of a 2-D tensor (regenerates only their blocks)."""
    names = weight_names(shape)
    idx = names.index(name)
    nrows, cols = weight_shape(shape, name)
    rows = list(rows)
    out = np.empty((len(rows), cols), dtype=np.float32)
    cache: Dict[int, np.ndarray] = {}
    for i, r in enumerate(rows):
        assert 0 <= r < nrows
        b = r // ROW_BLOCK
        if b not in cache:
            r0, r1 = b * ROW_BLOCK, min(nrows, (b + 1) * ROW_BLOCK)
            cache[b] = _draw_block(seed, idx, b, r1 - r0, cols, is_gain(name), _scale(name))
        out[i] = cache[b][r - b * ROW_BLOCK]
    return out


def make_weights(shape: Shape, seed: int = SEED_WEIGHTS, threads: Optional[int] = None,
                 skip: Iterable[str] = ()) -> Dict[str, object]:
    """All drafter weights, in storage form.

    f32 shapes: float32 arrays. bf16 shapes: bf16-exact float32 arrays. q4 shapes:
    Q4Tensor for fc, layer linears and lm_head; bf16-exact float32 for embed and gains.
    """
    skip = set(skip)
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    out: Dict[str, object] = {}
    with _cf.ThreadPoolExecutor(max_workers=threads) as pool:
        for name in weight_names(shape):
            if name in skip:
                continue
            w = draw_tensor(shape, name, seed, pool)
            if shape.weight_dtype == "f32":
                out[name] = w
            elif is_quantized(shape, name):
                out[name] = _quantize_parallel(w, shape.group, pool)
            else:
                out[name] = _bf16_parallel(w, pool)
    return out


def _bf16_parallel(w: np.ndarray, pool: _cf.Executor) -> np.ndarray:
    if w.ndim == 1 or w.shape[0] <= ROW_BLOCK:
        return to_bf16_values(w)
    out = np.empty_like(w)
    spans = [(r, min(w.shape[0], r + ROW_BLOCK * 4)) for r in range(0, w.shape[0], ROW_BLOCK * 4)]

    def f(s):
        out[s[0]:s[1]] = to_bf16_values(w[s[0]:s[1]])

    list(pool.map(f, spans))
    return out


def _quantize_parallel(w: np.ndarray, group: int, pool: _cf.Executor) -> Q4Tensor:
    spans = [(r, min(w.shape[0], r + ROW_BLOCK)) for r in range(0, w.shape[0], ROW_BLOCK)]
    parts = list(pool.map(lambda s: quantize_q4(w[s[0]:s[1]], group), spans))
    return Q4Tensor(packed=np.concatenate([p.packed for p in parts]),
                    scales=np.concatenate([p.scales for p in parts]),
                    biases=np.concatenate([p.biases for p in parts]), group=group)


def embed_rows(shape: Shape, ids: Iterable[int], seed: int = SEED_WEIGHTS) -> np.ndarray:
    """Storage-form rows of the embedding table, regenerated without the whole table."""
    r = draw_rows(shape, "embed", ids, seed)
    return r if shape.weight_dtype == "f32" else to_bf16_values(r)


# --------------------------------------------------------------------------------------
# activations and per-round draws
# --------------------------------------------------------------------------------------

def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def resid_rows(shape: Shape, n: int, tag: int, seed: int = SEED_RESID) -> np.ndarray:
    """Captured target residual rows [n, streams*width], N(0,1) in the activation dtype.

    tag 0 is the prefill slab; tag r+1 is the verify-row capture of round r.
    """
    z = _rng(seed, tag).standard_normal((n, shape.fc_in), dtype=np.float32)
    return z if shape.act_dtype == "f32" else to_bf16_values(z)


def verify_hidden(shape: Shape, n: int, rnd: int, seed: int = SEED_VERIFY) -> np.ndarray:
    """Target verify rows [n, hidden], N(0,1), fed through the shared lm_head."""
    z = _rng(seed, rnd).standard_normal((n, shape.hidden), dtype=np.float32)
    return z if shape.act_dtype == "f32" else to_bf16_values(z)


def anchor_token(shape: Shape, seed: int = SEED_ANCHOR, tag: int = 0) -> int:
    return int(_rng(seed, tag).integers(0, shape.vocab))


def accept_draws(block: int, rnd: int, tag: int = 0, seed: int = SEED_ACCEPT) -> np.ndarray:
    """Uniform [0,1) draws [3, block+1] for the p-accept synthetic target of one round."""
    return _rng(seed, tag, rnd).random((3, block + 1))


def synthetic_target_argmax(draft: np.ndarray, u: np.ndarray, p: float, vocab: int) -> np.ndarray:
    """Stand-in for the target's verify-row argmaxes (the target model is not built).

    Row i < B equals the draft token d[i] with probability p and otherwise a token
    guaranteed to differ from it; row B is uniform. Prefix-breaking follows from the
    greedy verify stopping at the first mismatch.
    """
    B = len(draft)
    a = np.empty(B + 1, dtype=np.int64)
    for i in range(B):
        d = int(draft[i])
        if u[0, i] < p:
            a[i] = d
        else:
            a[i] = (d + 1 + int(u[1, i] * (vocab - 1))) % vocab
    a[B] = int(u[2, B] * vocab) % vocab
    return a


def width_accept_p(blocks: Iterable[int], seed: int = SEED_WIDTH_P) -> Dict[int, float]:
    rng = _rng(seed, 0)
    return {int(b): float(rng.uniform(0.4, 0.8)) for b in blocks}


def random_depth_k(block: int, rnd: int, tag: int = 0, seed: int = SEED_TRIM) -> int:
    """Accepted length drawn uniformly from 0..block (trims of random depth block-k)."""
    return int(_rng(seed, tag, rnd).integers(0, block + 1))


def ring_phase_for_wrap(capacity: int, first_append_pos: int, rows: int) -> int:
    """Phase making positions first_append_pos..+rows-1 straddle the ring's last slot."""
    target_slot = capacity - 1 - max(0, rows // 2 - 1)
    return (target_slot - first_append_pos) % capacity


def sha256(a) -> str:
    if isinstance(a, Q4Tensor):
        h = hashlib.sha256()
        for t in (a.packed, a.scales, a.biases):
            h.update(np.ascontiguousarray(t).tobytes())
        return h.hexdigest()
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
