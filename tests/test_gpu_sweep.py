"""A seeded sweep of lock-step parity runs over random micro configurations, through the C-ABI:
the shape family (f32, bf16, 4-bit; DFlash and DSpark with either RoPE pairing and ranks 64
to 256), the window (8 to 1000), the widest block, the ring phase, the context length and,
per round, the block width and the accepted length; a third of the DFlash runs are batches
of up to 8 sequences with ragged contexts. Every run checks what the fixed cases check: the
drafted tokens (exact above the near-tie margin), hidden rows, the verify result, offsets
after every call and the live window after every trim."""
import numpy as np
import pytest
import torch

from block_drafting_dflash_amd import binding, synth
from tests import parity as P
from tests.test_gpu_batch import BatchLockStep, run_batch_rounds
from tests.test_gpu_dspark import DS_BF16, DS_F32
from tests.test_gpu_parity import MICRO_BF16, MICRO_F32

pytestmark = pytest.mark.gpu

BASES = {
    "f32": MICRO_F32, "bf16": MICRO_BF16, "q4": MICRO_BF16.with_(weight_dtype="q4"),
    "ds_f32": DS_F32, "ds_bf16": DS_BF16, "ds_q4": DS_BF16.with_(weight_dtype="q4", markov_rank=128),
    "ds_bf16_neox": DS_BF16.with_(rope_style="neox", markov_rank=64),
}
CONFIGS = 300


def draw(rng):
    name = str(rng.choice(list(BASES)))
    base = BASES[name]
    dspark = base.variant == "dspark"
    batch = (not dspark) and rng.random() < 0.3
    if dspark:  # a DSpark context stays within its window: 300 + 4 rounds of <= 32 rows
        window, mb = int(rng.choice([512, 1000])), int(rng.integers(1, 32))
    else:
        window = int(rng.choice([8, 9, 17, 20, 33, 64, 100, 257, 600]))
        mb = int(rng.integers(1, 9)) if batch else int(rng.integers(1, 65))
    return name, base.with_(window=window), batch, mb, int(rng.integers(0, 400)), int(rng.integers(0, 1 << 20))


def test_random_configurations_match_the_oracle():
    rng = np.random.default_rng(20261202)
    weights = {}
    done = 0
    while done < CONFIGS:
        name, sh, batch, mb, phase, tag = draw(rng)
        binding.query_sizes(binding.make_config(sh, mb, phase))  # every drawn configuration is valid
        if name not in weights:
            weights[name] = synth.make_weights(BASES[name])
        w = weights[name]
        label = f"configuration {done}: {name} W={sh.window} max_block={mb} phase={phase} tag={tag} batch={batch}"
        try:
            run_one(rng, sh, w, batch, mb, phase, tag)
        except AssertionError as ex:
            raise AssertionError(f"{label}: {ex}") from ex
        done += 1
    print(f"{done} random configurations matched the oracle")


def run_one(rng, sh, w, batch, mb, phase, tag):
    if batch:
        n = int(rng.integers(1, min(8, 512 // (mb + 1)) + 1))
        contexts = [int(x) for x in rng.integers(1, 300, n)]
        ls = BatchLockStep(sh, w, n, mb, phase)
        run_batch_rounds(ls, contexts, mb, 3, tag=tag)
    else:
        context = int(rng.integers(1, 300))
        ls = P.LockStep(sh, w, max_block=mb, phase=phase)
        ls.append(synth.resid_rows(sh, context, tag % 1000), commit=True)
        torch.cuda.synchronize()
        ls.check_window()
        anchor = synth.anchor_token(sh, tag=tag % 97)
        for r in range(4):
            g = int(rng.integers(1, mb + 1))
            d = ls.draft(anchor, g)
            kk = int(rng.integers(0, g + 1))
            a = P.target_with_accept_length(d, kk, sh.vocab, tail=anchor + 7 * r)
            k, bonus = ls.verify(d, a)
            assert k == kk
            ls.append(synth.resid_rows(sh, g + 1, tag % 1000 + 10 * r + 1))
            ls.trim(g - k)
            anchor = bonus


TARGET_CONFIGS = 150


def test_random_target_configurations_match_the_oracle():
    """The target's verify forward over seeded random micro configurations: window (1-119),
    max_context (512, 1024), which layers attend to everything, which streams are captured,
    the widest block (1-64), the prompt length (in forwards of the widest width) and rounds
    of random width with trims of random depth; argmaxes, captures, offsets and every cache
    window against the target oracle after every call."""
    from tests.test_gpu_target import D_BF16, T_BF16, T_F32, TargetLockStep

    rng = np.random.default_rng(20261203)
    d32 = synth.Shape(hidden=256, layers=1, q_heads=4, kv_heads=2, head_dim=64, intermediate=384, vocab=1040,
                      target_streams=2, target_width=256, window=9, weight_dtype="f32", act_dtype="f32")
    tw = {"bf16": synth.make_target_weights(T_BF16, synth.make_weights(D_BF16)),
          "f32": synth.make_target_weights(T_F32, synth.make_weights(d32))}
    bases = {"bf16": T_BF16, "f32": T_F32}
    for i in range(TARGET_CONFIGS):
        kind = str(rng.choice(["bf16", "f32"]))
        base = bases[kind]
        L = base.layers
        full = tuple(int(l) for l in range(L) if rng.random() < 0.35)
        caps = tuple(sorted(int(x) for x in rng.choice(L, int(rng.integers(1, L + 1)), replace=False)))
        sh = base.with_(window=int(rng.integers(1, 120)), max_context=int(rng.choice([512, 1024])),
                        full_layers=full, capture_layers=caps)
        mb, prompt_len, tag = int(rng.integers(1, 65)), int(rng.integers(1, 200)), int(rng.integers(0, 1 << 20))
        label = f"configuration {i}: {kind} W={sh.window} full={full} caps={caps} max_block={mb} prompt={prompt_len}"
        try:
            ls = TargetLockStep(sh, tw[kind], max_block=mb)
            prompt = [int(x) for x in synth.prompt_tokens(sh.vocab, prompt_len, tag=tag % 1000)]
            for s in range(0, prompt_len, ls.gpu.rows_max):
                ls.forward(prompt[s:s + ls.gpu.rows_max])
                ls.trim(0)
            ls.check_caches()
            anchor = int(prompt[-1])
            for r in range(4):
                g = int(rng.integers(1, mb + 1))
                a, _ = ls.forward([anchor] + [int(x) for x in rng.integers(0, sh.vocab, g)])
                k = int(rng.integers(0, g + 1))
                ls.trim(g - k)
                ls.check_caches()
                anchor = int(a[k])
        except AssertionError as ex:
            raise AssertionError(f"{label}: {ex}") from ex
    print(f"{TARGET_CONFIGS} random target configurations matched the oracle")


SHAPE_CONFIGS = 80


def draw_shape(rng):
    """A random drafter shape: weight dtype, head dim and GQA grouping, hidden / intermediate /
    fc widths in whole tile units, vocabulary, layers, window; and the widest block."""
    wt = str(rng.choice(["f32", "bf16", "q4"]))
    nkv = int(rng.choice([1, 2, 4]))
    unit = 128 if wt == "f32" else 256
    sh = synth.Shape(hidden=unit * int(rng.integers(1, 9)), layers=int(rng.integers(1, 4)),
                     q_heads=nkv * int(rng.choice([1, 2, 4, 8])), kv_heads=nkv, head_dim=int(rng.choice([64, 128])),
                     intermediate=unit * int(rng.integers(1, 17)), vocab=16 * int(rng.integers(40, 1500)),
                     target_streams=int(rng.integers(1, 6)), target_width=unit * int(rng.integers(1, 5)),
                     window=int(rng.choice([9, 33, 64, 200])), weight_dtype=wt,
                     act_dtype="f32" if wt == "f32" else "bf16")
    return sh, int(rng.integers(1, 33))


def test_random_shapes_match_the_oracle():
    """Drafter dimensions decide the GEMM launch plans (waves, chunks, tile and fold forms, the
    4-bit code paths) and the attention's query tiling. Every seeded random shape the library
    accepts (it refuses, before any device call, contraction lengths it has no plan for) runs
    a prefill and three rounds of random width and accepted length in lock-step with the oracle."""
    rng = np.random.default_rng(20261204)
    done = refused = 0
    while done < SHAPE_CONFIGS:
        sh, mb = draw_shape(rng)
        try:
            binding.query_sizes(binding.make_config(sh, mb, 0))
        except binding.DFlashError:
            refused += 1
            continue
        label = (f"shape {done}: {sh.weight_dtype} H={sh.hidden} L={sh.layers} q/kv={sh.q_heads}/{sh.kv_heads} "
                 f"hd={sh.head_dim} I={sh.intermediate} V={sh.vocab} F={sh.target_streams}x{sh.target_width} "
                 f"W={sh.window} max_block={mb}")
        try:
            ls = P.LockStep(sh, synth.make_weights(sh), max_block=mb, phase=int(rng.integers(0, 300)))
            tag = int(rng.integers(0, 1 << 20))
            ls.append(synth.resid_rows(sh, int(rng.integers(1, 120)), tag % 1000), commit=True)
            torch.cuda.synchronize()
            ls.check_window()
            anchor = synth.anchor_token(sh, tag=tag % 97)
            for r in range(3):
                g = int(rng.integers(1, mb + 1))
                d = ls.draft(anchor, g)
                kk = int(rng.integers(0, g + 1))
                k, bonus = ls.verify(d, P.target_with_accept_length(d, kk, sh.vocab, tail=anchor + 7 * r))
                assert k == kk
                ls.append(synth.resid_rows(sh, g + 1, tag % 1000 + 10 * r + 1))
                ls.trim(g - k)
                anchor = bonus
        except AssertionError as ex:
            raise AssertionError(f"{label}: {ex}") from ex
        done += 1
    print(f"{done} random shapes matched the oracle ({refused} drawn shapes refused at validation)")
