"""GPU parity of the DSpark form of the drafter (lablup/mlxcel #1751 "LFM2 / LFM2.5 DSpark
drafter on the DFlash loop"), through the C-ABI, against the oracle: gamma-row blocks with
every row's logits, the device-side Markov chain (each step checked against the oracle's
step from the GPU's own previous token, exact above the near-tie margin), adjacent-pair
RoPE through the deinterleaved weight fold (hidden rows and the live K/V window read back in
the original element order), the window refusal, and the pages' identity property with a
DSpark drafter on the synthetic target.
"""
import numpy as np
import pytest
import torch

from block_drafting_dflash_amd import binding, synth
from tests import parity as P
from tests import test_gpu_target as TG

pytestmark = pytest.mark.gpu

# ragged vocabularies: the chain's last pass over the vocabulary is partial for ranks whose
# pass is 32 or 64 rows (f32 rank 64, bf16 rank 64)
DS_F32 = synth.Shape(hidden=256, layers=2, q_heads=4, kv_heads=2, head_dim=64, intermediate=384, vocab=4112,
                     target_streams=3, target_width=128, window=160, weight_dtype="f32", act_dtype="f32",
                     variant="dspark", rope_style="traditional", markov_rank=64)
DS_BF16 = synth.Shape(hidden=512, layers=2, q_heads=8, kv_heads=2, head_dim=64, intermediate=768, vocab=3024,
                      target_streams=2, target_width=256, window=200, weight_dtype="bf16", act_dtype="bf16",
                      variant="dspark", rope_style="traditional", markov_rank=256)

CASES = {
    "f32-r64-trad": DS_F32,
    "f32-r256-neox": DS_F32.with_(markov_rank=256, rope_style="neox"),
    "bf16-r256-trad": DS_BF16,
    "bf16-r64-trad": DS_BF16.with_(markov_rank=64),
    "bf16-r512-neox": DS_BF16.with_(markov_rank=512, rope_style="neox"),
    "q4-r128-trad": DS_BF16.with_(weight_dtype="q4", markov_rank=128),
}

_weights = {}


def weights(name):
    if name not in _weights:
        _weights[name] = synth.make_weights(CASES[name])
    return _weights[name]


def run_varying_rounds(ls, context, max_block, rounds, tag):
    """Prefill, then rounds of a block width drawn from 1..max_block, verify rows that accept
    a random prefix, the gamma + 1 verify captures appended and the rejected ones trimmed."""
    sh = ls.sh
    ls.append(synth.resid_rows(sh, context, 0), commit=True)
    torch.cuda.synchronize()
    ls.check_window()
    rng = np.random.default_rng(tag)
    anchor = synth.anchor_token(sh, tag=tag)
    ks = []
    for r in range(rounds):
        g = int(rng.integers(1, max_block + 1))
        d = ls.draft(anchor, g)
        kk = int(rng.integers(0, g + 1))
        a = P.target_with_accept_length(d, kk, sh.vocab, tail=anchor + 7 * r)
        k, bonus = ls.verify(d, a)
        assert k == kk
        ls.append(synth.resid_rows(sh, g + 1, 1000 * tag + r + 1))
        ls.trim(g - k)
        ks.append(k)
        anchor = bonus
    return ks


@pytest.mark.parametrize("name,phase", [(n, 0) for n in CASES] + [("bf16-r256-trad", 208), ("f32-r64-trad", 168)])
def test_dspark_rounds_match_oracle(name, phase):
    """Every case at ring phase 0; two with a phase that puts the ring's wrap point inside the
    rounds' positions."""
    sh = CASES[name]
    ls = P.LockStep(sh, weights(name), max_block=9, phase=phase)
    ks = run_varying_rounds(ls, 37, 9, 10, tag=len(name) + phase)
    print(name, "stats", ls.stats, "ks", ks)
    assert ls.stats.rows_checked > 0


def test_dspark_widest_verify_window():
    """31 proposals (verify width 32, the clamp) in one block, after a context that puts the
    block's rows across two attention chunks."""
    sh = DS_BF16
    ls = P.LockStep(sh, weights("bf16-r256-trad"), max_block=31)
    ls.append(synth.resid_rows(sh, 50, 0), commit=True)
    for r, g in enumerate((31, 1, 31)):
        d = ls.draft(synth.anchor_token(sh, tag=r), g)
        ls.append(synth.resid_rows(sh, g + 1, r + 1))
        ls.trim(g - 2 if g > 2 else 0)
    print("width-32 stats", ls.stats)


def test_dspark_refuses_a_context_the_window_would_cut():
    sh = DS_F32.with_(window=40)
    w = weights("f32-r64-trad")
    d = binding.Drafter(sh, binding.to_device(sh, w), max_block=9)
    d.cache_append(torch.from_numpy(synth.resid_rows(sh, 36, 0)).cuda(), commit=True)
    toks = torch.empty(9, dtype=torch.int32, device="cuda")
    L = binding.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.dflash_draft_block(d.ctx, 3, 5, toks.data_ptr(), None, st) == 0  # 36 + 5 - 1 = 40
    assert L.dflash_draft_block(d.ctx, 3, 6, toks.data_ptr(), None, st) == 3  # 41 > 40
    assert b"window" in L.dflash_last_error(d.ctx)
    assert d.cache_state()[:2] == (36, 0)


def test_dspark_chain_is_bit_reproducible():
    sh = DS_BF16
    ls = P.LockStep(sh, weights("bf16-r256-trad"), max_block=9)
    ls.append(synth.resid_rows(sh, 20, 0), commit=True)
    outs = [ls.gpu.draft_block(11, 9).cpu().tolist() for _ in range(3)]
    assert outs[0] == outs[1] == outs[2]


D_DSPARK = synth.Shape(hidden=512, layers=2, q_heads=8, kv_heads=2, head_dim=64, intermediate=768, vocab=3008,
                       target_streams=3, target_width=512, window=512, weight_dtype="bf16", act_dtype="bf16",
                       variant="dspark", rope_style="traditional", markov_rank=256)


@pytest.mark.parametrize("p_right", [0.0, 0.75])
def test_dspark_speculative_loop_commits_the_tokens_of_classic_decoding(p_right):
    """The pages' identity check with a DSpark drafter (lablup/mlxcel #1751, Implementation
    Review Summary: output token-identical to classic decode): gamma = 7 proposals per round
    (verify width 8), the target's verify forward over [anchor, d_1..d_7], greedy verify, the
    captured streams appended and both caches trimmed by 7 - k."""
    dw = synth.make_weights(D_DSPARK)
    tw = synth.make_target_weights(TG.T_BF16, dw)  # the drafter binds the target's table and lm_head
    tdev = binding.to_device(TG.T_BF16, tw)
    ddev = binding.to_device(D_DSPARK, dw)
    prompt = [int(x) for x in synth.prompt_tokens(TG.T_BF16.vocab, 40, tag=16)]
    n_tokens, B = 48, 7
    want = TG.run_classic(TG.T_BF16, tdev, prompt, n_tokens + B + 1)
    rng = np.random.default_rng(int(100 * p_right) + 1)

    def proposals(pos, drafted):
        return [want[pos + i] if rng.random() < p_right else drafted[i] for i in range(B)]

    got, ks = TG.run_speculative(TG.T_BF16, D_DSPARK, tdev, ddev, prompt, n_tokens, B,
                                 proposals if p_right else None)
    assert got == want[:n_tokens]
    if p_right:
        assert 0 < np.mean(ks) < B
    print("dspark identity", p_right, "accepted", ks)
