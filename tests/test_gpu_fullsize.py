"""GPU parity at the Muse-shaped full sizes (hidden 2048, 5 layers, 32q/4kv x 128, I 6144,
vocab 202048, fc 5 x 4096 -> 2048, window 2048), in the launch configuration the bench
times, in lock-step with the CPU oracle.

Every round compares every drafted token (exact above the 1e-2 near-tie margin), the
final hidden rows (2e-2 relative per row and per element), the verify result, the cache
offsets, and after every trim the whole live K/V window of all five layers. Round counts are
the configurations' own: 16 rounds at block 4, 64 at block 16, 128 per width over the
16384-row context, 256 per width of the 4-bit sweep.
"""
import numpy as np
import pytest
import torch

from block_drafting_dflash_amd import binding, synth
from tests import parity as P

pytestmark = pytest.mark.gpu

SH = synth.MUSE_BF16


@pytest.fixture(scope="module")
def muse():
    w = synth.make_weights(SH)
    dev = binding.to_device(SH, w)
    # the oracle reads linears in f64: convert them once for all tests of this module
    w64 = {k: (np.asarray(v, dtype=np.float64) if k != "embed" and getattr(v, "ndim", 0) == 2 else v)
           for k, v in w.items()}
    del w
    return w64, dev


def _report(name, ls, ks):
    print(f"{name}: rounds {len(ks)} mean k {np.mean(ks):.3f} stats {ls.stats}", flush=True)


def test_block4_ctx1024_lm_head_verify(muse):
    """Block 4 after a 1024-row context; verify rows N(0,1) through the shared lm_head."""
    w64, dev = muse
    wl = synth.WORKLOADS["muse-bf16-b4-ctx1024"]
    ls = P.LockStep(SH, w64, max_block=4, dev_weights=dev)
    ks = P.run_lm_head_rounds(ls, wl.context, 4, wl.rounds)
    _report(wl.name, ls, ks)
    assert ls.stats.rows_checked == wl.rounds * (4 + 5)


def test_block4_ctx1024_deferred_kv(muse):
    """The bench's round sequence at block 4: the verified rows' K/V travel with the next
    draft's QKV launches and attention; the live window of all layers is read back every
    fourth trim and at the end."""
    w64, dev = muse
    wl = synth.WORKLOADS["muse-bf16-b4-ctx1024"]
    ls = P.LockStep(SH, w64, max_block=4, dev_weights=dev, window_period=4)
    ks = P.run_lm_head_rounds(ls, wl.context, 4, 8, anchor_tag=3)
    torch.cuda.synchronize()
    ls.check_window()
    _report(wl.name + " deferred", ls, ks)


def test_block16_ctx4096_synthetic_accept(muse):
    """Block 16 after a 4096-row prefill (2048 kept); p = 0.6 prefix-broken stand-in target."""
    w64, dev = muse
    wl = synth.WORKLOADS["muse-bf16-b16-ctx4096"]
    ls = P.LockStep(SH, w64, max_block=16, dev_weights=dev)
    ks = P.run_synthetic_rounds(ls, wl.context, 16, wl.rounds, p=wl.accept_p)
    _report(wl.name, ls, ks)
    assert any(k > 0 for k in ks)
    assert ls.gpu.cache_state()[0] == wl.context + sum(k + 1 for k in ks)


@pytest.mark.parametrize("block,rounds", [(8, 128), (32, 128)])
def test_ctx16384_forced_wraps_random_depth(muse, block, rounds):
    """16384-row prefill slab (drop-then-project keeps 2048), a ring phase that puts the
    first round's append across the last slot, trims of random depth, then the deepest
    legal rewind (S rows appended and all rewound) and one more round."""
    w64, dev = muse
    wl = synth.WORKLOADS["muse-bf16-ctx16384-wrap"]
    S = max(min(max(8 * block, 32), 128), block)
    # the library stores Cs slots (8-aligned) and rounds the phase down to a multiple of 8:
    # put the first round's append at slot Cs - 8 so its block + 1 >= 9 rows straddle the end
    Cs = (max(SH.window + S, SH.window + block + 1, 64) + 7) // 8 * 8
    phase = (Cs - 8 - wl.context) % Cs
    assert phase % 8 == 0
    ls = P.LockStep(SH, w64, max_block=block, phase=phase, dev_weights=dev)
    ks = P.run_random_depth_rounds(ls, wl.context, block, rounds, tag=block)
    e0 = ls.gpu.cache_state()[0]
    ls.append(synth.resid_rows(SH, S, 90_000 + block))
    ls.trim(S)
    assert ls.gpu.cache_state()[:2] == (e0, 0)
    ks += P.run_random_depth_rounds(ls, 0, block, 2, tag=500 + block, prefill=False)
    _report(f"{wl.name} block {block}", ls, ks)
    first_slot = (wl.context + phase) % Cs
    assert first_slot + block + 1 > Cs  # the first append did straddle the ring end


@pytest.fixture(scope="module")
def muse_q4():
    sh = synth.MUSE_Q4
    w = synth.make_weights(sh)
    dev = binding.to_device(sh, w)
    return w, dev


@pytest.mark.parametrize("block", [4, 5, 8, 16])
def test_q4_ctx2048_width_sweep(muse_q4, block):
    """4-bit Muse-shaped drafter (fc, layers and lm_head in q4, group 64; embedding bf16)
    after a 2048-row context, one ring per width, p-accept stand-in target with the
    width's own p."""
    w, dev = muse_q4
    wl = synth.WORKLOADS["muse-q4-sweep-ctx2048"]
    p = synth.width_accept_p(wl.blocks)[block]
    ls = P.LockStep(wl.shape, w, max_block=block, dev_weights=dev)
    ks = P.run_synthetic_rounds(ls, wl.context, block, wl.rounds, p=p, tag=block)
    _report(f"{wl.name} block {block} p {p:.3f}", ls, ks)
    assert ls.stats.max_hidden_rel <= 2e-3


def test_q4_ctx2048_deferred_kv(muse_q4):
    """4-bit Muse-shaped drafter at block 4 with the verified rows' K/V projected inside the
    next draft (window read back every third trim and at the end)."""
    w, dev = muse_q4
    wl = synth.WORKLOADS["muse-q4-sweep-ctx2048"]
    ls = P.LockStep(wl.shape, w, max_block=4, dev_weights=dev, window_period=3)
    ks = P.run_random_depth_rounds(ls, wl.context, 4, 8, tag=41)
    torch.cuda.synchronize()
    ls.check_window()
    _report(f"{wl.name} block 4 deferred", ls, ks)
    assert ls.stats.max_hidden_rel <= 2e-3
