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


@pytest.fixture(scope="module")
def muse_pair():
    """The Muse-shaped target (10 layers, window 2048, full layers 4 and 9, streams captured
    at layers 1, 3, 5, 7, 9) and the drafter it feeds (fc 5 x 2048 -> 2048), sharing the
    embedding table and lm_head."""
    t = synth.MUSE_BF16_TARGET
    dsh = synth.drafter_for(t, SH)
    dw = synth.make_weights(dsh)
    tw = synth.make_target_weights(t, dw)
    ddev = binding.to_device(dsh, dw)
    tdev = binding.to_device(t, {k: v for k, v in tw.items() if k not in ("embed", "lm_head")})
    tdev["embed"], tdev["lm_head"] = ddev["embed"], ddev["lm_head"]  # one device copy, shared
    f64 = lambda w: {k: (np.asarray(v, dtype=np.float64) if k != "embed" and getattr(v, "ndim", 0) == 2 else v)
                     for k, v in w.items()}
    dw64 = f64(dw)
    tw64 = {k: (dw64[k] if k in ("embed", "lm_head") else v) for k, v in f64(tw).items()}
    return t, dsh, dw64, tw64, ddev, tdev


def test_muse_target_rounds_match_oracles(muse_pair):
    """A 256-token prompt through the target in 32-row forwards (captured streams committed to
    the drafter), then rounds at block 4 with the drafter's own proposals: the target's
    verify argmaxes and captured streams, the drafter's tokens and hidden rows, the verify
    result and both caches' offsets in lock-step with the oracles; every target cache window
    and the drafter's live window at the end."""
    from tests.test_gpu_target import TargetLockStep

    t, dsh, dw64, tw64, ddev, tdev = muse_pair
    B = 4
    tls = TargetLockStep(t, tw64, max_block=B, dev=tdev)
    dls = P.LockStep(dsh, dw64, max_block=B, dev_weights=ddev, check_windows=False)
    prompt = [int(x) for x in synth.prompt_tokens(t.vocab, 256, tag=11)]
    for s in range(0, len(prompt), tls.gpu.rows_max):
        a, cap = tls.forward(prompt[s:s + tls.gpu.rows_max])
        tls.trim(0)
        # the drafter takes the oracle's captured rows: the same bits the GPU's are compared to
        dls.append(tls.orc_last_capture, commit=True)
    anchor = int(a[-1])
    for r in range(8):
        d = dls.draft(anchor, B)
        a, cap = tls.forward([anchor] + [int(x) for x in d])
        k, bonus = dls.verify(d, a)
        dls.append(tls.orc_last_capture)
        dls.trim(B - k)
        tls.trim(B - k)
        anchor = bonus
    tls.check_caches()
    torch.cuda.synchronize()
    dls.check_window()
    print("muse target rounds: near ties", tls.near_ties, "drafter", dls.stats)


def test_muse_speculative_loop_commits_the_tokens_of_classic_decoding(muse_pair):
    """The identity property at the Muse-shaped sizes, on the GPU alone: the speculative round
    loop commits bit-for-bit the tokens of classic greedy decoding of the same target."""
    from tests.test_gpu_target import run_classic, run_speculative

    t, dsh, _, _, ddev, tdev = muse_pair
    prompt = [int(x) for x in synth.prompt_tokens(t.vocab, 300, tag=12)]
    want = run_classic(t, tdev, prompt, 24)
    got, ks = run_speculative(t, dsh, tdev, ddev, prompt, 24, 4)
    assert got == want


@pytest.mark.parametrize("gamma", [7, 9])
def test_dspark_w8_w10_ctx1024_lm_head_verify(muse, gamma):
    """The DSpark form of the Muse-shaped drafter (rank-256 Markov head over the 202048-row
    vocabulary, adjacent-pair RoPE, window 4096) at verify widths 8 and 10, after a 1024-row
    context, verify rows through the shared lm_head: every chain step (from the GPU's own
    previous token), the hidden rows, the verify result, the offsets and the live window of
    all five layers after every trim."""
    w64, dev = muse
    wl = synth.WORKLOADS["muse-dspark-bf16-w8-w10-ctx1024"]
    sh = wl.shape
    w = dict(w64)
    dd = dict(dev)
    for name in ("markov_w1", "markov_w2"):
        m = synth.to_bf16_values(synth.draw_tensor(sh, name))
        w[name] = m.astype(np.float64)
        dd[name] = torch.from_numpy(m).to(torch.bfloat16).cuda()
    ls = P.LockStep(sh, w, max_block=gamma, dev_weights=dd)
    ks = P.run_lm_head_rounds(ls, wl.context, gamma, 6, anchor_tag=gamma)
    _report(f"{wl.name} gamma {gamma}", ls, ks)
    assert ls.stats.rows_checked == 6 * (gamma + gamma + 1)


def test_batch_of_four_ctx1024_lm_head_verify(muse):
    """Four independent Muse-shaped sequences drafted together at block 4 (20 rows per GEMM:
    the normed operands go through the row-norm planes), after contexts of 1024, 1000, 977 and
    1031 rows; verify rows through the shared lm_head; each sequence in lock-step with its
    own copy of the oracle (tokens, hidden rows, verify result, offsets, live windows)."""
    from tests.test_gpu_batch import BatchLockStep

    w64, dev = muse
    n, B = 4, 4
    ls = BatchLockStep(SH, w64, n, B, dev=dev)
    ls.append([synth.resid_rows(SH, c, 40 + s) for s, c in enumerate((1024, 1000, 977, 1031))], commit=True)
    anchors = [synth.anchor_token(SH, tag=60 + s) for s in range(n)]
    for r in range(4):
        d = ls.draft(anchors, B)
        rows = np.concatenate([synth.verify_hidden(SH, B + 1, 700 + 10 * r + s) for s in range(n)])
        a_gpu = ls.gpu.lm_head_argmax(ls._t(rows)).cpu().numpy().reshape(n, B + 1)
        a = []
        for s in range(n):
            oi, om = ls.orc.seqs[s].lm_head_argmax(rows[s * (B + 1):(s + 1) * (B + 1)])
            ls._agree(a_gpu[s], oi, om, f"sequence {s} verify argmax")
            a.append(oi)
        res = ls.verify(d, np.stack(a), B)
        ls.append([synth.resid_rows(SH, B + 1, 800 + 10 * r + s) for s in range(n)])
        ls.trim([B - k for k, _ in res])
        anchors = [bonus for _, bonus in res]
    print("batch of four: near ties", ls.near_ties)
