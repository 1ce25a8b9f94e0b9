"""GPU parity: the HIP path through the C-ABI against the CPU oracle, element by element."""
import ctypes

import numpy as np
import pytest
import torch

from block_drafting_dflash_amd import binding, synth
from tests import parity as P

pytestmark = pytest.mark.gpu

# small shapes that still span several MFMA tiles and ragged tails
MICRO_F32 = synth.Shape(hidden=256, layers=2, q_heads=4, kv_heads=2, head_dim=64, intermediate=384,
                        vocab=1040, target_streams=3, target_width=128, window=9,
                        weight_dtype="f32", act_dtype="f32")
MICRO_BF16 = synth.Shape(hidden=512, layers=2, q_heads=8, kv_heads=2, head_dim=64, intermediate=768,
                         vocab=3008, target_streams=2, target_width=256, window=20,
                         weight_dtype="bf16", act_dtype="bf16")


MICRO_Q4 = MICRO_BF16.with_(weight_dtype="q4")


@pytest.fixture(scope="module")
def micro_q4_w():
    return synth.make_weights(MICRO_Q4)


@pytest.fixture(scope="module")
def tiny_w():
    return synth.make_weights(synth.TINY_F32)


@pytest.fixture(scope="module")
def micro_f32_w():
    return synth.make_weights(MICRO_F32)


@pytest.fixture(scope="module")
def micro_bf16_w():
    return synth.make_weights(MICRO_BF16)


def test_tiny_f32_rounds_match_oracle(tiny_w):
    wl = synth.WORKLOADS["tiny-f32-b4-ctx64"]
    ls = P.LockStep(wl.shape, tiny_w, max_block=4)
    P.run_lm_head_rounds(ls, wl.context, 4, wl.rounds)
    assert ls.stats.max_hidden_rel <= 1e-4
    print("tiny-f32 stats", ls.stats)


@pytest.mark.parametrize("block,phase", [(1, 0), (3, 5), (8, -1)])
def test_micro_f32_synthetic_accept(micro_f32_w, block, phase):
    C = MICRO_F32.window + max(min(max(8 * block, 32), 128), block)
    ls = P.LockStep(MICRO_F32, micro_f32_w, max_block=block, phase=phase % C)
    ks = P.run_synthetic_rounds(ls, 23, block, 12, p=0.7, tag=block)
    assert any(k > 0 for k in ks)


# blocks 63 and 64 put the block's own keys into two or three 64-position chunks of the
# attention (window 20), and the GEMMs into two launches of rows
@pytest.mark.parametrize("block,phase,context",
                         [(4, 0, 50), (16, 3, 7), (17, 60, 33), (40, 0, 100), (63, 8, 70), (64, 16, 130)])
def test_micro_bf16_random_depth(micro_bf16_w, block, phase, context):
    ls = P.LockStep(MICRO_BF16, micro_bf16_w, max_block=block, phase=phase)
    P.run_random_depth_rounds(ls, context, block, 10, tag=block)
    print("micro-bf16 stats", block, ls.stats)


def check_argmax_against_oracle(sh, w, got, rows):
    """Verify-row argmaxes against the oracle's, exact above the near-tie margin."""
    from oracle import dflash_oracle as O

    oi, om = O.OracleDrafter(sh, w, 4).lm_head_argmax(rows)
    got = got.numpy()
    for i in range(len(rows)):
        assert om[i] <= P.MARGIN or got[i] == oi[i], (i, got[i], oi[i], om[i])


def test_lm_head_argmax_is_width_invariant(micro_bf16_w):
    """The verify-row argmax over 40, 48 and 49 rows (one, two and three 16-row tiles per
    launch, and a second launch past 48 rows) against the oracle, and bit-identical to the
    same rows taken in narrower calls."""
    sh = MICRO_BF16
    dev = binding.to_device(sh, micro_bf16_w)
    g = binding.Drafter(sh, dev, max_block=4)
    for n in (40, 48, 49):
        rows_np = synth.verify_hidden(sh, n, n)
        rows = torch.from_numpy(rows_np).to(torch.bfloat16).cuda()
        full = g.lm_head_argmax(rows).cpu()
        check_argmax_against_oracle(sh, micro_bf16_w, full, rows_np)
        for wd in (1, 4, 5, 16, 17, 33):
            part = torch.cat([g.lm_head_argmax(rows[i:i + wd].contiguous()).cpu() for i in range(0, n, wd)])
            assert torch.equal(part, full), (n, wd)


def test_draft_is_bit_reproducible(micro_bf16_w):
    sh = MICRO_BF16
    dev = binding.to_device(sh, micro_bf16_w)
    outs = []
    for _ in range(2):
        g = binding.Drafter(sh, dev, max_block=8)
        g.cache_append(torch.from_numpy(synth.resid_rows(sh, 30, 0)).to(torch.bfloat16).cuda(), commit=True)
        h = torch.empty((9, sh.hidden), dtype=torch.float32, device="cuda")
        t = g.draft_block(5, 8, hidden=h)
        outs.append((t.cpu(), h.cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_verify_result_into_pinned_host_memory(micro_f32_w):
    """The verify kernel writes (k, bonus, status) straight into pinned host memory: the same
    words as a device buffer, for accepted lengths 0..B and an out-of-range target id."""
    sh, B = MICRO_F32, 5
    g = binding.Drafter(sh, binding.to_device(sh, micro_f32_w), max_block=B)
    host = torch.full((3,), -7, dtype=torch.int32).pin_memory()
    d = torch.tensor([3, 1, 4, 1, 5], dtype=torch.int32, device="cuda")
    cases = [P.target_with_accept_length(d.cpu().numpy(), k, sh.vocab, tail=11 + k) for k in range(B + 1)]
    cases.append(np.array([3, sh.vocab + 2, 0, 0, 0, 0]))
    for a in cases:
        t = torch.from_numpy(a.astype(np.int32)).cuda()
        want = g.verify_greedy(d, t, B).cpu().tolist()
        host.fill_(-7)
        g.verify_greedy(d, t, B, out=host)
        torch.cuda.synchronize()
        assert host.tolist() == want, (a, want)
    with pytest.raises(ValueError):
        g.verify_greedy(d, t, B, out=torch.empty(3, dtype=torch.int32))  # not pinned


def test_verify_kernel_matches_oracle_across_widths(micro_f32_w):
    """Greedy verify through the C-ABI against the oracle's rule at widths on both sides of
    one wave's 64 rows (one ballot below 64 draft rows, several 64-row passes from 64 on):
    every accepted length 0..B at the small widths, sampled ones past them, and an
    out-of-range target id at the first, a middle and the bonus row, which refuses the
    whole block."""
    from oracle import dflash_oracle as O

    sh = MICRO_F32
    g = binding.Drafter(sh, binding.to_device(sh, micro_f32_w), max_block=200)
    rng = np.random.default_rng(77)
    for B in (1, 2, 5, 31, 63, 64, 65, 127, 128, 200):
        ks = range(B + 1) if B <= 8 else sorted({0, 1, B // 2, B - 1, B, int(rng.integers(0, B + 1))})
        for k in ks:
            d = rng.integers(0, sh.vocab, B).astype(np.int32)
            a = P.target_with_accept_length(d, k, sh.vocab, tail=int(rng.integers(0, sh.vocab))).astype(np.int32)
            got = g.verify_greedy(torch.from_numpy(d).cuda(), torch.from_numpy(a).cuda(), B).cpu().tolist()
            want = list(O.verify_greedy(d, a))
            assert got == want + [0], (B, k, got, want)
        for pos, bad in ((0, sh.vocab), (B // 2, -1), (B, sh.vocab + 3)):
            a = rng.integers(0, sh.vocab, B + 1).astype(np.int32)
            a[pos] = bad
            got = g.verify_greedy(torch.from_numpy(d).cuda(), torch.from_numpy(a).cuda(), B).cpu().tolist()
            assert got == [0, -1, 1], (B, pos, got)


def test_boundary_errors_leave_state_unchanged(micro_f32_w):
    sh = MICRO_F32
    g = binding.Drafter(sh, binding.to_device(sh, micro_f32_w), max_block=4)
    with pytest.raises(binding.DFlashError) as e:
        g.draft_block(1, 4)
    assert e.value.status == 4  # no context
    g.cache_append(torch.from_numpy(synth.resid_rows(sh, 12, 0)).cuda(), commit=True)
    st = g.cache_state()
    for call, status in [(lambda: g.draft_block(1, 5), 3), (lambda: g.draft_block(1, 0), 3),
                         (lambda: g.draft_block(sh.vocab, 2), 3), (lambda: g.cache_trim(1), 5)]:
        with pytest.raises(binding.DFlashError) as e:
            call()
        assert e.value.status == status
        assert g.cache_state() == st
    g.cache_append(torch.from_numpy(synth.resid_rows(sh, 3, 1)).cuda())
    with pytest.raises(binding.DFlashError) as e:
        g.draft_block(1, 2)
    assert e.value.status == 6
    with pytest.raises(binding.DFlashError) as e:
        g.cache_trim(4)
    assert e.value.status == 5
    g.cache_trim(2)
    assert g.cache_state()[:2] == (13, 0)
    # out-of-range target ids are reported by the verify status word
    out = g.verify_greedy(torch.tensor([1, 2], dtype=torch.int32, device="cuda"),
                          torch.tensor([1, sh.vocab, 0], dtype=torch.int32, device="cuda"), 2)
    assert out.cpu().tolist() == [0, -1, 1]


def test_outputs_do_not_depend_on_ring_phase(micro_bf16_w):
    """Drafted tokens, hidden rows and the live window are bit-identical for ring phases
    0, 1, C-1 and a random one: the slot of a position never changes what is computed."""
    sh, block, context, rounds = MICRO_BF16, 8, 50, 12
    C = sh.window + max(min(max(8 * block, 32), 128), block)
    dev = binding.to_device(sh, micro_bf16_w)
    phases = (0, 1, C - 1, int(np.random.default_rng(synth.SEED_PHASE).integers(2, C - 1)))
    runs = []
    for phase in phases:
        g = binding.Drafter(sh, dev, max_block=block, phase=phase)
        g.cache_append(torch.from_numpy(synth.resid_rows(sh, context, 0)).to(torch.bfloat16).cuda(), commit=True)
        anchor, outs = synth.anchor_token(sh), []
        for r in range(rounds):
            h = torch.empty((block + 1, sh.hidden), dtype=torch.float32, device="cuda")
            d = g.draft_block(anchor, block, hidden=h).cpu().numpy()
            a = P.target_with_accept_length(d, synth.random_depth_k(block, r), sh.vocab, tail=r)
            out = g.verify_greedy(torch.from_numpy(d).cuda(), torch.from_numpy(a.astype(np.int32)).cuda(), block)
            k, bonus, _ = out.cpu().tolist()
            g.cache_append(torch.from_numpy(synth.resid_rows(sh, block + 1, r + 1)).to(torch.bfloat16).cuda())
            g.cache_trim(block - k)
            outs.append((d, h.cpu(), k))
            anchor = bonus
        kv = [g.cache_read(l) for l in range(sh.layers)]
        runs.append((outs, [(k.cpu(), v.cpu()) for k, v in kv], g.cache_state()))
    for phase, (outs, kv, st) in zip(phases[1:], runs[1:]):
        assert st == runs[0][2], phase
        for (d0, h0, k0), (d1, h1, k1) in zip(runs[0][0], outs):
            assert np.array_equal(d0, d1) and k0 == k1 and torch.equal(h0, h1), phase
        for (k0, v0), (k1, v1) in zip(runs[0][1], kv):
            assert torch.equal(k0, k1) and torch.equal(v0, v1), phase


# the verified rows' K/V travel with the next draft (its QKV launches project them beside
# the draft rows, its attention writes them into the ring) while draft rows + committed rows
# fit a launch's two row tiles (32; past 16 staged in two phases); the window is read back
# only every third trim, so most rounds take that path, and block 24 takes it only when at
# most seven rows were committed
@pytest.mark.parametrize("block,phase,context", [(1, 0, 21), (4, 5, 50), (8, 16, 40), (13, 3, 64), (16, 7, 30),
                                                 (24, 0, 45)])
def test_micro_bf16_deferred_kv_rounds(micro_bf16_w, block, phase, context):
    ls = P.LockStep(MICRO_BF16, micro_bf16_w, max_block=block, phase=phase, window_period=3)
    P.run_random_depth_rounds(ls, context, block, 14, tag=200 + block)
    torch.cuda.synchronize()
    ls.check_window()
    print("micro-bf16 deferred stats", block, ls.stats)


def test_deferred_kv_call_sequences(micro_bf16_w):
    """Sequences the round loop never makes, in lock-step with the oracle: a read-back
    between an append and its trim, two pending appends before one trim, a committing
    append over deferred rows, a draft whose rows and the committed ones take two row tiles
    (folded, staged in two phases) and one where they pass a launch's 32 rows (the rows are
    projected on their own first)."""
    sh = MICRO_BF16
    ls = P.LockStep(sh, micro_bf16_w, max_block=30, phase=16, check_windows=False)
    ls.append(synth.resid_rows(sh, 27, 0), commit=True)
    anchor = synth.anchor_token(sh, tag=9)
    ls.draft(anchor, 4)
    ls.append(synth.resid_rows(sh, 5, 1))  # deferred
    ls.check_window()  # read-back projects the pending rows
    ls.trim(2)
    ls.draft((anchor + 1) % sh.vocab, 4)  # nothing left to fold
    ls.append(synth.resid_rows(sh, 5, 2))  # deferred
    ls.append(synth.resid_rows(sh, 3, 3))  # projects the first five, defers these three
    ls.trim(4)  # keeps 5 + 3 - 4 = 4 rows, of them 0 deferred
    ls.draft((anchor + 2) % sh.vocab, 8)
    ls.append(synth.resid_rows(sh, 9, 4))  # deferred
    ls.trim(1)  # 8 committed rows
    ls.draft((anchor + 3) % sh.vocab, 13)  # 14 + 8 rows: two row tiles, folded in two phases
    ls.append(synth.resid_rows(sh, 3, 5))  # deferred
    ls.trim(0)
    ls.append(synth.resid_rows(sh, 6, 6), commit=True)  # projects them, then these six
    ls.draft((anchor + 4) % sh.vocab, 1)
    ls.append(synth.resid_rows(sh, 9, 7))  # deferred
    ls.trim(1)  # 8 committed rows
    ls.draft((anchor + 5) % sh.vocab, 27)  # 28 + 8 rows > 32: projected first
    ls.append(synth.resid_rows(sh, 2, 8))  # deferred
    ls.trim(1)
    ls.draft((anchor + 6) % sh.vocab, 6)  # folds the one committed row
    torch.cuda.synchronize()
    ls.check_window()
    print("deferred sequences stats", ls.stats)


@pytest.mark.parametrize("block", [4, 8, 16])
def test_deferred_kv_matches_immediate_projection(micro_bf16_w, block):
    """The same rounds with the window read after every trim (the verified rows' K/V
    projected on their own, by the append path's kernels) and never (projected inside the
    next draft): drafted tokens, hidden rows and the final window are bit-identical."""
    sh, context, rounds = MICRO_BF16, 45, 12
    dev = binding.to_device(sh, micro_bf16_w)
    runs = []
    for read_back in (True, False):
        g = binding.Drafter(sh, dev, max_block=block, phase=8)
        g.cache_append(torch.from_numpy(synth.resid_rows(sh, context, 0)).to(torch.bfloat16).cuda(), commit=True)
        anchor, outs = synth.anchor_token(sh), []
        for r in range(rounds):
            h = torch.empty((block + 1, sh.hidden), dtype=torch.float32, device="cuda")
            d = g.draft_block(anchor, block, hidden=h).cpu().numpy()
            a = P.target_with_accept_length(d, synth.random_depth_k(block, r, 7), sh.vocab, tail=r)
            out = g.verify_greedy(torch.from_numpy(d).cuda(), torch.from_numpy(a.astype(np.int32)).cuda(), block)
            k, bonus, _ = out.cpu().tolist()
            g.cache_append(torch.from_numpy(synth.resid_rows(sh, block + 1, 300 + r)).to(torch.bfloat16).cuda())
            g.cache_trim(block - k)
            if read_back:
                for l in range(sh.layers):
                    g.cache_read(l)
            outs.append((d, h.cpu(), k))
            anchor = bonus
        kv = [g.cache_read(l) for l in range(sh.layers)]
        runs.append((outs, [(k.cpu(), v.cpu()) for k, v in kv], g.cache_state()))
    (o0, kv0, st0), (o1, kv1, st1) = runs
    assert st0 == st1
    for (d0, h0, k0), (d1, h1, k1) in zip(o0, o1):
        assert np.array_equal(d0, d1) and k0 == k1 and torch.equal(h0, h1)
    for (k0, v0), (k1, v1) in zip(kv0, kv1):
        assert torch.equal(k0, k1) and torch.equal(v0, v1)


@pytest.mark.parametrize("block,phase,context", [(4, 0, 50), (16, 7, 30), (17, 0, 9), (40, 3, 64)])
def test_micro_q4_random_depth(micro_q4_w, block, phase, context):
    """4-bit fc, layer linears and lm_head (group 64): the codes enter the MFMA as exact
    integers and each group is rescaled; the oracle dequantizes w = s q + b exactly."""
    ls = P.LockStep(MICRO_Q4, micro_q4_w, max_block=block, phase=phase)
    P.run_random_depth_rounds(ls, context, block, 10, tag=block)
    assert ls.stats.max_hidden_rel <= 2e-3, ls.stats
    print("micro-q4 stats", block, ls.stats)


@pytest.mark.parametrize("block,phase,context", [(4, 0, 50), (8, 24, 33)])
def test_micro_q4_deferred_kv_rounds(micro_q4_w, block, phase, context):
    """4-bit layers with the verified rows' K/V projected inside the next draft (window read
    back every third trim and at the end)."""
    ls = P.LockStep(MICRO_Q4, micro_q4_w, max_block=block, phase=phase, window_period=3)
    P.run_random_depth_rounds(ls, context, block, 12, tag=300 + block)
    torch.cuda.synchronize()
    ls.check_window()
    assert ls.stats.max_hidden_rel <= 2e-3, ls.stats


def test_q4_lm_head_argmax_is_width_invariant(micro_q4_w):
    sh = MICRO_Q4
    g = binding.Drafter(sh, binding.to_device(sh, micro_q4_w), max_block=4)
    for n in (40, 49):
        rows_np = synth.verify_hidden(sh, n, n)
        rows = torch.from_numpy(rows_np).to(torch.bfloat16).cuda()
        full = g.lm_head_argmax(rows).cpu()
        check_argmax_against_oracle(sh, micro_q4_w, full, rows_np)
        for wd in (1, 5, 16, 17):
            part = torch.cat([g.lm_head_argmax(rows[i:i + wd].contiguous()).cpu() for i in range(0, n, wd)])
            assert torch.equal(part, full), (n, wd)


def test_argmax_timing_hook(micro_bf16_w):
    """dflash_time_next_argmax: the events bracket the argmax kernel of the next lm_head call
    only (positive, and no longer than the whole call), leave its result unchanged, apply
    to one call, and a single NULL event is rejected."""
    sh = MICRO_BF16
    g = binding.Drafter(sh, binding.to_device(sh, micro_bf16_w), max_block=4)
    rows = torch.from_numpy(np.stack([synth.verify_hidden(sh, 5, r) for r in range(3)])).to(torch.bfloat16).cuda()
    plain = g.lm_head_argmax(rows[0]).cpu()
    stream = torch.cuda.current_stream()
    k0, k1, c0, c1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    g.time_next_argmax(k0, k1)
    c0.record(stream)
    timed = g.lm_head_argmax(rows[0]).cpu()
    c1.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(plain, timed)
    kernel_ms, call_ms = k0.elapsed_time(k1), c0.elapsed_time(c1)
    assert 0.0 < kernel_ms <= call_ms
    # the request is spent: the next call records nothing new
    g.lm_head_argmax(rows[1])
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == kernel_ms
    assert binding.lib().dflash_time_next_argmax(g.ctx, ctypes.c_void_p(k0.cuda_event), None) == 1  # DFLASH_E_ARG


def test_lm_head_exact_tie_goes_to_the_lowest_index(micro_bf16_w):
    """Two bit-identical lm_head rows give bit-identical logits, and the argmax takes the lower
    index (the first maximum), on the verify-row path (one bf16 operand plane) and on the
    drafted rows (final norm, hi/lo operand pairs); the oracle agrees with margin exactly 0."""
    from oracle import dflash_oracle as O

    sh = MICRO_BF16
    lm0 = micro_bf16_w["lm_head"]
    # verify rows: row 0 points along lm_head row t, whose copy sits at the end of the table
    t, s = 7, sh.vocab - 5
    lm = lm0.copy()
    lm[s] = lm[t]
    w = dict(micro_bf16_w, lm_head=lm)
    rows = synth.verify_hidden(sh, 45, 11)
    rows[0] = synth.to_bf16_values(lm[t] / np.float32(0.02))
    rows[41] = rows[0]  # the same tie in the third row tile of the launch
    g = binding.Drafter(sh, binding.to_device(sh, w), max_block=4)
    got = g.lm_head_argmax(torch.from_numpy(rows).to(torch.bfloat16).cuda()).cpu().numpy()
    oi, om = O.OracleDrafter(sh, w, 4).lm_head_argmax(rows)
    for i in (0, 41):
        assert om[i] == 0.0 and oi[i] == t and got[i] == t, i
    for i in range(1, len(rows)):
        assert om[i] <= P.MARGIN or got[i] == oi[i]
    # drafted rows: copy the winner v of a clearly decided drafted row into a lower, unused row
    prefill = synth.resid_rows(sh, 30, 0)
    anchor = 5
    od = O.OracleDrafter(sh, micro_bf16_w, 4)
    od.append(prefill, commit=True)
    ref = od.draft(anchor, 4)
    g0 = binding.Drafter(sh, binding.to_device(sh, micro_bf16_w), max_block=4)
    g0.cache_append(torch.from_numpy(prefill).to(torch.bfloat16).cuda(), commit=True)
    d0 = g0.draft_block(anchor, 4).cpu().numpy()
    j = next(j for j in range(4) if ref.margins[j] > P.MARGIN and d0[j] == ref.tokens[j] and d0[j] > 8)
    v = int(d0[j])
    m = min(set(range(v)) - set(int(x) for x in d0))
    lm2 = lm0.copy()
    lm2[m] = lm2[v]
    w2 = dict(micro_bf16_w, lm_head=lm2)
    g2 = binding.Drafter(sh, binding.to_device(sh, w2), max_block=4)
    g2.cache_append(torch.from_numpy(prefill).to(torch.bfloat16).cuda(), commit=True)
    d2 = g2.draft_block(anchor, 4).cpu().numpy()
    od2 = O.OracleDrafter(sh, w2, 4)
    od2.append(prefill, commit=True)
    r2 = od2.draft(anchor, 4)
    assert r2.tokens[j] == m and r2.margins[j] == 0.0
    assert d2[j] == m
    for i in range(4):
        assert d2[i] == (m if d0[i] == v else d0[i]), (i, d0, d2)


def test_append_without_a_residual_stream_is_refused(micro_f32_w):
    """dflash_cache_append through the C-ABI with a NULL slab, zero rows or a negative count:
    DFLASH_E_ARG ("no residual stream captured"), nothing enqueued, offsets unchanged; a real
    append afterwards still matches the oracle."""
    sh = MICRO_F32
    ls = P.LockStep(sh, micro_f32_w, max_block=4)
    L = binding.lib()
    stream = torch.cuda.current_stream().cuda_stream
    rows = torch.from_numpy(synth.resid_rows(sh, 4, 0)).cuda()
    st0 = ls.gpu.cache_state()
    for ptr, n in [(None, 4), (None, 0), (rows.data_ptr(), 0), (rows.data_ptr(), -2)]:
        for commit in (0, 1):
            assert L.dflash_cache_append(ls.gpu.ctx, ptr, n, commit, stream) == 1  # DFLASH_E_ARG
            assert b"no residual stream captured" in L.dflash_last_error(ls.gpu.ctx)
            assert ls.gpu.cache_state() == st0
    ls.append(synth.resid_rows(sh, 13, 0), commit=True)
    torch.cuda.synchronize()
    ls.check_window()


def test_micro_bf16_block129_deepest_rewind(micro_bf16_w):
    """Block 129: the slack is 129 rows (the block floor past the 128 cap). Rounds that accept
    nothing rewind 129 of the 130 appended rows, the deepest rewind a round makes; after
    every trim the live window is read back and compared with the oracle, and the next
    draft sees no corrupted key."""
    sh, B = MICRO_BF16, 129
    ls = P.LockStep(sh, micro_bf16_w, max_block=B, phase=8)
    assert ls.gpu.cache_state()[2] == B
    ls.append(synth.resid_rows(sh, 40, 0), commit=True)
    torch.cuda.synchronize()
    ls.check_window()
    anchor = synth.anchor_token(sh, tag=129)
    for r, kk in enumerate([0, 0, 5, B, 0]):
        d = ls.draft(anchor, B)
        a = P.target_with_accept_length(d, kk, sh.vocab, tail=anchor + r)
        k, bonus = ls.verify(d, a)
        assert k == kk
        ls.append(synth.resid_rows(sh, B + 1, 700 + r))
        ls.trim(B - k)
        anchor = bonus
    print("block 129 stats", ls.stats)


def test_micro_bf16_block256_widest_block(micro_bf16_w):
    """Block 256, the widest a context takes: 257 draft rows (nine row launches per GEMM, the
    normed operands through the row-norm planes, 65 query tiles per kv head, eight argmax
    launches of 32 rows), slack 256; rounds that accept nothing, everything and a few rows,
    with the live window read back after every trim."""
    sh, B = MICRO_BF16, 256
    ls = P.LockStep(sh, micro_bf16_w, max_block=B, phase=16)
    assert ls.gpu.cache_state()[2] == B
    ls.append(synth.resid_rows(sh, 33, 0), commit=True)
    torch.cuda.synchronize()
    ls.check_window()
    anchor = synth.anchor_token(sh, tag=256)
    for r, kk in enumerate([0, B, 17]):
        d = ls.draft(anchor, B)
        a = P.target_with_accept_length(d, kk, sh.vocab, tail=anchor + r)
        k, bonus = ls.verify(d, a)
        assert k == kk
        ls.append(synth.resid_rows(sh, B + 1, 900 + r))
        ls.trim(B - k)
        anchor = bonus
    print("block 256 stats", ls.stats)


def test_micro_bf16_widest_window(micro_bf16_w):
    """Window 4096, the widest a context takes, full after a 4400-row prefill (the rows before
    the window dropped ahead of the encoder): a query's keys span 66-67 chunks of 64, so the
    combine merges the most partials it takes; block 16, rounds of random accept length with
    the whole live window read back after every trim, across the ring's wrap point."""
    sh, B = MICRO_BF16.with_(window=4096), 16
    ls = P.LockStep(sh, micro_bf16_w, max_block=B, phase=4000)
    ls.append(synth.resid_rows(sh, 4400, 0), commit=True)
    torch.cuda.synchronize()
    ls.check_window()
    anchor = synth.anchor_token(sh, tag=4096)
    rng = np.random.default_rng(4096)
    for r in range(3):
        d = ls.draft(anchor, B)
        kk = int(rng.integers(0, B + 1))
        a = P.target_with_accept_length(d, kk, sh.vocab, tail=anchor + r)
        k, bonus = ls.verify(d, a)
        assert k == kk
        ls.append(synth.resid_rows(sh, B + 1, 4500 + r))
        ls.trim(B - k)
        anchor = bonus
    print("window 4096 stats", ls.stats)


@pytest.mark.parametrize("p,widens", [(0.95, True), (0.3, False)])
def test_adaptive_width_rounds_match_oracle(micro_bf16_w, p, widens):
    """Rounds whose block the library's width controller picks (depth 4, ceiling 16, windows of
    4 rounds, a challenge after every 2): drafts at both widths in lock-step with the oracle
    drafter (the ring sized for the ceiling), and the controller's decisions replayed through
    the oracle controller. Round times are a fixed model (0.1 + 0.02 * block ms), so a high
    accept probability makes the ceiling pay and a low one does not."""
    from oracle.width_controller import WidthController as OracleController

    sh = MICRO_BF16
    ctl = binding.WidthController(4, 16, 4, 2)
    orc = OracleController(4, 16, 4, 2)
    ls = P.LockStep(sh, micro_bf16_w, max_block=16, phase=24, window_period=5)
    ls.append(synth.resid_rows(sh, 48, 0), commit=True)
    anchor = synth.anchor_token(sh, tag=77)
    used = set()
    for r in range(48):
        b = ctl.width()
        assert b == orc.width()
        used.add(b)
        d = ls.draft(anchor, b)
        a = synth.synthetic_target_argmax(d, synth.accept_draws(b, r, 77), p, sh.vocab)
        k, bonus = ls.verify(d, a)
        ls.append(synth.resid_rows(sh, b + 1, 9000 + r))
        ls.trim(b - k)
        ms = 0.1 + 0.02 * b
        ctl.record(b, k + 1, ms)
        orc.record(b, k + 1, ms)
        anchor = bonus
    st = ctl.state()
    assert st["incumbent"] == orc.incumbent and st["adoptions"] == sum(x[3] for x in orc.decisions)
    assert used == {4, 16}
    assert (st["incumbent"] == 16) == widens
    print("adaptive", p, st, ls.stats)
