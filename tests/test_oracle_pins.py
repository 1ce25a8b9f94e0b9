"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the pages print
or state (tests/golden/, each file with its citation), hand-worked values, closed forms,
invariants, brute force on tiny inputs, and torch library routines (F.rms_norm, F.silu,
F.scaled_dot_product_attention with an explicit mask, F.embedding/F.linear, torch's own
float32 -> bfloat16 conversion).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from block_drafting_dflash_amd import synth
from block_drafting_dflash_amd.counters import RoundCounters
from oracle import dflash_oracle as O
from tests.torch_formulation import TorchDrafter

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


MICRO = synth.Shape(hidden=32, layers=2, q_heads=4, kv_heads=2, head_dim=8, intermediate=48,
                    vocab=97, target_streams=2, target_width=16, window=5,
                    weight_dtype="f32", act_dtype="f32", rope_theta=10000.0)
MICRO_BF16 = MICRO.with_(weight_dtype="bf16", act_dtype="bf16")


@pytest.fixture(scope="module")
def micro_w():
    return synth.make_weights(MICRO, threads=2)


@pytest.fixture(scope="module")
def micro_bf16_w():
    return synth.make_weights(MICRO_BF16, threads=2)


# ---------------------------------------------------------------------------------------
# closed forms and hand-worked values
# ---------------------------------------------------------------------------------------

def test_slack_rule_matches_page_table():
    g = gold("slack_table.json")
    for b, s in g["table"].items():
        assert O.speculative_slack(int(b)) == s, b
    # the floor: slack never falls below the block it buffers
    for b in range(1, 400):
        assert O.speculative_slack(b) >= b


def test_round_bf16_hand_values():
    for c in gold("bf16_round_hand.json")["cases"]:
        r = float(O.round_bf16(c["x"]))
        want = np.array([int(c["bits"], 16) << 16], dtype=np.uint32).view(np.float32)[0]
        if math.isinf(want):
            assert math.isinf(r) and r > 0, c
        else:
            assert r == float(want), c


def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormal range
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875], dtype=np.float32),
    ])
    # midpoints exactly: mantissa low half == 0x8000
    u = rng.integers(0x3F000000 >> 16, 0x47000000 >> 16, 2000).astype(np.uint32) << 16 | 0x8000
    x = np.concatenate([x, u.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_rms_norm_and_silu_match_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 33))
    g = 1 + 0.1 * rng.standard_normal(33)
    want = F.rms_norm(torch.from_numpy(x), (33,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), want, rtol=1e-14, atol=0)
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-15)


def test_rope_hand_values_fix_pairing_and_sign():
    g = gold("rope_neox_hand.json")
    for c in g["cases"]:
        x = np.array(c["x"], dtype=np.float64)[None, None, :]
        out = O.rope_neox(x, np.array([c["pos"]]), g["theta"])[0, 0]
        np.testing.assert_allclose(out, c["out"], rtol=0, atol=1e-15)


def test_rope_identities():
    rng = np.random.default_rng(2)
    hd = 16
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    # rotation preserves each pair's norm
    r = O.rope_neox(q, np.array([37]), 1e6)[0, 0]
    half = hd // 2
    np.testing.assert_allclose(r[:half] ** 2 + r[half:] ** 2, q[0, 0, :half] ** 2 + q[0, 0, half:] ** 2, rtol=1e-12)
    # q(m) . k(n) depends only on m - n
    dots = []
    for m, n in [(5, 2), (105, 102), (2003, 2000)]:
        qm = O.rope_neox(q, np.array([m]), 1e4)[0, 0]
        kn = O.rope_neox(k, np.array([n]), 1e4)[0, 0]
        dots.append(qm @ kn)
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)


def test_q4_pack_hand_values_and_quantizer_round_trip():
    g = gold("q4_pack_hand.json")
    words = np.array([[int(w, 16) for w in g["words"]]], dtype=np.uint32)
    deq = O.dequant_q4(words, np.array([[g["scale"]]]), np.array([[g["bias"]]]), g["group"])
    np.testing.assert_array_equal(deq[0], g["dequant"])
    # the synthetic quantizer's output decodes to within half a step of the draws
    rng = np.random.default_rng(3)
    w = (0.02 * rng.standard_normal((6, 128))).astype(np.float32)
    t = synth.quantize_q4(w, 64)
    assert t.packed.shape == (6, 128 * 4 // 32)
    d = O.dequant_q4(t.packed, t.scales, t.biases, 64)
    s = np.repeat(t.scales.astype(np.float64), 64, axis=1)
    # bias and scale are bf16-rounded, so allow the rounding of the bias on top of s/2
    b_err = np.repeat(np.abs(t.biases - w.reshape(6, 2, 64).min(axis=2)), 64, axis=1)
    assert np.all(np.abs(d - w) <= s / 2 + b_err + 16 * s * 2 ** -8 + 1e-12)


def test_argmax_first_max_and_margin():
    logits = np.array([[1.0, 3.0, 3.0, 2.0], [0.5, -1.0, 0.25, 0.5], [-2.0, -1.0, -3.0, -1.5]])
    idx, margin = O.argmax_with_margin(logits)
    assert list(idx) == [1, 0, 1]
    np.testing.assert_allclose(margin, [0.0, 0.0, 0.5])


# ---------------------------------------------------------------------------------------
# the verify rows through the shared lm_head
# ---------------------------------------------------------------------------------------

def _hand_lm_head_drafter(g, act):
    sh = synth.Shape(hidden=g["hidden"], layers=1, q_heads=1, kv_heads=1, head_dim=4, intermediate=4,
                     vocab=len(g["lm_head"]), target_streams=1, target_width=4, window=2,
                     weight_dtype=act, act_dtype=act)
    w = {k: np.array(g[k], dtype=np.float32) for k in ("lm_head", "embed", "final_norm")}
    return O.OracleDrafter(sh, w, 1)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_verify_row_lm_head_argmax_hand_values(act):
    """Hand-worked logits of bf16-exact rows through a 5-row lm_head: plain dot products (no
    norm, no scale), the first index of the maximum on exact ties, and the top-2 margins."""
    g = gold("lm_head_argmax_hand.json")
    od = _hand_lm_head_drafter(g, act)
    rows = np.array(g["rows"], dtype=np.float32)
    np.testing.assert_array_equal(od.lm_head_logits(rows), np.array(g["logits"], dtype=np.float64))
    idx, margin = od.lm_head_argmax(rows)
    assert idx.tolist() == g["argmax"]
    np.testing.assert_array_equal(margin, np.array(g["margin"], dtype=np.float64))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_verify_row_lm_head_argmax_matches_torch_linear(micro_w, micro_bf16_w, act):
    """The verify rows (storage dtype) through torch's F.linear with the shared lm_head, then
    torch.argmax (first maximum) and torch.topk margins, all in float64."""
    sh, w = (MICRO, micro_w) if act == "f32" else (MICRO_BF16, micro_bf16_w)
    rows = synth.verify_hidden(sh, 11, 3)
    od = O.OracleDrafter(sh, w, 4)
    idx, margin = od.lm_head_argmax(rows)
    logits = F.linear(torch.from_numpy(rows.astype(np.float64)), torch.from_numpy(w["lm_head"].astype(np.float64)))
    assert idx.tolist() == torch.argmax(logits, dim=1).tolist()
    top = torch.topk(logits, 2, dim=1).values
    np.testing.assert_allclose(margin, (top[:, 0] - top[:, 1]).numpy(), rtol=1e-12, atol=1e-14)
    # a tie planted by duplicating the winning lm_head row below itself goes to the lower row
    w2 = dict(w)
    lm = w["lm_head"].copy()
    lm[2] = lm[idx[0]]
    w2["lm_head"] = lm
    idx2, margin2 = O.OracleDrafter(sh, w2, 4).lm_head_argmax(rows[:1])
    if idx[0] > 2:
        assert idx2[0] == 2 and margin2[0] == 0.0


# ---------------------------------------------------------------------------------------
# verify, synthetic target and counters
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6])
def test_verify_exhaustive_over_binary_blocks(B):
    for d in itertools.product([0, 1], repeat=B):
        for a in itertools.product([0, 1], repeat=B + 1):
            k, bonus = O.verify_greedy(d, a)
            # brute force: the largest j whose first j draft tokens all match
            kb = max(j for j in range(B + 1) if all(d[i] == a[i] for i in range(j)))
            assert k == kb and 0 <= k <= B
            assert bonus == a[k]
            assert (k == B) == all(d[i] == a[i] for i in range(B))


def test_synthetic_target_accept_distribution():
    B, p, V = 16, 0.6, 202048
    draft = np.arange(100, 100 + B)
    counts = np.zeros(B + 1)
    n = 20000
    for r in range(n):
        u = synth.accept_draws(B, r)
        a = synth.synthetic_target_argmax(draft, u, p, V)
        assert np.all((a[:B] == draft) == (u[0, :B] < p))
        k, _ = O.verify_greedy(draft, a)
        counts[k] += 1
    probs = np.array([p ** j * (1 - p) for j in range(B)] + [p ** B])
    mean = (counts * np.arange(B + 1)).sum() / n
    assert abs(p * (1 - p ** B) / (1 - p) - 1.4996) < 1e-4
    assert abs(mean - 1.4996) < 0.05
    # chi-square over the bins with enough mass (df ~ 8, 99.9% quantile ~ 26)
    m = probs * n >= 5
    exp = np.append(probs[m] * n, probs[~m].sum() * n)
    obs = np.append(counts[m], counts[~m].sum())
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert chi2 < 30, chi2


def test_counter_definitions_reproduce_page_arithmetic():
    for run in gold("page_counters.json")["runs"]:
        c = RoundCounters(rounds=run["rounds"], proposed=run["proposed"], accepted=run["accepted"])
        if "mean_accepted_no_bonus" in run:
            assert round(c.mean_accepted(), 2) == run["mean_accepted_no_bonus"], run["cite"]
        if "mean_accepted_with_bonus" in run:
            assert round(c.mean_accepted_with_bonus(), 2) == run["mean_accepted_with_bonus"], run["cite"]
        if "acceptance" in run:
            assert round(c.acceptance(), 3) == run["acceptance"], run["cite"]
        if "emitted_per_verify" in run:
            assert round(RoundCounters.emitted_per_verify(run["tokens"], run["rounds"]), 3) == run["emitted_per_verify"]
        if "tokens" in run and "mean_accepted_no_bonus" in run:
            assert c.emitted == run["tokens"]  # accepted + one bonus per round


# ---------------------------------------------------------------------------------------
# the drafter and its ring: brute force, library formulation, invariants
# ---------------------------------------------------------------------------------------

def _run_rounds(shape, w, ctx, block, rounds, phase, seed, max_block=None, history=None):
    """Drive prefill + rounds on the oracle; returns (drafter, committed history rows)."""
    rng = np.random.default_rng(seed)
    od = O.OracleDrafter(shape, w, max_block or block, phase=phase)
    hist = [synth.resid_rows(shape, ctx, 0)]
    od.append(hist[0], commit=True)
    anchor = int(rng.integers(0, shape.vocab))
    for r in range(rounds):
        od.draft(anchor, block)
        rows = synth.resid_rows(shape, block + 1, r + 1)
        od.append(rows)
        k = int(rng.integers(0, block + 1))
        od.trim(block - k)
        hist.append(rows[: k + 1])
        anchor = int(rng.integers(0, shape.vocab))
    return od, np.concatenate(hist), anchor


@pytest.mark.parametrize("window,ctx,block,phase", [(5, 3, 2, 0), (5, 12, 3, 4), (3, 20, 4, 1), (2, 9, 1, 0),
                                                    (5, 40, 4, 31)])
def test_forward_matches_torch_formulation_over_rounds(micro_w, window, ctx, block, phase):
    sh = MICRO.with_(window=window)
    od, hist, anchor = _run_rounds(sh, micro_w, ctx, block, rounds=6, phase=phase, seed=window + ctx)
    res = od.draft(anchor, block)
    hid, logits = TorchDrafter(sh, micro_w).forward(hist, anchor, block)
    np.testing.assert_allclose(res.hidden, hid, rtol=1e-11, atol=1e-12)
    idx = np.argmax(logits, axis=1)
    assert np.array_equal(res.tokens, idx)
    np.testing.assert_allclose(res.logits_top, logits[np.arange(block), idx], rtol=1e-11)


def test_forward_bf16_matches_torch_formulation(micro_bf16_w):
    sh = MICRO_BF16
    od, hist, anchor = _run_rounds(sh, micro_bf16_w, 17, 4, rounds=5, phase=3, seed=5)
    res = od.draft(anchor, 4)
    hid, logits = TorchDrafter(sh, micro_bf16_w).forward(hist, anchor, 4)
    # only the cached K/V are rounded to bf16; on these seeded inputs torch's f64 -> f32 ->
    # bf16 conversion rounds every one of them as the oracle's direct rounding does
    np.testing.assert_allclose(res.hidden, hid, rtol=1e-12, atol=1e-12)
    idx = np.argmax(logits, axis=1)
    assert np.array_equal(res.tokens, idx)
    np.testing.assert_allclose(res.logits_top, logits[np.arange(4), idx], rtol=1e-12)


def test_uniform_query_attention_counts_the_inclusive_window(micro_w):
    """W_q = 0 makes every visible key equally weighted: outputs reveal the visible count."""
    sh = MICRO.with_(window=4)
    od = O.OracleDrafter(sh, micro_w, 3)
    od.append(synth.resid_rows(sh, 9, 0), commit=True)
    R = 4
    q = np.zeros((R, sh.q_heads, sh.head_dim))
    kb = np.zeros((R, sh.kv_heads, sh.head_dim))
    # context values 1 on kv head 0 / 2 on kv head 1, block values 0: mean reveals the count
    od.V[0, 0, :, :] = 1.0
    od.V[0, 1, :, :] = 2.0
    vb = np.zeros((R, sh.kv_heads, sh.head_dim))
    qpos = od.e + np.arange(R)
    out = od._attention(0, q, kb, vb, qpos)
    for j in range(R):
        n_ctx = sum(1 for p in range(od.e) if abs(qpos[j] - p) <= 4)
        n_blk = sum(1 for i in range(R) if abs(j - i) <= 4)
        for h in range(sh.q_heads):
            g = h // (sh.q_heads // sh.kv_heads)
            np.testing.assert_allclose(out[j, h], (g + 1.0) * n_ctx / (n_ctx + n_blk), rtol=1e-14)
    # the anchor query at e sees exactly W context rows
    assert sum(1 for p in range(od.e) if abs(qpos[0] - p) <= 4) == 4


def test_zero_layers_reduce_to_lm_head_of_the_embedding(micro_w):
    w = dict(micro_w)
    for l in range(MICRO.layers):
        for t in ("o", "down"):
            w[f"layers.{l}.{t}"] = np.zeros_like(micro_w[f"layers.{l}.{t}"])
    od = O.OracleDrafter(MICRO, w, 4)
    od.append(synth.resid_rows(MICRO, 7, 0), commit=True)
    res = od.draft(11, 4)
    E = torch.from_numpy(micro_w["embed"].astype(np.float64))
    x = F.embedding(torch.tensor([11, MICRO.mask_id, MICRO.mask_id, MICRO.mask_id, MICRO.mask_id]), E)
    np.testing.assert_array_equal(res.hidden, x.numpy())
    z = F.rms_norm(x[1:], (MICRO.hidden,), weight=torch.from_numpy(micro_w["final_norm"].astype(np.float64)), eps=1e-6)
    logits = F.linear(z, torch.from_numpy(micro_w["lm_head"].astype(np.float64))).numpy()
    assert np.array_equal(res.tokens, np.argmax(logits, axis=1))
    assert len(set(res.tokens.tolist())) == 1  # every mask row reads the same token here


def test_full_window_reduces_to_unmasked_attention(micro_w):
    """W past every distance: the masked attention is plain bidirectional SDPA (no mask)."""
    sh = MICRO.with_(window=1000)
    od = O.OracleDrafter(sh, micro_w, 3)
    od.append(synth.resid_rows(sh, 6, 0), commit=True)
    rng = np.random.default_rng(4)
    R = 4
    q = rng.standard_normal((R, sh.q_heads, sh.head_dim))
    kb = rng.standard_normal((R, sh.kv_heads, sh.head_dim))
    vb = rng.standard_normal((R, sh.kv_heads, sh.head_dim))
    out = od._attention(0, q, kb, vb, od.e + np.arange(R))
    pos, K, V = od.live_window(0)
    kall = torch.from_numpy(np.concatenate([K, kb.transpose(1, 0, 2)], axis=1))[None]
    vall = torch.from_numpy(np.concatenate([V, vb.transpose(1, 0, 2)], axis=1))[None]
    want = F.scaled_dot_product_attention(torch.from_numpy(q.transpose(1, 0, 2))[None], kall, vall,
                                          enable_gqa=True)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)


def test_dropping_rows_before_the_encoder_changes_nothing(micro_w):
    """Rows past the window projected or not: same live window, same draft."""
    sh = MICRO.with_(window=5)
    rows = synth.resid_rows(sh, 23, 0)
    a = O.OracleDrafter(sh, micro_w, 4)
    a.append(rows, commit=True)  # drops all but the last W before the encoder
    b = O.OracleDrafter(sh, micro_w, 4)
    for i in range(23):  # every row projected, one at a time, then committed
        b.append(rows[i:i + 1])
        b.trim(0)
    for l in range(sh.layers):
        pa, ka, va = a.live_window(l)
        pb, kb, vb = b.live_window(l)
        assert np.array_equal(pa, pb)
        np.testing.assert_allclose(ka, kb, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(va, vb, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a.draft(3, 4).hidden, b.draft(3, 4).hidden, rtol=1e-12)


@pytest.mark.parametrize("block", [1, 3, 4])
def test_post_trim_window_equals_cache_rebuilt_from_committed_prefix(micro_w, block):
    sh = MICRO.with_(window=6)
    od, hist, anchor = _run_rounds(sh, micro_w, 10, block, rounds=12, phase=2, seed=block)
    fresh = O.OracleDrafter(sh, micro_w, block, phase=0)
    fresh.append(hist, commit=True)
    assert (od.e, od.span) == (fresh.e, fresh.span) == (len(hist), 0)
    for l in range(sh.layers):
        p1, k1, v1 = od.live_window(l)
        p2, k2, v2 = fresh.live_window(l)
        assert np.array_equal(p1, p2)
        np.testing.assert_allclose(k1, k2, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(v1, v2, rtol=1e-13, atol=1e-15)
    r1, r2 = od.draft(anchor, block), fresh.draft(anchor, block)
    assert np.array_equal(r1.tokens, r2.tokens)
    np.testing.assert_allclose(r1.hidden, r2.hidden, rtol=1e-12)


def test_pending_appends_equal_one_append(micro_w):
    """Two pending appends before one trim place their rows at consecutive positions: the
    same offsets, window and next draft as one append of both row sets."""
    sh = MICRO.with_(window=6)
    a = O.OracleDrafter(sh, micro_w, 4)
    b = O.OracleDrafter(sh, micro_w, 4)
    for od in (a, b):
        od.append(synth.resid_rows(sh, 9, 0), commit=True)
    r1, r2 = synth.resid_rows(sh, 3, 1), synth.resid_rows(sh, 2, 2)
    a.append(r1)
    a.append(r2)
    b.append(np.concatenate([r1, r2]))
    assert a.state() == b.state() == (9, 5, a.S, a.C)
    a.trim(1)
    b.trim(1)
    assert a.state()[:2] == b.state()[:2] == (13, 0)
    for l in range(sh.layers):
        pa, ka, va = a.live_window(l)
        pb, kb, vb = b.live_window(l)
        assert np.array_equal(pa, pb)
        np.testing.assert_array_equal(ka, kb)
        np.testing.assert_array_equal(va, vb)
    np.testing.assert_array_equal(a.draft(7, 4).hidden, b.draft(7, 4).hidden)


def test_outputs_do_not_depend_on_ring_phase(micro_w):
    sh = MICRO.with_(window=5)
    C = sh.window + O.speculative_slack(3)
    outs = []
    for phase in [0, 1, C - 1, 17]:
        od, hist, anchor = _run_rounds(sh, micro_w, 8, 3, rounds=9, phase=phase, seed=77)
        outs.append((od.e, od.draft(anchor, 3)))
    for e, r in outs[1:]:
        assert e == outs[0][0]
        assert np.array_equal(r.tokens, outs[0][1].tokens)
        np.testing.assert_allclose(r.hidden, outs[0][1].hidden, rtol=1e-12)


def test_slack_below_the_block_corrupts_the_window_and_the_rewind_is_refused(micro_w):
    """Slack 128 at block 129 (the cap without the floor): the append overwrites a row the
    next window still needs, and the k = 0 rewind of 129 rows exceeds the slack."""
    sh = MICRO.with_(window=6)
    B = 129
    bad = O.OracleDrafter(sh, micro_w, B, slack_override=128)
    bad.append(synth.resid_rows(sh, 10, 0), commit=True)
    bad.draft(0, B)
    bad.append(synth.resid_rows(sh, B + 1, 1))
    with pytest.raises(O.OracleError):
        bad.trim(B - 0)
    bad.e, bad.span = bad.e + 1, 0  # what an unchecked rewind would leave behind
    with pytest.raises(O.OracleError):
        bad.live_window(0)
    good = O.OracleDrafter(sh, micro_w, B)  # the floor: slack 129
    assert good.S == 129
    good.append(synth.resid_rows(sh, 10, 0), commit=True)
    good.draft(0, B)
    good.append(synth.resid_rows(sh, B + 1, 1))
    good.trim(B)
    good.live_window(0)


def test_boundary_errors_leave_state_unchanged(micro_w):
    od = O.OracleDrafter(MICRO, micro_w, 4)
    with pytest.raises(O.OracleError):
        od.draft(1, 4)  # empty context
    with pytest.raises(O.OracleError):
        od.append(np.zeros((0, MICRO.fc_in)))
    with pytest.raises(O.OracleError):
        od.append(np.zeros((2, MICRO.fc_in + 1)))
    od.append(synth.resid_rows(MICRO, 7, 0), commit=True)
    st = od.state()
    for bad in [lambda: od.draft(1, 5), lambda: od.draft(1, 0), lambda: od.draft(MICRO.vocab, 2),
                lambda: od.trim(1)]:
        with pytest.raises(O.OracleError):
            bad()
        assert od.state() == st
    od.append(synth.resid_rows(MICRO, 3, 1))
    with pytest.raises(O.OracleError):
        od.draft(1, 2)  # uncommitted rows pending
    with pytest.raises(O.OracleError):
        od.trim(4)  # more than span
    od.trim(2)
    assert od.state()[:2] == (8, 0)


def test_q4_drafter_equals_the_dequantized_f64_drafter():
    sh = MICRO.with_(weight_dtype="q4", act_dtype="bf16", hidden=64, intermediate=128,
                     target_width=32, group=32)
    wq = synth.make_weights(sh, threads=2)
    wd = {k: (O.dequant_q4(v.packed, v.scales, v.biases, v.group) if hasattr(v, "packed") else v)
          for k, v in wq.items()}
    a = O.OracleDrafter(sh, wq, 3)
    b = O.OracleDrafter(sh.with_(weight_dtype="bf16"), wd, 3)
    rows = synth.resid_rows(sh, 9, 0)
    a.append(rows, commit=True)
    b.append(rows, commit=True)
    ra, rb = a.draft(5, 3), b.draft(5, 3)
    np.testing.assert_array_equal(ra.hidden, rb.hidden)
    np.testing.assert_array_equal(ra.tokens, rb.tokens)
    # and the packed weights hold dim*4/32 words per row
    assert wq["layers.0.q"].packed.shape == (sh.q_heads * sh.head_dim, sh.hidden // 8)
