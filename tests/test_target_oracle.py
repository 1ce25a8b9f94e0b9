"""Pins of the target oracle (the verify forward of a DFlash round's target) against what
the pages and the mathematics fix: a cacheless torch formulation with explicit masks, the
pages' identity property (speculative output token-identical to classic greedy decoding),
the post-trim cache against a target rebuilt from the committed tokens, the capture point
(before the final norm) and the slack rule."""
import numpy as np
import pytest

from block_drafting_dflash_amd import synth
from oracle import dflash_oracle as O
from oracle.target_oracle import OracleTarget
from tests.torch_target import TorchTarget

MICRO_T = synth.TargetShape(hidden=32, layers=4, q_heads=4, kv_heads=2, head_dim=8, intermediate=48, vocab=97,
                            window=5, full_layers=(2,), capture_layers=(0, 1, 3), weight_dtype="f32",
                            act_dtype="f32", rope_theta=10000.0, max_context=256)
MICRO_D = synth.Shape(hidden=32, layers=2, q_heads=4, kv_heads=2, head_dim=8, intermediate=48, vocab=97,
                      target_streams=3, target_width=32, window=6, weight_dtype="f32", act_dtype="f32",
                      rope_theta=10000.0)


def weights(t, d=MICRO_D):
    dw = synth.make_weights(d.with_(weight_dtype=t.weight_dtype, act_dtype=t.act_dtype), threads=2)
    return dw, synth.make_target_weights(t, dw, threads=2)


@pytest.fixture(scope="module")
def micro():
    return weights(MICRO_T)


@pytest.fixture(scope="module")
def micro_bf16():
    return weights(MICRO_T.with_(weight_dtype="bf16", act_dtype="bf16"))


def greedy(target_shape, tw, prompt, n):
    """Classic decode: one target forward per token, each committed."""
    ot = OracleTarget(target_shape, tw, 1)
    a = ot.prefill(prompt, 4).argmax[-1]
    out = [int(a)]
    for _ in range(n - 1):
        a = ot.forward([out[-1]]).argmax[0]
        ot.trim(0)
        out.append(int(a))
    return out


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_verify_forward_matches_torch_formulation(micro, micro_bf16, act):
    """Prefill, then verify forwards of random proposals with random trims; each forward's
    argmaxes, margins and captured streams equal the cacheless torch pass over the committed
    tokens plus the block."""
    t = MICRO_T if act == "f32" else MICRO_T.with_(weight_dtype="bf16", act_dtype="bf16")
    _, tw = micro if act == "f32" else micro_bf16
    ot = OracleTarget(t, tw, 4)
    tt = TorchTarget(t, tw)
    rng = np.random.default_rng(3)
    hist = [int(x) for x in synth.prompt_tokens(t.vocab, 9, tag=1)]
    ot.prefill(hist, 4)
    anchor = int(rng.integers(0, t.vocab))
    for r in range(7):
        B = int(rng.integers(1, 5))
        block = [anchor] + [int(x) for x in rng.integers(0, t.vocab, B)]
        res = ot.forward(block)
        ta, tm, tc = tt.forward(hist + block)
        np.testing.assert_array_equal(res.argmax, ta[-(B + 1):])
        np.testing.assert_allclose(res.margins, tm[-(B + 1):], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(res.capture, tc[-(B + 1):], rtol=1e-11, atol=1e-12)
        k = int(rng.integers(0, B + 1))
        ot.trim(B - k)
        hist += block[:k + 1]
        anchor = int(res.argmax[k])
        assert ot.state()[:2] == (len(hist), 0)


def test_capture_is_the_residual_stream_before_the_final_norm(micro):
    _, tw = micro
    t = MICRO_T.with_(capture_layers=(1, 3))  # 3 is the last layer: its stream is the final hidden
    ot = OracleTarget(t, tw, 4)
    res = ot.forward([5, 6, 7])
    np.testing.assert_array_equal(res.capture[:, -t.hidden:], res.hidden)
    z = O.rms_norm(res.hidden, np.asarray(tw["final_norm"], dtype=np.float64), t.rms_eps)
    assert not np.allclose(res.capture[:, -t.hidden:], z)
    assert res.capture.shape == (3, 2 * t.hidden)


@pytest.mark.parametrize("p_right", [0.0, 0.7, 1.0])
def test_speculative_decoding_is_token_identical_to_greedy_decoding(micro, p_right):
    """The pages' identity check on synthetic weights: the round loop (drafter oracle draft,
    target verify forward, greedy verify, captured streams appended to the drafter, both
    trimmed by B - k) commits exactly the tokens classic greedy decoding of the target emits.
    With p_right > 0 each proposal is replaced by the target's own greedy token with that
    probability, so rounds accept 0..B tokens."""
    dw, tw = micro
    B, n_tokens = 4, 40
    prompt = [int(x) for x in synth.prompt_tokens(MICRO_T.vocab, 11, tag=2)]
    want = greedy(MICRO_T, tw, prompt, n_tokens)
    ot = OracleTarget(MICRO_T, tw, B)
    od = O.OracleDrafter(MICRO_D, dw, B)
    pre = ot.prefill(prompt, 4)
    od.append(pre.capture, commit=True)
    out = [int(pre.argmax[-1])]
    rng = np.random.default_rng(int(10 * p_right))
    ks = []
    while len(out) < n_tokens:
        anchor = out[-1]
        d = od.draft(anchor, B).tokens
        pos = len(out)
        d = np.array([want[pos + i] if (pos + i < n_tokens and rng.random() < p_right) else d[i] for i in range(B)])
        res = ot.forward([anchor] + [int(x) for x in d])
        k, bonus = O.verify_greedy(d, res.argmax)
        od.append(res.capture)
        od.trim(B - k)
        ot.trim(B - k)
        out += [int(x) for x in d[:k]] + [bonus]
        ks.append(k)
    assert out[:n_tokens] == want
    if p_right == 1.0:
        assert min(ks[:-1]) == B
    if p_right == 0.7:
        assert 0 < np.mean(ks) < B
    assert ot.state()[0] == od.state()[0]  # both caches hold the same committed prefix


def test_post_trim_caches_equal_a_target_rebuilt_from_the_committed_tokens(micro):
    _, tw = micro
    ot = OracleTarget(MICRO_T, tw, 4)
    rng = np.random.default_rng(8)
    hist = [int(x) for x in synth.prompt_tokens(MICRO_T.vocab, 6, tag=3)]
    ot.prefill(hist, 4)
    for r in range(9):
        B = 4
        block = [int(x) for x in rng.integers(0, MICRO_T.vocab, B + 1)]
        ot.forward(block)
        k = int(rng.integers(0, B + 1))
        ot.trim(B - k)
        hist += block[:k + 1]
    fresh = OracleTarget(MICRO_T, tw, 4)
    fresh.prefill(hist, 3)
    assert ot.state() == fresh.state()
    for l in range(MICRO_T.layers):
        p1, k1, v1 = ot.window(l)
        p2, k2, v2 = fresh.window(l)
        assert np.array_equal(p1, p2)
        assert len(p1) == (len(hist) if MICRO_T.layer_kind(l) == "full" else min(len(hist), MICRO_T.window - 1))
        np.testing.assert_allclose(k1, k2, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(v1, v2, rtol=1e-12, atol=1e-14)


def test_sliding_window_past_the_context_equals_full_attention(micro):
    _, tw = micro
    toks = [int(x) for x in synth.prompt_tokens(MICRO_T.vocab, 14, tag=4)]
    a = OracleTarget(MICRO_T.with_(window=1000), tw, 4).prefill(toks, 5)
    b = OracleTarget(MICRO_T.with_(full_layers=(0, 1, 2, 3)), tw, 4).prefill(toks, 5)
    np.testing.assert_allclose(a.capture, b.capture, rtol=1e-13, atol=1e-15)
    c = OracleTarget(MICRO_T.with_(window=2), tw, 4).prefill(toks, 5)
    assert not np.allclose(a.capture, c.capture)


def test_target_trim_legality_and_the_slack_floor(micro):
    _, tw = micro
    ot = OracleTarget(MICRO_T, tw, 4)
    ot.forward([1, 2, 3])
    st = ot.state()
    for m in (-1, 4):
        with pytest.raises(O.OracleError):
            ot.trim(m)
        assert ot.state() == st
    with pytest.raises(O.OracleError):
        ot.forward([4])  # pending rows
    ot.trim(3)
    assert ot.state()[:2] == (0, 0)
    assert OracleTarget(MICRO_T, tw, 129).S == 129 and OracleTarget(MICRO_T, tw, 16).S == 128
    with pytest.raises(O.OracleError):
        ot.forward([MICRO_T.vocab])
