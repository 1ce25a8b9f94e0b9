"""The batch oracle: n independent copies of the pinned single-sequence oracle. Its own
logic is the split of ragged rows by count, the all-or-nothing trim, and independence
(a sequence's drafts do not depend on what the others append)."""
import numpy as np
import pytest

from block_drafting_dflash_amd import synth
from oracle import dflash_oracle as O
from oracle.batch_oracle import OracleBatch

MICRO = synth.Shape(hidden=32, layers=2, q_heads=4, kv_heads=2, head_dim=8, intermediate=48, vocab=97,
                    target_streams=2, target_width=16, window=7, weight_dtype="f32", act_dtype="f32",
                    rope_theta=10000.0)


@pytest.fixture(scope="module")
def w():
    return synth.make_weights(MICRO, threads=2)


def test_batch_equals_independent_sequences_with_ragged_rows(w):
    n = 3
    ob = OracleBatch(MICRO, w, n, 4)
    singles = [O.OracleDrafter(MICRO, w, 4) for _ in range(n)]
    rng = np.random.default_rng(1)
    counts = [9, 4, 13]
    rows = [synth.resid_rows(MICRO, c, 10 + s) for s, c in enumerate(counts)]
    ob.append(np.concatenate(rows), counts, commit=True)
    for od, r in zip(singles, rows):
        od.append(r, commit=True)
    for r in range(5):
        B = int(rng.integers(1, 5))
        anchors = [int(a) for a in rng.integers(0, MICRO.vocab, n)]
        got = ob.draft(anchors, B)
        for s in range(n):
            want = singles[s].draft(anchors[s], B)
            np.testing.assert_array_equal(got[s].tokens, want.tokens)
            np.testing.assert_array_equal(got[s].hidden, want.hidden)
        app = [B + 1 if s != 1 or r % 2 else 0 for s in range(n)]  # sequence 1 skips some appends
        rows = [synth.resid_rows(MICRO, c, 100 * r + s) for s, c in enumerate(app)]
        ob.append(np.concatenate([x for x in rows if len(x)]), app)
        m = [int(rng.integers(0, c + 1)) if c else 0 for c in app]
        m = [min(mm, c) for mm, c in zip(m, app)]
        ob.trim(m)
        for s in range(n):
            if app[s]:
                singles[s].append(rows[s])
            singles[s].trim(m[s])
            assert ob.state(s) == singles[s].state()


def test_trim_is_all_or_nothing(w):
    ob = OracleBatch(MICRO, w, 2, 4)
    ob.append(synth.resid_rows(MICRO, 10, 0), [5, 5], commit=True)
    ob.append(synth.resid_rows(MICRO, 5, 1), [3, 2])
    before = [ob.state(s) for s in range(2)]
    with pytest.raises(O.OracleError):
        ob.trim([1, 3])  # sequence 1 has only 2 pending rows
    assert [ob.state(s) for s in range(2)] == before
    ob.trim([1, 2])
    assert [ob.state(s)[:2] for s in range(2)] == [(7, 0), (5, 0)]


def test_a_sequence_ignores_the_others(w):
    """Sequence 0's draft is the same whatever sequence 1 holds."""
    outs = []
    for tag in (0, 1):
        ob = OracleBatch(MICRO, w, 2, 3)
        ob.append(np.concatenate([synth.resid_rows(MICRO, 8, 50), synth.resid_rows(MICRO, 6, 60 + tag)]), [8, 6],
                  commit=True)
        outs.append(ob.draft([5, 7], 3))
    np.testing.assert_array_equal(outs[0][0].hidden, outs[1][0].hidden)
    assert not np.array_equal(outs[0][1].hidden, outs[1][1].hidden)


def test_batch_refusals(w):
    ob = OracleBatch(MICRO, w, 2, 3)
    with pytest.raises(O.OracleError):
        ob.append(synth.resid_rows(MICRO, 3, 0), [2, 2])  # counts do not match the rows
    with pytest.raises(O.OracleError):
        ob.append(synth.resid_rows(MICRO, 0, 0), [0, 0])
    ob.append(synth.resid_rows(MICRO, 3, 0), [3, 0], commit=True)
    with pytest.raises(O.OracleError):
        ob.draft([1, 1], 2)  # sequence 1 has no context: nothing drafts
    assert ob.state(0)[:2] == (3, 0)
