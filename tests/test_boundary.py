"""Host-side tests of the C-ABI library: no GPU needed (no device call is made).

They check that libdflash.so loads and exports every function include/dflash.h declares,
that the binding describes each of them, and the host-side validation of
dflash_query_sizes / dflash_create, including the ring size implied by the slack rule.
"""
import ctypes
import json
import os
import re

import pytest

from block_drafting_dflash_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12, names
    L = binding.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding.EXPORTS)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(binding, "LIB_PATH", "/nonexistent/libdflash.so")
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(ImportError):
        binding.lib()


def sizes(shape, max_block=4, phase=0):
    return binding.query_sizes(binding.make_config(shape, max_block, phase))


def status_of(shape, max_block=4, **cfg_over):
    cfg = binding.make_config(shape, max_block)
    for k, v in cfg_over.items():
        setattr(cfg, k, v)
    try:
        binding.query_sizes(cfg)
        return 0
    except binding.DFlashError as e:
        return e.status


def test_ring_size_follows_the_slack_rule():
    """ring bytes = layers * 2 (K,V) * kv_heads * Cs * head_dim * element size, where the
    stored slots Cs are the capacity W + S (S from the slack table the page states), raised
    to W + block + 1 and 64 at least, rounded up to a multiple of 8."""
    table = json.load(open(os.path.join(ROOT, "tests", "golden", "slack_table.json")))["table"]
    for sh in (synth.TINY_F32, synth.MUSE_BF16, synth.TINY_F32.with_(window=9)):
        elt = 4 if sh.act_dtype == "f32" else 2
        for b, S in table.items():
            if int(b) > 256:
                continue
            cs = max(sh.window + S, sh.window + int(b) + 1, 64)
            cs = (cs + 7) // 8 * 8
            ring, ws, packed = sizes(sh, int(b))
            assert ring == sh.layers * 2 * sh.kv_heads * cs * sh.head_dim * elt, (sh, b)
            assert cs >= sh.window + S  # the capacity the slack rule asks for is there


def test_packed_size_covers_every_linear_once():
    sh = synth.MUSE_BF16
    _, _, packed = sizes(sh)
    H, qd, kvd = sh.hidden, sh.q_heads * sh.head_dim, sh.kv_heads * sh.head_dim
    n = H * sh.fc_in + sh.vocab * H + sh.layers * (qd * H + 2 * kvd * H + H * qd + 3 * sh.intermediate * H)
    assert n * 2 <= packed <= n * 2 + 256 * (2 + 7 * sh.layers)


def test_packed_size_of_4bit_linears():
    """q4: codes (K/2 bytes per row) plus one (scale, bias) pair per 64-k group (4 bytes),
    for every linear once; the ring stays bf16."""
    sh = synth.MUSE_Q4
    ring, _, packed = sizes(sh)
    H, qd, kvd = sh.hidden, sh.q_heads * sh.head_dim, sh.kv_heads * sh.head_dim
    n = H * sh.fc_in + sh.vocab * H + sh.layers * (qd * H + 2 * kvd * H + H * qd + 3 * sh.intermediate * H)
    assert n * 9 // 16 <= packed <= n * 9 // 16 + 256 * (2 + 7 * sh.layers)
    assert ring == sizes(synth.MUSE_BF16)[0]


def test_query_sizes_validation_statuses():
    sh = synth.TINY_F32
    E_ARG, E_SHAPE, E_RANGE = 1, 2, 3
    assert status_of(sh) == 0
    assert status_of(sh, head_dim=60) == E_SHAPE
    assert status_of(sh, q_heads=3) == E_SHAPE  # not a multiple of kv_heads
    assert status_of(sh, hidden=0) == E_SHAPE
    assert status_of(sh, window=-1) == E_SHAPE
    assert status_of(sh, mask_token_id=sh.vocab) == E_RANGE
    assert status_of(sh, mask_token_id=-1) == E_RANGE
    assert status_of(sh, max_block=257) == E_RANGE
    assert status_of(sh, vocab=4100) == E_SHAPE  # not a multiple of 16
    assert status_of(sh, act_dtype=binding.DFLASH_BF16) == E_ARG  # f32 weights need f32 activations
    assert status_of(sh, weight_dtype=7) == E_ARG
    assert status_of(sh, rms_eps=0.0) == E_ARG
    assert status_of(sh, intermediate=200) == E_SHAPE  # no launch plan for this contraction
    # a dimension product past the int32 range is refused, not wrapped
    assert status_of(synth.MUSE_BF16, vocab=2 ** 20 + 16) == E_SHAPE


def test_create_refuses_null_buffers_before_any_device_call():
    sh = synth.TINY_F32
    cfg = binding.make_config(sh, 4)
    L = binding.lib()
    h = ctypes.c_void_p()
    st = L.dflash_create(ctypes.byref(cfg), None, None, 0, None, 0, None, 0, None, ctypes.byref(h))
    assert st == 1 and not h.value
    assert b"NULL" in L.dflash_last_error(None)
    w = binding.dflash_weights()
    st = L.dflash_create(ctypes.byref(cfg), ctypes.byref(w), None, 0, None, 0, None, 0, None, ctypes.byref(h))
    assert st == 1


def test_status_strings():
    L = binding.lib()
    for s in range(8):
        assert L.dflash_status_string(s)
    assert L.dflash_status_string(99) == b"unknown status"


def test_dspark_config_validation_and_sizes():
    """DSpark contexts (lablup/mlxcel #1751, Security fixes): the verify width max_block + 1 is
    clamped at 32, the Markov rank is one the chain kernel tiles, a DFlash context takes no
    Markov rank; the workspace holds the block's backbone logits, and adjacent-pair RoPE adds
    one deinterleaved copy of each layer's q_norm and k_norm to the packed weights."""
    E_ARG, E_SHAPE, E_RANGE = 1, 2, 3
    ds = synth.TINY_DSPARK_F32
    assert status_of(ds, max_block=31) == 0
    assert status_of(ds, max_block=32) == E_RANGE
    assert status_of(ds, max_block=31, markov_rank=100) == E_SHAPE
    assert status_of(ds, max_block=31, markov_rank=512) == E_SHAPE  # f32 factors: at most 256
    assert status_of(synth.MUSE_DSPARK_BF16, max_block=9, markov_rank=512) == 0
    assert status_of(ds, max_block=31, markov_rank=0) == E_SHAPE
    assert status_of(synth.TINY_F32, markov_rank=64) == E_ARG
    assert status_of(synth.TINY_F32, variant=2) == E_ARG
    assert status_of(synth.TINY_F32, rope_traditional=2) == E_ARG
    r0, w0, p0 = sizes(synth.TINY_F32, 9)
    r1, w1, p1 = sizes(ds.with_(window=synth.TINY_F32.window), 9)
    assert r1 == r0
    assert w0 + 4 * 9 * ds.vocab <= w1 <= w0 + 4 * 9 * ds.vocab + 2 * 8 * 4096 + 2 * 256  # logits, two steps of keys
    assert p1 == p0 + ds.layers * 2 * 256  # head_dim 64 f32 gains: one 256-byte block each
    _, _, p2 = sizes(synth.TINY_F32.with_(rope_style="traditional"), 9)
    assert p2 == p1


def test_batch_sizes_and_validation():
    """A batch of n sequences: n rings of the single-sequence size back to back, the same
    packed weights, a workspace for n blocks; n in 1..64, n * (max_block + 1) <= 512, DFlash
    form only."""
    L = binding.lib()
    sh = synth.MUSE_BF16
    r1, w1, p1 = sizes(sh, 4)

    def bsizes(shape, n, max_block=4, **over):
        cfg = binding.make_config(shape, max_block)
        for k, v in over.items():
            setattr(cfg, k, v)
        rb, wb, pb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        st = L.dflash_batch_query_sizes(ctypes.byref(cfg), n, ctypes.byref(rb), ctypes.byref(wb), ctypes.byref(pb))
        return st, rb.value, wb.value, pb.value

    st, rb, wb, pb = bsizes(sh, 4)
    assert st == 0 and rb == 4 * r1 and pb == p1 and wb > w1
    assert bsizes(sh, 1)[1:] == (r1, bsizes(sh, 1)[2], p1)
    assert bsizes(sh, 0)[0] == 3 and bsizes(sh, 65)[0] == 3
    assert bsizes(sh, 64, max_block=7)[0] == 0  # 512 rows
    assert bsizes(sh, 64, max_block=8)[0] == 3  # 576 rows
    assert bsizes(synth.MUSE_DSPARK_BF16, 2, max_block=7)[0] == 1
    h = ctypes.c_void_p()
    cfg = binding.make_config(sh, 4)
    assert L.dflash_batch_create(ctypes.byref(cfg), 2, None, None, 0, None, 0, None, 0, None, ctypes.byref(h)) == 1
    assert not h.value
