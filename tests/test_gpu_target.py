"""GPU parity of the target's verify forward (dflash_target_*, through the C-ABI) against the
target oracle, and the pages' identity property on the GPU: the speculative round loop
(drafter and target in the library) commits exactly the tokens that classic greedy decoding
of the same target emits, one forward per token."""
import numpy as np
import pytest
import torch

from block_drafting_dflash_amd import binding, synth
from oracle import dflash_oracle as O
from oracle.target_oracle import OracleTarget
from tests import parity as P

pytestmark = pytest.mark.gpu

T_BF16 = synth.TargetShape(hidden=512, layers=4, q_heads=8, kv_heads=2, head_dim=64, intermediate=768, vocab=3008,
                           window=20, full_layers=(2,), capture_layers=(0, 1, 3), weight_dtype="bf16",
                           act_dtype="bf16", max_context=512)
T_F32 = synth.TargetShape(hidden=256, layers=3, q_heads=4, kv_heads=2, head_dim=64, intermediate=384, vocab=1040,
                          window=9, full_layers=(1,), capture_layers=(0, 2), weight_dtype="f32", act_dtype="f32",
                          max_context=256)
D_BF16 = synth.Shape(hidden=512, layers=2, q_heads=8, kv_heads=2, head_dim=64, intermediate=768, vocab=3008,
                     target_streams=3, target_width=512, window=20, weight_dtype="bf16", act_dtype="bf16")


class TargetLockStep:
    """The library's target and the oracle target on the same rows, compared after every call."""

    def __init__(self, tshape, tw, max_block, dev=None):
        self.sh = tshape
        self.dev = dev if dev is not None else binding.to_device(tshape, tw)
        self.gpu = binding.Target(tshape, self.dev, max_block)
        self.orc = OracleTarget(tshape, tw, max_block)
        self.tol = 1e-4 if tshape.act_dtype == "f32" else 2e-2
        self.margin = P.MARGIN_F32 if tshape.act_dtype == "f32" else P.MARGIN
        self.bf16 = tshape.act_dtype == "bf16"
        self.near_ties = 0

    def forward(self, tokens) -> np.ndarray:
        n = len(tokens)
        toks = torch.tensor(tokens[1:] if n > 1 else [0], dtype=torch.int32, device="cuda")
        cap = torch.empty((n, len(self.sh.capture_layers) * self.sh.hidden), dtype=self.gpu.act_dtype, device="cuda")
        a, _ = self.gpu.forward(tokens[0], toks, n, capture=cap)
        res = self.orc.forward(tokens)
        torch.cuda.synchronize()
        got = a.cpu().numpy()
        for i in range(n):
            if res.margins[i] <= self.margin:
                self.near_ties += 1
                continue
            assert got[i] == res.argmax[i], (i, got[i], res.argmax[i], res.margins[i])
        cg = cap.float().cpu().numpy()
        assert P.rel_rows(cg, res.capture).max() <= self.tol
        assert P.elem_excess(cg, res.capture, self.tol, self.bf16) <= 1.0
        assert self.gpu.state()[:2] == self.orc.state()[:2]
        self.orc_last_capture = res.capture
        return res.argmax, cap

    def trim(self, m):
        self.gpu.trim(m)
        self.orc.trim(m)
        assert self.gpu.state() == self.orc.state()

    def check_caches(self):
        torch.cuda.synchronize()
        for l in range(self.sh.layers):
            k, v = self.gpu.cache_read(l)
            pos, ok, ov = self.orc.window(l)
            assert k.shape[1] == len(pos), (l, k.shape, len(pos))
            for g_, o_ in ((k, ok), (v, ov)):
                gg = g_.float().cpu().numpy()
                assert P.rel_rows(gg, o_).max(initial=0) <= self.tol
                assert P.elem_excess(gg, o_, self.tol, self.bf16) <= 1.0


@pytest.fixture(scope="module")
def bf16_pair():
    dw = synth.make_weights(D_BF16)
    return dw, synth.make_target_weights(T_BF16, dw)


@pytest.fixture(scope="module")
def f32_target():
    d = synth.Shape(hidden=256, layers=1, q_heads=4, kv_heads=2, head_dim=64, intermediate=384, vocab=1040,
                    target_streams=2, target_width=256, window=9, weight_dtype="f32", act_dtype="f32")
    return synth.make_target_weights(T_F32, synth.make_weights(d))


@pytest.mark.parametrize("kind,prompt_len,block", [("bf16", 45, 4), ("bf16", 70, 16), ("f32", 37, 3)])
def test_target_prefill_and_verify_rounds_match_oracle(bf16_pair, f32_target, kind, prompt_len, block):
    """A prompt in forwards of up to 32 rows (each committed), then verify forwards of random
    proposals with trims of random depth; argmaxes (exact above the near-tie margin),
    captured residual streams (per row and per element), offsets after every call, and every
    layer's cache window (sliding and full) after every trim."""
    tshape, tw = (T_BF16, bf16_pair[1]) if kind == "bf16" else (T_F32, f32_target)
    ls = TargetLockStep(tshape, tw, max_block=block)
    prompt = [int(x) for x in synth.prompt_tokens(tshape.vocab, prompt_len, tag=5)]
    for s in range(0, prompt_len, ls.gpu.rows_max):
        ls.forward(prompt[s:s + ls.gpu.rows_max])
        ls.trim(0)
    ls.check_caches()
    rng = np.random.default_rng(block)
    anchor = int(prompt[-1])
    for r in range(10):
        block_toks = [anchor] + [int(x) for x in rng.integers(0, tshape.vocab, block)]
        a, _ = ls.forward(block_toks)
        k = int(rng.integers(0, block + 1))
        ls.trim(block - k)
        ls.check_caches()
        anchor = int(a[k])
    print(kind, "near ties", ls.near_ties)


def test_target_widest_verify_forward(bf16_pair):
    """Block 64, the widest verify a target takes (65-row forwards, slack 128): the prompt in
    65-row forwards, then rounds of 65 rows with trims of random depth, argmaxes, captures,
    offsets and every cache window (sliding and full) against the oracle after every trim."""
    tshape, tw, block = T_BF16.with_(max_context=1024), bf16_pair[1], 64
    ls = TargetLockStep(tshape, tw, max_block=block)
    assert ls.gpu.rows_max == block + 1
    prompt = [int(x) for x in synth.prompt_tokens(tshape.vocab, 100, tag=64)]
    for s in range(0, len(prompt), ls.gpu.rows_max):
        ls.forward(prompt[s:s + ls.gpu.rows_max])
        ls.trim(0)
    ls.check_caches()
    rng = np.random.default_rng(64)
    anchor = int(prompt[-1])
    for k in (0, block, 23, 5):
        block_toks = [anchor] + [int(x) for x in rng.integers(0, tshape.vocab, block)]
        a, _ = ls.forward(block_toks)
        ls.trim(block - k)
        ls.check_caches()
        anchor = int(a[k])
    print("block 64 near ties", ls.near_ties)


def test_target_boundary_errors(bf16_pair):
    t = binding.Target(T_BF16, binding.to_device(T_BF16, bf16_pair[1]), max_block=4)
    toks = torch.zeros(40, dtype=torch.int32, device="cuda")
    out = torch.empty(40, dtype=torch.int32, device="cuda")
    L = binding.lib()
    stream = torch.cuda.current_stream().cuda_stream
    assert L.dflash_target_forward(t.t, 0, toks.data_ptr(), 33, out.data_ptr(), None, stream) == 3  # > 32 rows
    assert L.dflash_target_forward(t.t, T_BF16.vocab, toks.data_ptr(), 2, out.data_ptr(), None, stream) == 3
    assert L.dflash_target_forward(t.t, 0, None, 2, out.data_ptr(), None, stream) == 1
    assert L.dflash_target_forward(t.t, 0, toks.data_ptr(), 2, None, None, stream) == 1
    assert t.state() == (0, 0, 32)
    t.forward(1, toks, 3, out)
    assert L.dflash_target_forward(t.t, 0, toks.data_ptr(), 2, out.data_ptr(), None, stream) == 6  # pending
    assert L.dflash_target_trim(t.t, 4) == 5
    t.trim(1)
    assert t.state() == (2, 0, 32)


def run_classic(tshape, dev, prompt, n_tokens):
    """Classic greedy decode: one target forward per token (each committed)."""
    t = binding.Target(tshape, dev, max_block=1)
    for s in range(0, len(prompt), t.rows_max):
        chunk = prompt[s:s + t.rows_max]
        a, _ = t.forward(chunk[0], torch.tensor(chunk[1:] or [0], dtype=torch.int32, device="cuda"), len(chunk))
        t.trim(0)
    out = [int(a[-1].item())]
    while len(out) < n_tokens:
        a, _ = t.forward(out[-1], None, 1)
        t.trim(0)
        out.append(int(a[0].item()))
    return out


def run_speculative(tshape, dsh, tdev, ddev, prompt, n_tokens, B, proposals=None):
    """The round loop on the GPU: drafter draft, target verify forward over [anchor, drafts],
    greedy verify, the captured streams appended to the drafter, both trimmed by B - k.
    With `proposals` (host function of the position) some drafts are replaced before the
    verify forward."""
    t = binding.Target(tshape, tdev, max_block=B)
    d = binding.Drafter(dsh, ddev, max_block=B)
    ncap = len(tshape.capture_layers) * tshape.hidden
    for s in range(0, len(prompt), t.rows_max):
        chunk = prompt[s:s + t.rows_max]
        cap = torch.empty((len(chunk), ncap), dtype=t.act_dtype, device="cuda")
        a, _ = t.forward(chunk[0], torch.tensor(chunk[1:] or [0], dtype=torch.int32, device="cuda"), len(chunk),
                         capture=cap)
        t.trim(0)
        d.cache_append(cap, commit=True)
    out = [int(a[-1].item())]
    ks = []
    toks = torch.empty(B, dtype=torch.int32, device="cuda")
    cap = torch.empty((B + 1, ncap), dtype=t.act_dtype, device="cuda")
    while len(out) < n_tokens:
        anchor = out[-1]
        d.draft_block(anchor, B, tokens=toks)
        if proposals is not None:
            toks.copy_(torch.tensor(proposals(len(out), toks.cpu().tolist()), dtype=torch.int32, device="cuda"))
        a, _ = t.forward(anchor, toks, B + 1, capture=cap)
        res = d.verify_greedy(toks, a, B).cpu().tolist()
        k, bonus, status = res
        assert status == 0
        d.cache_append(cap)
        d.cache_trim(B - k)
        t.trim(B - k)
        out += toks[:k].cpu().tolist() + [bonus]
        ks.append(k)
    assert d.cache_state()[0] == t.state()[0]
    return out[:n_tokens], ks


@pytest.mark.parametrize("p_right", [0.0, 0.75])
def test_speculative_loop_commits_the_tokens_of_classic_decoding(bf16_pair, p_right):
    """The pages' identity check, on the GPU: whatever the drafter proposes, the committed
    stream equals classic greedy decoding of the target bit for bit (the forward of a row does
    not depend on how many rows share the call). p_right > 0 replaces each proposal by the
    classic token with that probability, so rounds accept 0..B tokens."""
    dw, tw = bf16_pair
    tdev = binding.to_device(T_BF16, tw)
    ddev = binding.to_device(D_BF16, dw)
    prompt = [int(x) for x in synth.prompt_tokens(T_BF16.vocab, 40, tag=6)]
    n_tokens, B = 48, 4
    want = run_classic(T_BF16, tdev, prompt, n_tokens + B + 1)
    rng = np.random.default_rng(int(100 * p_right))

    def proposals(pos, drafted):
        return [want[pos + i] if rng.random() < p_right else drafted[i] for i in range(B)]

    got, ks = run_speculative(T_BF16, D_BF16, tdev, ddev, prompt, n_tokens, B, proposals if p_right else None)
    assert got == want[:n_tokens]
    if p_right:
        assert 0 < np.mean(ks) < B
    print("identity", p_right, "accepted", ks)


def test_classic_decode_matches_the_oracle(bf16_pair):
    """The GPU target's greedy decode against the oracle's, token by token (near ties, where
    either token is correct, continue with the oracle's)."""
    _, tw = bf16_pair
    ls = TargetLockStep(T_BF16, tw, max_block=1)
    prompt = [int(x) for x in synth.prompt_tokens(T_BF16.vocab, 33, tag=7)]
    a, _ = ls.forward(prompt[:32])
    ls.trim(0)
    a, _ = ls.forward(prompt[32:])
    ls.trim(0)
    tok = int(a[-1])
    for _ in range(24):
        a, _ = ls.forward([tok])
        ls.trim(0)
        tok = int(a[0])
    ls.check_caches()
