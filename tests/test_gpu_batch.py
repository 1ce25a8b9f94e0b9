"""GPU parity of independent sequences drafted together (dflash_batch_*, through the C-ABI):
in lock-step with n copies of the oracle (ragged contexts and accept lengths, every
sequence's tokens, hidden rows, verify result, offsets and live window), and bit for bit
against n single-sequence contexts fed the same calls (a sequence computes what it would
alone: the GEMMs reduce in an order that does not depend on the row count)."""
import numpy as np
import pytest
import torch

from block_drafting_dflash_amd import binding, synth
from oracle import dflash_oracle as O
from oracle.batch_oracle import OracleBatch
from tests import parity as P
from tests.test_gpu_parity import MICRO_BF16, MICRO_F32

pytestmark = pytest.mark.gpu


class BatchLockStep:
    def __init__(self, shape, w, n, max_block, phase=0, dev=None):
        self.sh, self.n = shape, n
        self.gpu = binding.Batch(shape, dev if dev is not None else binding.to_device(shape, w), n, max_block, phase)
        self.orc = OracleBatch(shape, w, n, max_block, phase)
        self.tol = 1e-4 if shape.act_dtype == "f32" else 2e-2
        self.margin = P.MARGIN_F32 if shape.act_dtype == "f32" else P.MARGIN
        self.bf16 = shape.act_dtype == "bf16"
        self.dt = binding.act_torch_dtype(shape)
        self.near_ties = 0

    def _t(self, a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.dt).to(self.gpu.device)

    def check_state(self):
        for s in range(self.n):
            e, pend = self.gpu.state(s)
            oe, ospan, _, _ = self.orc.state(s)
            assert (e, pend) == (oe, ospan), (s, (e, pend), (oe, ospan))

    def check_windows(self):
        torch.cuda.synchronize()
        for s in range(self.n):
            for l in range(self.sh.layers):
                k, v = self.gpu.cache_read(s, l)
                pos, ok, ov = self.orc.seqs[s].live_window(l)
                assert k.shape[1] == len(pos), (s, l)
                for g_, o_ in ((k, ok), (v, ov)):
                    gg = g_.float().cpu().numpy()
                    assert P.rel_rows(gg, o_).max(initial=0) <= self.tol
                    assert P.elem_excess(gg, o_, self.tol, self.bf16) <= 1.0

    def append(self, rows, commit=False):
        counts = [len(r) for r in rows]
        cat = np.concatenate([r for r in rows if len(r)])
        self.gpu.append(self._t(cat), counts, commit=commit)
        self.orc.append(cat, counts, commit=commit)
        self.check_state()

    def trim(self, m):
        self.gpu.trim(m)
        self.orc.trim(m)
        self.check_state()
        self.check_windows()

    def _agree(self, got, want, margins, what):
        for i in range(len(want)):
            if margins[i] <= self.margin:
                self.near_ties += 1
                continue
            assert got[i] == want[i], f"{what} row {i}: gpu {got[i]} oracle {want[i]} (margin {margins[i]:.4g})"

    def draft(self, anchors, B):
        hidden = torch.empty((self.n, B + 1, self.sh.hidden), dtype=torch.float32, device=self.gpu.device)
        toks = self.gpu.draft(anchors, B, hidden=hidden)
        res = self.orc.draft(anchors, B)
        torch.cuda.synchronize()
        tg, hg = toks.cpu().numpy(), hidden.cpu().numpy()
        for s in range(self.n):
            assert P.rel_rows(hg[s], res[s].hidden).max() <= self.tol
            assert P.elem_excess(hg[s], res[s].hidden, self.tol, False) <= 1.0
            self._agree(tg[s], res[s].tokens, res[s].margins, f"sequence {s} draft")
        return np.stack([r.tokens for r in res])

    def verify(self, d, a, B):
        out = self.gpu.verify_greedy(torch.tensor(d, dtype=torch.int32, device=self.gpu.device),
                                     torch.tensor(a, dtype=torch.int32, device=self.gpu.device), B)
        got = out.cpu().tolist()
        res = []
        for s in range(self.n):
            k, bonus = O.verify_greedy(d[s], a[s])
            assert got[s] == [k, bonus, 0], (s, got[s], k, bonus)
            res.append((k, bonus))
        return res


def run_batch_rounds(ls, contexts, B, rounds, tag):
    sh, n = ls.sh, ls.n
    ls.append([synth.resid_rows(sh, c, 10 * tag + s) for s, c in enumerate(contexts)], commit=True)
    ls.check_windows()
    rng = np.random.default_rng(tag)
    anchors = [int(a) for a in rng.integers(0, sh.vocab, n)]
    ks = []
    for r in range(rounds):
        d = ls.draft(anchors, B)
        kk = [int(rng.integers(0, B + 1)) for _ in range(n)]
        a = np.stack([P.target_with_accept_length(d[s], kk[s], sh.vocab, tail=anchors[s] + 7 * r) for s in range(n)])
        res = ls.verify(d, a, B)
        assert [k for k, _ in res] == kk
        ls.append([synth.resid_rows(sh, B + 1, 1000 * tag + 10 * r + s) for s in range(n)])
        ls.trim([B - k for k, _ in res])
        anchors = [b for _, b in res]
        ks.append(kk)
    return ks


@pytest.mark.parametrize("kind,n,B,phase", [("bf16", 3, 4, 0), ("bf16", 5, 4, 8), ("bf16", 8, 7, 0), ("f32", 2, 3, 16),
                                            ("bf16", 1, 16, 0), ("q4", 4, 4, 24)])
def test_batch_rounds_match_oracle(kind, n, B, phase):
    """Ragged prefills and accept lengths; 15, 25 and 64 rows per GEMM (one launch with the
    norm staged in LDS in one phase, one staged in two phases, two launches), f32, one
    sequence, 4-bit weights."""
    sh = {"bf16": MICRO_BF16, "f32": MICRO_F32, "q4": MICRO_BF16.with_(weight_dtype="q4")}[kind]
    w = synth.make_weights(sh)
    ls = BatchLockStep(sh, w, n, B, phase)
    contexts = [7 + 13 * s for s in range(n)]
    ks = run_batch_rounds(ls, contexts, B, 8, tag=n + B)
    print(kind, n, B, "near ties", ls.near_ties, "ks", ks)


def test_batch_at_its_limits():
    """64 sequences (the most a batch takes) at block 7: 512 rows per GEMM, the row limit,
    with ragged contexts from a few rows to far past the window and ragged accept lengths."""
    sh, n, B = MICRO_BF16, 64, 7
    ls = BatchLockStep(sh, synth.make_weights(sh), n, B, phase=8)
    contexts = [1 + 5 * s for s in range(n)]
    ks = run_batch_rounds(ls, contexts, B, 3, tag=64)
    print("64 sequences: near ties", ls.near_ties, "ks", ks)


@pytest.mark.parametrize("n", [3, 5, 8])
def test_batch_equals_single_contexts_bit_for_bit(n):
    """15, 25 and 40 rows per GEMM: the normed launches stage their raw rows in one phase,
    in two (19-32 rows), and as a two-phase launch of 32 rows plus one of 8; a sequence's
    tokens, hidden rows and ring windows are bit for bit those of a single context."""
    sh = MICRO_BF16
    w = synth.make_weights(sh)
    dev = binding.to_device(sh, w)
    B = 4
    batch = binding.Batch(sh, dev, n, B)
    singles = [binding.Drafter(sh, dev, B) for _ in range(n)]
    rows = [synth.resid_rows(sh, 9 + 11 * s, 70 + s) for s in range(n)]
    batch.append(torch.from_numpy(np.concatenate(rows)).to(torch.bfloat16).cuda(), [len(r) for r in rows], commit=True)
    for d, r in zip(singles, rows):
        d.cache_append(torch.from_numpy(r).to(torch.bfloat16).cuda(), commit=True)
    rng = np.random.default_rng(5)
    anchors = [3, 500, 2000, 7, 911, 1234, 42, 2999][:n]
    for r in range(6):
        hb = torch.empty((n, B + 1, sh.hidden), dtype=torch.float32, device="cuda")
        tb = batch.draft(anchors, B, hidden=hb)
        for s in range(n):
            hs = torch.empty((B + 1, sh.hidden), dtype=torch.float32, device="cuda")
            ts = singles[s].draft_block(anchors[s], B, hidden=hs)
            assert torch.equal(tb[s], ts), (r, s)
            assert torch.equal(hb[s], hs), (r, s, (hb[s] - hs).abs().max().item())
        app = [synth.resid_rows(sh, B + 1, 900 + 10 * r + s) for s in range(n)]
        batch.append(torch.from_numpy(np.concatenate(app)).to(torch.bfloat16).cuda(), [B + 1] * n)
        m = [int(x) for x in rng.integers(0, B + 1, n)]
        batch.trim(m)
        for s in range(n):
            singles[s].cache_append(torch.from_numpy(app[s]).to(torch.bfloat16).cuda())
            singles[s].cache_trim(m[s])
            assert batch.state(s) == singles[s].cache_state()[:2]
        anchors = [int(x) for x in rng.integers(0, sh.vocab, n)]
    for s in range(n):
        for l in range(sh.layers):
            kb, vb = batch.cache_read(s, l)
            ks_, vs_ = singles[s].cache_read(l)
            assert torch.equal(kb, ks_) and torch.equal(vb, vs_), (s, l)


def test_batch_boundary_errors_leave_state_unchanged():
    sh = MICRO_F32
    w = synth.make_weights(sh)
    b = binding.Batch(sh, binding.to_device(sh, w), 2, 4)
    L = binding.lib()
    st = torch.cuda.current_stream().cuda_stream
    toks = torch.empty((2, 4), dtype=torch.int32, device="cuda")
    anchors = binding._i32_array([1, 2])
    assert L.dflash_batch_draft(b.b, anchors, 4, toks.data_ptr(), None, st) == 4  # no context yet
    rows = torch.from_numpy(synth.resid_rows(sh, 6, 0)).cuda()
    assert L.dflash_batch_append(b.b, rows.data_ptr(), binding._i32_array([-1, 7]), 1, st) == 1
    assert L.dflash_batch_append(b.b, rows.data_ptr(), binding._i32_array([0, 0]), 1, st) == 1
    b.append(rows, [6, 0], commit=True)
    assert L.dflash_batch_draft(b.b, anchors, 4, toks.data_ptr(), None, st) == 4  # sequence 1 still empty
    b.append(rows, [2, 4])
    assert b.state(0) == (6, 2) and b.state(1) == (0, 4)
    assert L.dflash_batch_draft(b.b, anchors, 4, toks.data_ptr(), None, st) == 6  # pending rows
    assert L.dflash_batch_trim(b.b, binding._i32_array([1, 5])) == 5  # sequence 1 has 4 pending
    assert b.state(0) == (6, 2) and b.state(1) == (0, 4)
    b.trim([1, 0])
    assert b.state(0) == (7, 0) and b.state(1) == (4, 0)
    assert L.dflash_batch_draft(b.b, binding._i32_array([1, sh.vocab]), 4, toks.data_ptr(), None, st) == 3
    assert L.dflash_batch_state(b.b, 2, None, None) == 3
