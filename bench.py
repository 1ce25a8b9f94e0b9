"""Throughput of one DFlash speculative round at batch 1 on one MI355X.

A step is one whole round over one block of synthetic input: the drafter's block forward
(dflash_draft_block), the target's verify-row argmaxes (through the shared lm_head with
dflash_lm_head_argmax, or a stand-in target), greedy verify (dflash_verify_greedy, whose
kernel writes (k, bonus, status) into pinned host memory), the append of the B+1 verify
residual rows (dflash_cache_append), the host's wait for that result (polled in pinned
memory, so the append still runs while the host trims and enqueues the next round) and the
trim (dflash_cache_trim). Inputs are resident in HBM before the timed region starts. The
timed rounds record no timing events (a HIP event record holds the stream for a few
microseconds); the host stamps the arrival of each round's verify result, whose spacing gives
the per-round time distribution, and a pass of up to 100 more rounds after them records
events around the draft, the append and the lm_head argmax kernel for the per-call
breakdown and `roofline`.

Workload (timed as `value`): muse-bf16-b4-ctx1024 -- Muse-assistant-shaped bf16 drafter
(hidden 2048, 5 layers, 32/4 heads x 128, intermediate 6144, vocab 202048, untied lm_head,
fc 20480 -> 2048), context 1024, window 2048, block 4, verify rows N(0,1) through the
lm_head. Also reported, each with the round counters the pages print (draft_rounds, draft_n,
draft_n_accepted, mean accepted with and without the bonus, committed tok/s, accept
histogram, SHA-256 of the committed token stream): the block-16 round (muse-bf16-b16-ctx4096,
p = 0.6 stand-in target), the 16384-row context with ring wraps at blocks 8 and 32 (prefill
timed on its own), the adaptive verify width (the library's controller between blocks 4 and 16
against both fixed widths), speculative decoding through a synthetic Muse-shaped target
against classic greedy decoding of it, the 4-bit width sweep (muse-q4-sweep-ctx2048, blocks 4/5/8/16), the tiny
f32 round (tiny-f32-b4-ctx64), an HBM streaming-read probe, and the CPU oracle on the host
cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BREAKDOWN_ROUNDS = 100  # event-timed rounds after the timed ones (per-call breakdown, kernel timing)


def await_verify(hv, timeout_s: float = 10.0):
    """Spin until the verify kernel has written (k, bonus, status) into the pinned words hv
    (each preset to -1). Each word changes once, from -1 to its value; k and status are
    never -1 once written, bonus only with status 1. The append enqueued after the verify may
    still run: the next round's launches queue behind it on the stream."""
    t0 = time.perf_counter()
    while True:
        k, bonus, status = int(hv[0]), int(hv[1]), int(hv[2])
        if k != -1 and status != -1 and (bonus != -1 or status == 1):
            return k, bonus, status
        if time.perf_counter() - t0 > timeout_s:
            raise RuntimeError("the verify result did not arrive in pinned host memory")


def alg_bytes(sh, block: int, ctx_visible: int) -> dict:
    """Algorithmic bytes of one round: every weight read once, live K/V window, inputs.

    Weights cost 4 bytes per parameter in f32, 2 in bf16 and 9/16 in q4 (a 4-bit code plus
    a bf16 scale and bias per 64 inputs); activations, the ring and the embedding rows take
    the activation dtype."""
    e = 4 if sh.act_dtype == "f32" else 2
    we = {"f32": 4, "bf16": 2, "q4": 9 / 16}[sh.weight_dtype]
    H, I, V, F = sh.hidden, sh.intermediate, sh.vocab, sh.fc_in
    qd, kvd = sh.q_heads * sh.head_dim, sh.kv_heads * sh.head_dim
    layer = (qd * H + 2 * kvd * H + H * qd + 2 * I * H + H * I) * we
    fc = H * F * we
    lm = V * H * we
    kv = sh.layers * 2 * min(ctx_visible, sh.window) * kvd * e
    dspark = getattr(sh, "variant", "dflash") == "dspark"
    rows = block if dspark else block + 1  # DSpark: gamma block rows
    inputs = (block + 1) * F * e + rows * H * e
    fwd = fc + sh.layers * layer + lm + kv + inputs
    out = {"fc": fc, "layers": sh.layers * layer, "lm_head": lm, "kv": kv}
    if dspark:
        # every row's f32 logits written once and read once by its chain step, and per step
        # the whole markov_w2 plus one markov_w1 row (the factors take the activation dtype)
        step = V * sh.markov_rank * e + V * 4 + sh.markov_rank * e
        out.update(markov_step=step, chain=block * step, logits=2 * block * V * 4)
        fwd += block * step + block * V * 4
    out.update(block_forward=fwd, round_lm_verify=fwd + lm + (block + 1) * H * e)
    return out


def counted_traffic():
    """HBM bytes per lm_head launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    (scaled by the same counters on a 1 GiB copy), or None if the kernel source changed since."""
    try:
        d = json.load(open(os.path.join(ROOT, "profiles", "lm_head_argmax_counters.json")))
        src = open(os.path.join(ROOT, "block_drafting_dflash_amd", "csrc", "gemm_impl.h"), "rb").read()
    except OSError:
        return None
    return d["traffic_bytes"] if d.get("kernel_source_sha256") == hashlib.sha256(src).hexdigest() else None


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


class Leg:
    """Rounds of one drafter context: block B, a verify source, timed without events, then a
    breakdown pass with events; round counters and the committed token stream."""

    def __init__(self, sh, dw, B: int, context: int, phase: int = 0):
        import torch

        from block_drafting_dflash_amd import binding, synth

        self.torch, self.synth, self.binding = torch, synth, binding
        self.sh, self.B = sh, B
        self.dev = torch.device("cuda", 0)
        self.stream = torch.cuda.current_stream()
        self.act = binding.act_torch_dtype(sh)
        self.g = binding.Drafter(sh, dw, max_block=B, phase=phase)
        slab = torch.from_numpy(synth.resid_rows(sh, context, 0)).to(self.act).to(self.dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        self.g.cache_append(slab, commit=True, stream=self.stream)
        e1.record(self.stream)
        torch.cuda.synchronize()
        self.prefill_ms = e0.elapsed_time(e1)
        del slab

    def run(self, warmup: int, steps: int, verify, resid_tag: int, anchor_tag: int, lm_timing: bool = False,
            chain_timing: bool = False) -> dict:
        """verify(r, toks_r, out_r): enqueue the target's argmaxes of round r into out_r;
        verify.prepare(tgt), if present, fills what does not depend on the draft beforehand."""
        torch, synth = self.torch, self.synth
        g, sh, B, dev, stream = self.g, self.sh, self.B, self.dev, self.stream
        nb = min(steps, BREAKDOWN_ROUNDS)
        n = warmup + steps + nb
        resid = torch.from_numpy(np.stack([synth.resid_rows(sh, B + 1, resid_tag + r) for r in range(n)]))
        resid = resid.to(self.act).to(dev)
        toks = torch.empty((n, B), dtype=torch.int32, device=dev)  # each round's drafted tokens stay
        tgt = torch.empty((n, B + 1), dtype=torch.int32, device=dev)
        host = torch.empty(3, dtype=torch.int32, pin_memory=True)  # the verify kernel writes here
        hv = host.numpy()
        if hasattr(verify, "prepare"):
            verify.prepare(tgt)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nb)]
        evk = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nb)] if lm_timing else None
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nb)] if chain_timing else None
        for pair in (evk or []) + (evc or []):
            for x in pair:
                x.record(stream)  # creates the underlying events before the timed region
        anchor = synth.anchor_token(sh, tag=anchor_tag)
        ks, bonuses, stamps = [], [], []
        torch.cuda.synchronize()
        t0 = el = None
        b0 = warmup + steps
        for r in range(n):
            if r == warmup:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                stamps.append(t0)
            if r == b0:
                torch.cuda.synchronize()
                el = time.perf_counter() - t0
            e = ev[r - b0] if r >= b0 else None
            if e: e[0].record(stream)
            if e and evc: g.time_next_chain(*evc[r - b0])
            g.draft_block(anchor, B, tokens=toks[r], stream=stream)
            if e: e[1].record(stream)
            if e and evk: g.time_next_argmax(*evk[r - b0])
            verify(r, toks[r], tgt[r])
            if e: e[2].record(stream)
            hv[:] = -1
            g.verify_greedy(toks[r], tgt[r], B, out=host, stream=stream)
            if e: e[3].record(stream)
            g.cache_append(resid[r], stream=stream)
            if e: e[4].record(stream)
            k, bonus, status = await_verify(hv)  # the round's one host round trip
            if warmup <= r < b0:
                stamps.append(time.perf_counter())
            assert status == 0
            g.cache_trim(B - k)
            anchor = bonus
            ks.append(k)
            bonuses.append(bonus)
        torch.cuda.synchronize()
        from block_drafting_dflash_amd.counters import RoundCounters

        d = toks.cpu().numpy()
        stream_toks = []
        cnt = RoundCounters()
        for r in range(n):
            stream_toks.extend(int(x) for x in d[r, :ks[r]])
            stream_toks.append(bonuses[r])
            if warmup <= r < b0:
                cnt.record(B, ks[r])
        rs = steps / el
        gaps_ms = np.diff(np.asarray(stamps)) * 1e3
        by = alg_bytes(sh, B, g.cache_state()[0])
        fwd = [x[0].elapsed_time(x[1]) + x[3].elapsed_time(x[4]) for x in ev]
        out = {
            "block": B, "rounds_per_s": round(rs, 2), "drafted_tok_s": round(rs * B, 1),
            "committed_tok_s": round(cnt.emitted / el, 1),
            "round_ms": {"mean": round(1e3 * el / steps, 4), "median": round(pct(gaps_ms, 50), 4),
                         "p90": round(pct(gaps_ms, 90), 4)},
            "rounds_per_s_median": round(1e3 / pct(gaps_ms, 50), 2),
            "block_forward_ms": round(float(np.mean(fwd)), 4),
            "block_forward_hbm_frac": round(by["block_forward"] / (float(np.mean(fwd)) * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "draft_ms": round(float(np.mean([x[0].elapsed_time(x[1]) for x in ev])), 4),
            "append_ms": round(float(np.mean([x[3].elapsed_time(x[4]) for x in ev])), 4),
            **cnt.as_dict(),
            "committed_token_sha256": hashlib.sha256(np.asarray(stream_toks, dtype="<i4").tobytes()).hexdigest(),
            "committed_tokens": len(stream_toks), "steps": steps, "breakdown_rounds": nb,
            "_bytes": by, "_elapsed_s": el,
        }
        if evk:
            out["_lm_ms"] = float(np.mean([x[0].elapsed_time(x[1]) for x in evk]))
            out["_lm_call_ms"] = float(np.mean([x[1].elapsed_time(x[2]) for x in ev]))
        if evc:
            out["_chain_ms"] = float(np.mean([x[0].elapsed_time(x[1]) for x in evc]))
        return out


def lm_head_verify(leg, n_rounds: int, seed_tag: int = 0):
    """Verify rows N(0,1) [B+1, hidden] of each round through the shared lm_head."""
    torch, synth = leg.torch, leg.synth
    rows = torch.from_numpy(np.stack([synth.verify_hidden(leg.sh, leg.B + 1, seed_tag + r) for r in range(n_rounds)]))
    rows = rows.to(leg.act).to(leg.dev)

    def verify(r, toks_r, out_r):
        leg.g.lm_head_argmax(rows[r], out=out_r, stream=leg.stream)
    return verify


def flip_verify(leg, flip, last):
    """Stand-in target (the target model is not built): row i < B takes the draft token with
    its lowest bit flipped where flip[r, i] is 1 (a valid, different id since the vocabulary
    size is even), the draft token itself elsewhere; row B is last[r]. One kernel per round."""
    torch = leg.torch
    assert leg.sh.vocab % 2 == 0, "the stand-in target flips the lowest bit of a token id"
    flip = flip.to(torch.int32).to(leg.dev)
    last = last.to(torch.int32).to(leg.dev)

    def verify(r, toks_r, out_r):
        torch.bitwise_xor(toks_r, flip[r], out=out_r[:leg.B])

    def prepare(tgt):
        tgt[:, leg.B] = last[:tgt.shape[0]]
    verify.prepare = prepare
    return verify


def accept_p_verify(leg, n_rounds: int, p: float, tag: int):
    """p-accept stand-in: row i keeps the draft token with probability p (pre-drawn uniforms)."""
    torch, synth = leg.torch, leg.synth
    u = torch.from_numpy(np.stack([synth.accept_draws(leg.B, r, tag) for r in range(n_rounds)]))
    flip = (u[:, 0, :leg.B] >= p).int()
    last = torch.floor(u[:, 2, leg.B] * leg.sh.vocab) % leg.sh.vocab
    return flip_verify(leg, flip, last)


def random_depth_verify(leg, n_rounds: int, tag: int):
    """Accepted length drawn uniformly from 0..B each round: the draft token is flipped at
    row k only (trims of random depth B - k)."""
    torch, synth = leg.torch, leg.synth
    B = leg.B
    flip = torch.zeros((n_rounds, B), dtype=torch.int32)
    for r in range(n_rounds):
        k = synth.random_depth_k(B, r, tag)
        if k < B:
            flip[r, k] = 1
    last = torch.tensor([synth.anchor_token(leg.sh, tag=90_000 + r) for r in range(n_rounds)])
    return flip_verify(leg, flip, last)


def public(d: dict) -> dict:
    return {k: v for k, v in d.items() if not k.startswith("_")}


def run_c1(args, sh, dw) -> dict:
    leg = Leg(sh, dw, 4, 1024)
    n = args.warmup + args.steps + min(args.steps, BREAKDOWN_ROUNDS)
    res = leg.run(args.warmup, args.steps, lm_head_verify(leg, n), resid_tag=1, anchor_tag=0, lm_timing=True)
    by = res["_bytes"]
    rs = res["rounds_per_s"]
    res["round_hbm_frac"] = round(by["round_lm_verify"] * rs / (HBM_PEAK_GBS * 1e9), 4)
    res["drafted_tok_s_hbm_frac"] = res["round_hbm_frac"]
    return res


def run_synthetic_p(args, sh, dw, B, context, steps, p, tag) -> dict:
    leg = Leg(sh, dw, B, context)
    n = args.warmup + steps + min(steps, BREAKDOWN_ROUNDS)
    res = leg.run(args.warmup, steps, accept_p_verify(leg, n, p, tag), resid_tag=1000 * (tag + 1), anchor_tag=tag)
    res["accept_p"] = round(p, 4)
    res["round_hbm_frac"] = round(res["_bytes"]["block_forward"] * res["rounds_per_s"] / (HBM_PEAK_GBS * 1e9), 4)
    return res


def run_c3(args, sh, dw) -> dict:
    """16384-row prefill slab (rows the window cannot see dropped before the encoder; the
    prefill is timed on its own), then random-depth rounds with the ring phase set so that
    the first round's append straddles the ring's last slot."""
    from block_drafting_dflash_amd import synth

    wl = synth.WORKLOADS["muse-bf16-ctx16384-wrap"]
    out = {"workload": wl.name, "context": wl.context, "widths": []}
    for B in wl.blocks:
        S = max(min(max(8 * B, 32), 128), B)
        Cs = (max(sh.window + S, sh.window + B + 1, 64) + 7) // 8 * 8
        phase = (Cs - 8 - wl.context) % Cs
        leg = Leg(sh, dw, B, wl.context, phase=phase)
        n = args.warmup + args.c3_steps + min(args.c3_steps, BREAKDOWN_ROUNDS)
        res = leg.run(args.warmup, args.c3_steps, random_depth_verify(leg, n, tag=B), resid_tag=5000 * B,
                      anchor_tag=B)
        slab_bytes = wl.context * sh.fc_in * 2
        kept = min(wl.context, sh.window)
        pre_alg = kept * sh.fc_in * 2 + sh.hidden * sh.fc_in * 2 + sh.layers * 2 * sh.kv_heads * sh.head_dim * (
            sh.hidden * 2 + kept * 2)
        res["prefill"] = {"ms": round(leg.prefill_ms, 3), "slab_bytes": slab_bytes, "rows_projected": kept,
                          "alg_bytes": pre_alg,
                          "gbs": round(pre_alg / (leg.prefill_ms * 1e-3) / 1e9, 1)}
        res["round_hbm_frac"] = round(res["_bytes"]["block_forward"] * res["rounds_per_s"] / (HBM_PEAK_GBS * 1e9), 4)
        out["widths"].append(public(res))
        del leg
    return out


def run_c0(args) -> dict:
    """The tiny f32 round: weights and ring fit the caches, so it is launch-latency bound."""
    import torch

    from block_drafting_dflash_amd import binding, synth

    wl = synth.WORKLOADS["tiny-f32-b4-ctx64"]
    dw = binding.to_device(wl.shape, synth.make_weights(wl.shape))
    leg = Leg(wl.shape, dw, 4, wl.context)
    n = args.warmup + args.c0_steps + min(args.c0_steps, BREAKDOWN_ROUNDS)
    res = leg.run(args.warmup, args.c0_steps, lm_head_verify(leg, n), resid_tag=1, anchor_tag=0)
    torch.cuda.synchronize()
    return {"workload": wl.name, **public(res)}


def run_q4(args) -> dict:
    """The 4-bit Muse-shaped drafter (fc, layers and lm_head in q4, group 64) after a
    2048-row context, one ring per width, each width with its own accept probability."""
    import torch

    from block_drafting_dflash_amd import binding, synth

    wl = synth.WORKLOADS["muse-q4-sweep-ctx2048"]
    sh = wl.shape
    t0 = time.time()
    dw = binding.to_device(sh, synth.make_weights(sh))
    torch.cuda.synchronize()
    print(f"[bench] q4 weights generated and resident in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    ps = synth.width_accept_p(wl.blocks)
    widths = [public(run_synthetic_p(args, sh, dw, B, wl.context, args.q4_steps, ps[B], tag=B)) for B in wl.blocks]
    return {"workload": wl.name, "widths": widths}


def run_adaptive(args, sh, dw) -> dict:
    """Rounds whose block the library's width controller picks between the declared depth 4 and
    the ceiling 16 (windows of 32 rounds, a challenge after every 3; shorter windows are too
    noisy under geometric accept lengths), fed with the rounds' real periods (spacing of the
    verify results' arrivals) and committed tokens, beside the same rounds at fixed widths 4
    and 16; p-accept stand-in target at p = 0.6 and 0.9, 2048-row context. The ring is sized
    for the ceiling."""
    import torch

    from block_drafting_dflash_amd import binding, synth

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    D, C, WIN, EVERY = 4, 16, 32, 3
    n = args.warmup + args.adaptive_steps
    out = {"depth": D, "ceiling": C, "window": WIN, "challenge_every": EVERY, "context": 2048, "runs": []}
    prefill = torch.from_numpy(synth.resid_rows(sh, 2048, 0)).to(torch.bfloat16).to(dev)
    resid = torch.from_numpy(np.stack([synth.resid_rows(sh, C + 1, 7000 + r) for r in range(n)]))
    resid = resid.to(torch.bfloat16).to(dev)
    u = torch.from_numpy(np.stack([synth.accept_draws(C, r, 33) for r in range(n)]))
    for p in (0.6, 0.9):
        for mode in ("fixed-4", "fixed-16", "adaptive"):
            g = binding.Drafter(sh, dw, max_block=C)
            g.cache_append(prefill, commit=True)
            flip = (u[:, 0, :C] >= p).int().to(dev)
            tgt = (torch.floor(u[:, 2, C] * sh.vocab) % sh.vocab).int()[:, None].repeat(1, C + 1).contiguous().to(dev)
            toks = torch.empty((n, C), dtype=torch.int32, device=dev)
            host = torch.empty(3, dtype=torch.int32, pin_memory=True)
            hv = host.numpy()
            ctl = binding.WidthController(D, C, WIN, EVERY) if mode == "adaptive" else None
            fixed = {"fixed-4": D, "fixed-16": C}.get(mode)
            anchor = synth.anchor_token(sh, tag=33)
            torch.cuda.synchronize()
            last = time.perf_counter()
            tokens, widths, t0 = 0, [], None
            for r in range(n):
                if r == args.warmup:
                    t0 = time.perf_counter()
                b = ctl.width() if ctl else fixed
                g.draft_block(anchor, b, tokens=toks[r, :b], stream=stream)
                torch.bitwise_xor(toks[r, :b], flip[r, :b], out=tgt[r, :b])
                hv[:] = -1
                g.verify_greedy(toks[r, :b], tgt[r, :b + 1], b, out=host, stream=stream)
                g.cache_append(resid[r, :b + 1], stream=stream)
                k, bonus, status = await_verify(hv)
                now = time.perf_counter()
                assert status == 0
                g.cache_trim(b - k)
                if ctl:
                    ctl.record(b, k + 1, (now - last) * 1e3)
                last = now
                anchor = bonus
                if r >= args.warmup:
                    tokens += k + 1
                    widths.append(b)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            run = {"p": p, "mode": mode, "rounds": len(widths), "committed_tok_s": round(tokens / el, 1),
                   "rounds_per_s": round(len(widths) / el, 1),
                   "rounds_at_ceiling": int(sum(1 for w in widths if w == C))}
            if ctl:
                st = ctl.state()
                run.update({"final_width": st["incumbent"], "challenges": st["challenges"],
                            "adoptions": st["adoptions"], "tok_per_ms_incumbent": round(st["incumbent_rate"], 3)})
            out["runs"].append(run)
            del g
    return out


def run_target(args) -> dict:
    """Speculative decoding against classic greedy decoding of the same synthetic target (the
    pages' comparison, on synthetic weights): the Muse-shaped target (10 layers, window 2048,
    full layers 4 and 9, streams captured at layers 1, 3, 5, 7, 9) and the drafter it feeds
    (fc 5 x 2048 -> 2048), sharing one device copy of the embedding table and lm_head. A
    1024-token prompt goes through the target in 32-row forwards, its captured streams into
    the drafter. Classic decode: one target forward per token, its argmax read back. A
    speculative round at block 4: draft, target verify forward over [anchor, drafts] (its
    captured streams kept), greedy verify into pinned host memory, the drafter's append of
    the captured rows, both trims. With random weights the drafter's proposals are rarely
    the target's tokens, so the rounds mostly commit one token each; the committed stream
    equals the classic one."""
    import torch

    from block_drafting_dflash_amd import binding, synth

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    t = synth.MUSE_BF16_TARGET
    dsh = synth.drafter_for(t, synth.MUSE_BF16)
    t0 = time.time()
    dw = synth.make_weights(dsh)
    tw = synth.make_target_weights(t, dw)
    ddev = binding.to_device(dsh, dw)
    tdev = binding.to_device(t, {k: v for k, v in tw.items() if k not in ("embed", "lm_head")})
    tdev["embed"], tdev["lm_head"] = ddev["embed"], ddev["lm_head"]
    del dw, tw
    torch.cuda.synchronize()
    print(f"[bench] target pair resident in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    prompt = torch.from_numpy(synth.prompt_tokens(t.vocab, 1024, tag=13).astype(np.int32)).to(dev)
    ncap = t.streams * t.hidden

    def prefill(tg, dr):
        a = None
        for s0 in range(0, 1024, tg.rows_max):
            n = min(tg.rows_max, 1024 - s0)
            cap = torch.empty((n, ncap), dtype=torch.bfloat16, device=dev) if dr else None
            a, _ = tg.forward(int(prompt[s0].item()), prompt[s0 + 1:s0 + n], n, capture=cap, stream=stream)
            tg.trim(0)
            if dr:
                dr.cache_append(cap, commit=True, stream=stream)
        return int(a[-1].item())

    # classic greedy decode
    tc = binding.Target(t, tdev, max_block=1)
    tok = prefill(tc, None)
    n_classic = args.target_steps
    classic = [tok]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    for i in range(n_classic):
        a, _ = tc.forward(classic[-1], None, 1, stream=stream)
        tc.trim(0)
        classic.append(int(a[0].item()))
    classic_s = time.perf_counter() - t0
    e0.record(stream)
    tc.forward(classic[-1], None, 1, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    fwd1_ms = e0.elapsed_time(e1)
    del tc
    # speculative rounds
    B = 4
    tg = binding.Target(t, tdev, max_block=B)
    dr = binding.Drafter(dsh, ddev, max_block=B)
    first = prefill(tg, dr)
    assert first == classic[0]
    n = args.warmup + args.target_steps
    toks = torch.empty((n, B), dtype=torch.int32, device=dev)
    av = torch.empty((n, B + 1), dtype=torch.int32, device=dev)
    cap = torch.empty((B + 1, ncap), dtype=torch.bfloat16, device=dev)
    host = torch.empty(3, dtype=torch.int32, pin_memory=True)
    hv = host.numpy()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ks, bonuses = [], []
    anchor = first
    torch.cuda.synchronize()
    t0 = None
    for r in range(n):
        if r == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        timed = r == n - 1
        if timed: ev[0].record(stream)
        dr.draft_block(anchor, B, tokens=toks[r], stream=stream)
        if timed: ev[1].record(stream)
        tg.forward(anchor, toks[r], B + 1, argmax=av[r], capture=cap, stream=stream)
        if timed: ev[2].record(stream)
        hv[:] = -1
        dr.verify_greedy(toks[r], av[r], B, out=host, stream=stream)
        dr.cache_append(cap, stream=stream)
        if timed: ev[3].record(stream)
        k, bonus, status = await_verify(hv)
        assert status == 0
        dr.cache_trim(B - k)
        tg.trim(B - k)
        ks.append(k)
        bonuses.append(bonus)
        anchor = bonus
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    rounds = args.target_steps
    d = toks.cpu().numpy()
    out = [first]
    for r in range(n):
        out += [int(x) for x in d[r, :ks[r]]] + [bonuses[r]]
    committed = sum(k + 1 for k in ks[args.warmup:])
    m = min(len(out), len(classic))
    tb = t.layers * (2 * (t.q_heads + 2 * t.kv_heads) * t.head_dim * t.hidden + 2 * 3 * t.intermediate * t.hidden) \
        + 2 * t.vocab * t.hidden
    return {"workload": "muse-bf16-target-b4-prompt1024", "block": B, "target_layers": t.layers,
            "classic_tok_s": round(n_classic / classic_s, 1), "classic_forward_ms": round(fwd1_ms, 4),
            "classic_forward_hbm_frac": round(tb / (fwd1_ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "speculative_rounds_per_s": round(rounds / el, 1), "speculative_committed_tok_s": round(committed / el, 1),
            "speedup_vs_classic": round((committed / el) / (n_classic / classic_s), 3),
            "mean_accepted": round(float(np.mean(ks[args.warmup:])), 4),
            "round_ms": {"draft": round(ev[0].elapsed_time(ev[1]), 4), "target_verify_forward": round(ev[1].elapsed_time(ev[2]), 4),
                         "verify_and_append": round(ev[2].elapsed_time(ev[3]), 4)},
            "committed_equals_classic": out[:m] == classic[:m], "tokens_compared": m, "rounds": rounds}


def run_dspark(args, weights, dw) -> dict:
    """The DSpark form of the Muse-shaped drafter (rank-256 Markov head, adjacent-pair RoPE,
    window 4096) at the pages' verify widths 8 and 10 (7 and 9 proposals per round), after a
    1024-row context, verify rows through the shared lm_head. The drafter's other tensors are
    the block-4 workload's (same seeds); the Markov factors are drawn for it. The chain's
    gamma step launches are event-timed in the breakdown rounds: per step the kernel streams
    markov_w2 once."""
    import torch

    from block_drafting_dflash_amd import binding, synth

    wl = synth.WORKLOADS["muse-dspark-bf16-w8-w10-ctx1024"]
    sh = wl.shape
    dd = dict(dw)
    for name in ("markov_w1", "markov_w2"):
        dd[name] = torch.from_numpy(synth.to_bf16_values(synth.draw_tensor(sh, name))).to(torch.bfloat16).cuda()
    torch.cuda.synchronize()
    widths = []
    for B in wl.blocks:
        leg = Leg(sh, dd, B, wl.context)
        n = args.warmup + args.dspark_steps + min(args.dspark_steps, BREAKDOWN_ROUNDS)
        res = leg.run(args.warmup, args.dspark_steps, lm_head_verify(leg, n, seed_tag=500 * B), resid_tag=7000 + B,
                      anchor_tag=B, chain_timing=True)
        by = res["_bytes"]
        step_ms = res["_chain_ms"] / B
        res.update(verify_width=B + 1, round_hbm_frac=round(by["round_lm_verify"] * res["rounds_per_s"] /
                                                              (HBM_PEAK_GBS * 1e9), 4),
                   chain_ms=round(res["_chain_ms"], 5), markov_step_us=round(1e3 * step_ms, 3),
                   markov_step_gbs=round(by["markov_step"] / (step_ms * 1e-3) / 1e9, 1))
        widths.append(public(res))
        del leg
        torch.cuda.empty_cache()
    best = max(widths, key=lambda w: w["markov_step_gbs"])
    step_bytes = alg_bytes(sh, 1, 0)["markov_step"]
    return {"workload": wl.name, "markov_rank": sh.markov_rank, "rope": sh.rope_style, "widths": widths,
            "roofline_markov_step": {"bound": "hbm", "kernel": "Markov chain step (markov_w2 202048x256 bf16 + "
                                                               "one f32 logit row)",
                                     "achieved": best["markov_step_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(best["markov_step_gbs"] / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes_per_launch": step_bytes,
                                     "avg_launch_us": best["markov_step_us"], "traffic": None}}


def run_batch(args, sh, dw) -> dict:
    """Independent sequences drafted together (dflash_batch_*): n sequences, each after its own
    1024-row context, block 4, verify rows N(0,1) of all sequences through the shared lm_head
    in one call, one verify launch, one append of every sequence's 5 rows, per-sequence trims;
    the host waits for the n verify results in pinned memory. One sequence alone is the
    block-4 round of the main leg through the batch entry points."""
    import torch

    from block_drafting_dflash_amd import binding, synth
    from block_drafting_dflash_amd.counters import RoundCounters

    B, ctx_rows = 4, 1024
    out = {"workload": "muse-bf16-b4-ctx1024-batch", "block": B, "context": ctx_rows, "sizes": []}
    stream = torch.cuda.current_stream()
    for n in args.batch_sizes:
        bt = binding.Batch(sh, dw, n, B)
        slab = torch.cat([torch.from_numpy(synth.resid_rows(sh, ctx_rows, 5000 + s)) for s in range(n)])
        bt.append(slab.to(binding.act_torch_dtype(sh)).cuda(), [ctx_rows] * n, commit=True)
        del slab
        steps, warm = args.batch_steps, args.warmup
        nb = min(steps, BREAKDOWN_ROUNDS)
        total = warm + steps + nb
        rows = torch.from_numpy(np.stack([np.concatenate([synth.verify_hidden(sh, B + 1, 20000 + 100 * r + s)
                                                          for s in range(n)]) for r in range(min(total, 64))]))
        rows = rows.to(binding.act_torch_dtype(sh)).cuda()
        resid = torch.from_numpy(np.stack([np.concatenate([synth.resid_rows(sh, B + 1, 30000 + 100 * r + s)
                                                           for s in range(n)]) for r in range(min(total, 64))]))
        resid = resid.to(binding.act_torch_dtype(sh)).cuda()
        toks = torch.empty((total, n, B), dtype=torch.int32, device="cuda")
        tgt = torch.empty((total, n, B + 1), dtype=torch.int32, device="cuda")
        host = torch.empty((n, 3), dtype=torch.int32, pin_memory=True)
        hv = host.numpy()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nb)]
        anchors = [synth.anchor_token(sh, tag=s) for s in range(n)]
        cnt = RoundCounters()
        stream_toks = []
        torch.cuda.synchronize()
        t0 = el = None
        for r in range(total):
            if r == warm:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            if r == warm + steps:
                torch.cuda.synchronize()
                el = time.perf_counter() - t0
            e = ev[r - warm - steps] if r >= warm + steps else None
            if e: e[0].record(stream)
            bt.draft(anchors, B, tokens=toks[r], stream=stream)
            if e: e[1].record(stream)
            bt.lm_head_argmax(rows[r % 64].view(n * (B + 1), -1), out=tgt[r].view(-1), stream=stream)
            hv[:] = -1
            bt.verify_greedy(toks[r], tgt[r], B, out=host, stream=stream)
            bt.append(resid[r % 64].view(n * (B + 1), -1), [B + 1] * n, stream=stream)
            if e: e[2].record(stream)
            t_wait = time.perf_counter()
            while (hv[:, 0] == -1).any() or (hv[:, 2] == -1).any() or ((hv[:, 1] == -1) & (hv[:, 2] != 1)).any():
                if time.perf_counter() - t_wait > 10.0:
                    raise RuntimeError("the batch verify results did not arrive")
            res = hv.copy()
            assert (res[:, 2] == 0).all()
            bt.trim([B - int(k) for k in res[:, 0]])
            if warm <= r < warm + steps:
                for s in range(n):
                    cnt.record(B, int(res[s, 0]))
            anchors = [int(b) for b in res[:, 1]]
        torch.cuda.synchronize()
        rs = steps / el
        d_ms = float(np.mean([x[0].elapsed_time(x[1]) for x in ev]))
        by = alg_bytes(sh, B, ctx_rows)
        weights = by["fc"] + by["layers"] + by["lm_head"]
        per_seq = by["block_forward"] - weights
        fwd_bytes = weights + n * per_seq
        out["sizes"].append({
            "n_seq": n, "rows_per_gemm": n * (B + 1), "rounds_per_s": round(rs, 2),
            "sequence_rounds_per_s": round(n * rs, 2), "drafted_tok_s": round(n * B * rs, 1),
            "round_ms": round(1e3 * el / steps, 4), "draft_ms": round(d_ms, 4),
            "round_ms_with_events": round(float(np.mean([x[0].elapsed_time(x[2]) for x in ev])), 4),
            "draft_hbm_frac": round(fwd_bytes / (d_ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "mean_accepted": round(cnt.as_dict()["mean_accepted"], 4), "steps": steps})
        print(f"[bench] batch of {n}: {n * rs:.1f} sequence-rounds/s", file=sys.stderr, flush=True)
        del bt, rows, resid, toks, tgt
        torch.cuda.empty_cache()
    return out


def stream_probe(mib: int, reps: int = 10) -> dict:
    """The in-repo HBM streaming-read probe: mib MiB read `reps` times, event-timed."""
    import torch

    from block_drafting_dflash_amd import binding

    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    best = None
    for groups in (1024, 2048, 4096):
        sink = torch.empty(groups, dtype=torch.int32, device="cuda")
        binding.hbm_read_probe(src, sink, groups)  # warm
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            binding.hbm_read_probe(src, sink, groups)
        e1.record()
        torch.cuda.synchronize()
        gbs = (mib << 20) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "groups": groups}
    return {"mib": mib, "reps": reps, **best, "frac_of_peak": round(best["gbs"] / HBM_PEAK_GBS, 4)}


def cpu_baseline(sh, weights, budget_s: float) -> dict:
    """The oracle as it stands, timed on the host cores over a bounded sample of rounds."""
    from block_drafting_dflash_amd import synth
    from oracle import dflash_oracle as O

    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    B = 4
    od = O.OracleDrafter(sh, weights, B)
    t0 = time.time()
    od.append(synth.resid_rows(sh, 1024, 0), commit=True)
    od.draft(0, B)  # warms the f64 weight cache (not timed)
    od.lm_head_argmax(synth.verify_hidden(sh, B + 1, 0))
    setup = time.time() - t0
    anchor = synth.anchor_token(sh)
    done = 0
    t1 = time.perf_counter()
    while True:
        d = od.draft(anchor, B).tokens
        a, _ = od.lm_head_argmax(synth.verify_hidden(sh, B + 1, done))
        k, bonus = O.verify_greedy(d, a)
        od.append(synth.resid_rows(sh, B + 1, done + 1))
        od.trim(B - k)
        anchor = bonus
        done += 1
        if time.perf_counter() - t1 > budget_s or done >= 400:
            break
    el = time.perf_counter() - t1
    return {"value": done / el, "unit": "rounds/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} full block-4 rounds (draft, verify lm_head, verify, append, trim) of "
                      f"muse-bf16-b4-ctx1024 after an untimed 1024-row prefill and f64 weight "
                      f"conversion ({setup:.1f}s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--block16-steps", type=int, default=320)
    ap.add_argument("--c3-steps", type=int, default=128, help="timed rounds per width at 16384 context (0 = skip)")
    ap.add_argument("--q4-steps", type=int, default=200, help="timed rounds per width of the q4 sweep (0 = skip)")
    ap.add_argument("--c0-steps", type=int, default=500, help="timed rounds of the tiny f32 round (0 = skip)")
    ap.add_argument("--target-steps", type=int, default=96,
                    help="rounds (and classic decode tokens) against the synthetic target (0 = skip)")
    ap.add_argument("--dspark-steps", type=int, default=200,
                    help="timed rounds per verify width of the DSpark drafter (0 = skip)")
    ap.add_argument("--batch-steps", type=int, default=200,
                    help="timed rounds per batch size of the batched-sequence leg (0 = skip)")
    ap.add_argument("--batch-sizes", type=lambda t: [int(x) for x in t.split(",")], default=[1, 2, 4, 8])
    ap.add_argument("--adaptive-steps", type=int, default=768,
                    help="rounds per run of the adaptive-width comparison (0 = skip)")
    ap.add_argument("--probe-mib", type=int, default=1024, help="HBM streaming-read probe size (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB five times (counter reference) and exit")
    args = ap.parse_args()
    if args.copy_probe_mib:
        import torch
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_mib": args.copy_probe_mib, "launches": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the round at batch 1 is measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch

    from block_drafting_dflash_amd import binding, synth

    if not os.path.exists(binding.LIB_PATH):
        from block_drafting_dflash_amd import build as _b
        _b.build()
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS["muse-bf16-b4-ctx1024"]
    sh = wl.shape
    t0 = time.time()
    weights = synth.make_weights(sh)
    dw = binding.to_device(sh, weights)
    torch.cuda.synchronize()
    print(f"[bench] weights generated and resident in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    res = run_c1(args, sh, dw)
    print(f"[bench] block 4: {res['rounds_per_s']} rounds/s", file=sys.stderr, flush=True)
    b16 = None
    if args.block16_steps > 0:
        wl2 = synth.WORKLOADS["muse-bf16-b16-ctx4096"]
        b16 = {"workload": wl2.name, **public(run_synthetic_p(args, sh, dw, 16, wl2.context, args.block16_steps,
                                                               wl2.accept_p, tag=0))}
        print(f"[bench] block 16: {b16['rounds_per_s']} rounds/s", file=sys.stderr, flush=True)
    c3 = run_c3(args, sh, dw) if args.c3_steps > 0 else None
    if c3:
        print("[bench] 16384 context done", file=sys.stderr, flush=True)
    adaptive = run_adaptive(args, sh, dw) if args.adaptive_steps > 0 else None
    dspark = run_dspark(args, weights, dw) if args.dspark_steps > 0 else None
    batch = run_batch(args, sh, dw) if args.batch_steps > 0 else None
    if dspark:
        print("[bench] dspark: " + ", ".join(f"width {w['verify_width']} {w['rounds_per_s']} rounds/s"
                                             for w in dspark["widths"]), file=sys.stderr, flush=True)
    del dw
    torch.cuda.empty_cache()
    target = run_target(args) if args.target_steps > 0 else None
    torch.cuda.empty_cache()
    q4 = run_q4(args) if args.q4_steps > 0 else None
    c0 = run_c0(args) if args.c0_steps > 0 else None
    probe = stream_probe(args.probe_mib) if args.probe_mib > 0 else None
    cpu = None if args.no_cpu_baseline else cpu_baseline(sh, weights, args.cpu_budget)
    traffic = counted_traffic()
    by = res["_bytes"]
    lm_ms = res["_lm_ms"]
    fwd_ms = res["block_forward_ms"]
    line = {
        "metric": "DFlash rounds/s at block 4 (B=1), with drafted tok/s and % of HBM roofline",
        "value": res["rounds_per_s"], "unit": "rounds/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["round_ms"]["mean"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) weights, N(0,1) residual/verify rows)",
        "config": {"workload": "muse-bf16-b4-ctx1024", "block": 4, "context": 1024, "window": 2048,
                   "hidden": 2048, "layers": 5, "vocab": 202048},
        "drafted_tok_s": res["drafted_tok_s"],
        "round_hbm_frac": res["round_hbm_frac"],
        "round_ms": res["round_ms"], "rounds_per_s_median": res["rounds_per_s_median"],
        "counters": {k: res[k] for k in ("draft_rounds", "draft_n", "draft_n_accepted", "mean_accepted",
                                         "mean_accepted_with_bonus", "accept_hist", "committed_tok_s",
                                         "committed_token_sha256", "committed_tokens")},
        "block_forward": {"ms": fwd_ms, "per_s": round(1e3 / fwd_ms, 1), "hbm_frac": res["block_forward_hbm_frac"],
                          "draft_ms": res["draft_ms"], "append_ms": res["append_ms"]},
        "roofline": {"bound": "hbm", "kernel": "lm_head argmax GEMM (202048x2048 bf16, 5 verify rows)",
                     "achieved": round(by["lm_head"] / (lm_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(by["lm_head"] / (lm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic / (lm_ms * 1e-3) / 1e9, 1) if traffic else None),
                     "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": by["lm_head"],
                     "avg_launch_ms": round(lm_ms, 5), "avg_call_ms": round(res["_lm_call_ms"], 5)},
        "roofline_block_forward": {"bound": "hbm", "span": "drafter + lm_head block forward (append fc + draft)",
                                   "achieved": round(by["block_forward"] / (fwd_ms * 1e-3) / 1e9, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": res["block_forward_hbm_frac"],
                                   "algorithmic_bytes": by["block_forward"], "avg_ms": fwd_ms},
        "hbm_stream_probe": probe,
        "block16": b16,
        "ctx16384": c3,
        "adaptive_width": adaptive,
        "dspark": dspark,
        "batch": batch,
        "target": target,
        "q4": q4,
        "tiny_f32": c0,
        "cpu_baseline": cpu,
        "mean_accepted": res["mean_accepted"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
