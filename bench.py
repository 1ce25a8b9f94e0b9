"""Throughput of one DFlash speculative round at batch 1 on one MI355X.

A step is one whole round over one block of synthetic input: the drafter's block forward
(dflash_draft_block), the target verify rows through the shared lm_head
(dflash_lm_head_argmax), greedy verify (dflash_verify_greedy, whose kernel writes (k,
bonus, status) into pinned host memory), the append of the B+1 verify residual rows
(dflash_cache_append), the host's wait for that result (polled in pinned memory, so the
append still runs while the host trims and enqueues the next round) and the trim
(dflash_cache_trim). Inputs are resident in HBM before the timed region starts. The
timed rounds record no timing events (a HIP event record holds the stream for a few
microseconds); a pass of up to 100 more rounds after them records events around the draft,
the append and the lm_head argmax kernel for the per-call breakdown and `roofline`.

Workload (timed as `value`): muse-bf16-b4-ctx1024 -- Muse-assistant-shaped bf16 drafter
(hidden 2048, 5 layers, 32/4 heads x 128, intermediate 6144, vocab 202048, untied lm_head,
fc 20480 -> 2048), context 1024, window 2048, block 4, verify rows N(0,1) through the
lm_head. Also reported: the block-16 round (muse-bf16-b16-ctx4096, p = 0.6 synthetic
target), the 4-bit width sweep (muse-q4-sweep-ctx2048, blocks 4/5/8/16) and the CPU oracle
timed on the host cores.

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

    Weights cost 2 bytes per parameter in bf16 and 9/16 in q4 (a 4-bit code plus a bf16
    scale and bias per 64 inputs); activations, the ring and the embedding rows are bf16."""
    e = 2  # bf16
    we = 9 / 16 if sh.weight_dtype == "q4" else 2
    H, I, V, F = sh.hidden, sh.intermediate, sh.vocab, sh.fc_in
    qd, kvd = sh.q_heads * sh.head_dim, sh.kv_heads * sh.head_dim
    layer = (qd * H + 2 * kvd * H + H * qd + 2 * I * H + H * I) * we
    fc = H * F * we
    lm = V * H * we
    kv = sh.layers * 2 * min(ctx_visible, sh.window) * kvd * e
    inputs = (block + 1) * F * e + (block + 1) * H * e
    fwd = fc + sh.layers * layer + lm + kv + inputs
    return {"fc": fc, "layers": sh.layers * layer, "lm_head": lm, "kv": kv, "block_forward": fwd,
            "round_lm_verify": fwd + lm + (block + 1) * H * e}


def counted_traffic():
    """HBM bytes per lm_head launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs
    (scaled by the same counters on a 1 GiB copy), or None if the kernel source changed since."""
    try:
        d = json.load(open(os.path.join(ROOT, "profiles", "lm_head_argmax_counters.json")))
        src = open(os.path.join(ROOT, "block_drafting_dflash_amd", "csrc", "gemm_impl.h"), "rb").read()
    except OSError:
        return None
    return d["traffic_bytes"] if d.get("kernel_source_sha256") == hashlib.sha256(src).hexdigest() else None


def run_gpu(args):
    import torch

    from block_drafting_dflash_amd import binding, synth

    if not os.path.exists(binding.LIB_PATH):
        from block_drafting_dflash_amd import build as _b
        _b.build()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    wl = synth.WORKLOADS["muse-bf16-b4-ctx1024"]
    sh = wl.shape
    t0 = time.time()
    weights = synth.make_weights(sh)
    dw = binding.to_device(sh, weights)
    torch.cuda.synchronize()
    print(f"[bench] weights generated and resident in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    # ---------------- block 4, verify rows through the shared lm_head ------------------
    B = 4
    g = binding.Drafter(sh, dw, max_block=B)
    g.cache_append(torch.from_numpy(synth.resid_rows(sh, wl.context, 0)).to(torch.bfloat16).to(dev), commit=True)
    # timed rounds carry no timing events (each event record costs the stream a few
    # microseconds); a shorter pass after them, with events, gives the breakdown
    nb = min(args.steps, BREAKDOWN_ROUNDS)
    n = args.warmup + args.steps + nb
    vrows = torch.from_numpy(np.stack([synth.verify_hidden(sh, B + 1, r) for r in range(n)])).to(torch.bfloat16).to(dev)
    resid = torch.from_numpy(np.stack([synth.resid_rows(sh, B + 1, r + 1) for r in range(n)])).to(torch.bfloat16).to(dev)
    toks = torch.empty(B, dtype=torch.int32, device=dev)
    a = torch.empty(B + 1, dtype=torch.int32, device=dev)
    host = torch.empty(3, dtype=torch.int32, pin_memory=True)  # the verify kernel writes (k, bonus, status) here
    hv = host.numpy()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(nb)]
    # events around the argmax kernel alone (the library records them on the call's stream)
    evk = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nb)]
    for pair in evk:
        for x in pair:
            x.record(stream)  # creates the underlying events before the timed region
    anchor = synth.anchor_token(sh)
    ks = []
    torch.cuda.synchronize()
    t_start = elapsed = None
    b0 = args.warmup + args.steps  # first breakdown round
    for r in range(n):
        if r == args.warmup:
            torch.cuda.synchronize()
            t_start = time.perf_counter()
        if r == b0:
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t_start
        e = ev[r - b0] if r >= b0 else None
        if e: e[0].record(stream)
        g.draft_block(anchor, B, tokens=toks, stream=stream)
        if e: e[1].record(stream)
        if e: g.time_next_argmax(*evk[r - b0])
        g.lm_head_argmax(vrows[r], out=a, stream=stream)
        if e: e[2].record(stream)
        hv[:] = -1
        g.verify_greedy(toks, a, B, out=host, stream=stream)
        if e: e[3].record(stream)
        g.cache_append(resid[r], stream=stream)
        if e: e[4].record(stream)
        k, bonus, status = await_verify(hv)  # the round's one host round trip
        assert status == 0
        g.cache_trim(B - k)
        anchor = bonus
        ks.append(k)
    torch.cuda.synchronize()
    ms_draft = [x[0].elapsed_time(x[1]) for x in ev]
    ms_lm_call = [x[1].elapsed_time(x[2]) for x in ev]
    ms_lm = [x[0].elapsed_time(x[1]) for x in evk]
    ms_append = [x[3].elapsed_time(x[4]) for x in ev]
    e_end = g.cache_state()[0]
    by = alg_bytes(sh, B, e_end)
    rounds_s = args.steps / elapsed
    lm_ms = float(np.mean(ms_lm))
    fwd_ms = float(np.mean(ms_draft) + np.mean(ms_append))
    res = {
        "rounds_per_s": rounds_s, "ms_per_step": 1e3 * elapsed / args.steps, "drafted_tok_s": rounds_s * B,
        "round_hbm_frac": by["round_lm_verify"] * rounds_s / (HBM_PEAK_GBS * 1e9),
        "drafted_tok_s_hbm_frac": by["round_lm_verify"] * rounds_s / (HBM_PEAK_GBS * 1e9),
        "block_forward_ms": fwd_ms, "block_forward_per_s": 1e3 / fwd_ms,
        "block_forward_hbm_frac": by["block_forward"] / (fwd_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "draft_ms": float(np.mean(ms_draft)), "append_ms": float(np.mean(ms_append)),
        "lm_head_ms": lm_ms, "lm_head_gbs": by["lm_head"] / (lm_ms * 1e-3) / 1e9,
        "lm_head_call_ms": float(np.mean(ms_lm_call)),
        "mean_accepted": float(np.mean(ks[args.warmup:b0])), "bytes": by, "breakdown_rounds": nb,
    }

    # ---------------- block 16, p = 0.6 synthetic target --------------------------------
    b16 = None
    if args.block16_steps > 0:
        del g
        wl2 = synth.WORKLOADS["muse-bf16-b16-ctx4096"]
        b16 = synthetic_rounds(sh, dw, 16, wl2.context, args.warmup, args.block16_steps, wl2.accept_p, tag=0)
        b16 = {"workload": wl2.name, **b16}
    return sh, weights, dw, res, b16


def synthetic_rounds(sh, dw, B: int, context: int, warmup: int, steps: int, p: float, tag: int) -> dict:
    """Rounds of block B whose verify-row argmaxes come from the p-accept stand-in target
    (computed on the device from pre-drawn uniforms): draft, verify (result written into
    pinned host memory), append, the host's wait for (k, bonus), trim. The block forward is
    the event-timed draft plus append."""
    import torch

    from block_drafting_dflash_amd import binding, synth

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    g = binding.Drafter(sh, dw, max_block=B)
    g.cache_append(torch.from_numpy(synth.resid_rows(sh, context, 0)).to(torch.bfloat16).to(dev), commit=True)
    nb = min(steps, BREAKDOWN_ROUNDS)  # event-timed rounds after the timed ones
    n = warmup + steps + nb
    resid = torch.from_numpy(np.stack([synth.resid_rows(sh, B + 1, 1000 * (tag + 1) + r) for r in range(n)]))
    resid = resid.to(torch.bfloat16).to(dev)
    u = torch.from_numpy(np.stack([synth.accept_draws(B, r, tag) for r in range(n)])).to(dev)  # f64 [n, 3, B+1]
    V = sh.vocab
    # the stand-in target's draws that do not depend on the draft, made before timing: per
    # row a 0/1 word that rejects the row (its token then differs from the draft token in the
    # lowest bit, a valid id since the vocabulary size is even), and the bonus row's token
    assert V % 2 == 0, "the stand-in target flips the lowest bit of a token id"
    flip = (u[:, 0, :B] >= p).int()
    tgt_all = torch.empty((n, B + 1), dtype=torch.int32, device=dev)
    tgt_all[:, B] = (torch.floor(u[:, 2, B] * V) % V).int()
    toks = torch.empty(B, dtype=torch.int32, device=dev)
    host = torch.empty(3, dtype=torch.int32, pin_memory=True)  # the verify kernel writes (k, bonus, status) here
    hv = host.numpy()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nb)]
    anchor = synth.anchor_token(sh, tag=tag)
    ks = []
    torch.cuda.synchronize()
    t0 = el = None
    b0 = warmup + steps
    for r in range(n):
        if r == warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        if r == b0:
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
        e = ev[r - b0] if r >= b0 else None
        if e: e[0].record(stream)
        g.draft_block(anchor, B, tokens=toks, stream=stream)
        if e: e[1].record(stream)
        # stand-in for the target's verify-row argmaxes (the target model is out of scope):
        # row i keeps the draft token with probability p, else another token (one kernel)
        tgt = tgt_all[r]
        torch.bitwise_xor(toks, flip[r], out=tgt[:B])
        hv[:] = -1
        g.verify_greedy(toks, tgt, B, out=host, stream=stream)
        if e: e[2].record(stream)
        g.cache_append(resid[r], stream=stream)
        if e: e[3].record(stream)
        k, bonus, status = await_verify(hv)  # the round's one host round trip
        assert status == 0
        g.cache_trim(B - k)
        anchor = bonus
        ks.append(k)
    torch.cuda.synchronize()
    by = alg_bytes(sh, B, g.cache_state()[0])
    rs = steps / el
    fwd = float(np.mean([x[0].elapsed_time(x[1]) + x[2].elapsed_time(x[3]) for x in ev]))
    return {"block": B, "accept_p": round(p, 4), "rounds_per_s": round(rs, 2), "drafted_tok_s": round(rs * B, 1),
            "round_hbm_frac": round(by["block_forward"] * rs / (HBM_PEAK_GBS * 1e9), 4),
            "block_forward_ms": round(fwd, 4),
            "block_forward_hbm_frac": round(by["block_forward"] / (fwd * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "mean_accepted": round(float(np.mean(ks[warmup:b0])), 4), "steps": steps}


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
    widths = [synthetic_rounds(sh, dw, B, wl.context, args.warmup, args.q4_steps, ps[B], tag=B) for B in wl.blocks]
    return {"workload": wl.name, "widths": widths}



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
    ap.add_argument("--q4-steps", type=int, default=200, help="timed rounds per width of the q4 sweep (0 = skip)")
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
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the round at batch 1 is measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    sh, weights, dw, res, b16 = run_gpu(args)
    del dw
    q4 = run_q4(args) if args.q4_steps > 0 else None
    cpu = None if args.no_cpu_baseline else cpu_baseline(sh, weights, args.cpu_budget)
    traffic = counted_traffic()
    line = {
        "metric": "DFlash rounds/s at block 4 (B=1), with drafted tok/s and % of HBM roofline",
        "value": round(res["rounds_per_s"], 2), "unit": "rounds/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) weights, N(0,1) residual/verify rows)",
        "config": {"workload": "muse-bf16-b4-ctx1024", "block": 4, "context": 1024, "window": 2048,
                   "hidden": 2048, "layers": 5, "vocab": 202048},
        "drafted_tok_s": round(res["drafted_tok_s"], 1),
        "round_hbm_frac": round(res["round_hbm_frac"], 4),
        "block_forward": {"ms": round(res["block_forward_ms"], 4), "per_s": round(res["block_forward_per_s"], 1),
                          "hbm_frac": round(res["block_forward_hbm_frac"], 4),
                          "draft_ms": round(res["draft_ms"], 4), "append_ms": round(res["append_ms"], 4)},
        "roofline": {"bound": "hbm", "kernel": "lm_head argmax GEMM (202048x2048 bf16, 5 verify rows)",
                     "achieved": round(res["lm_head_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(res["lm_head_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic / (res["lm_head_ms"] * 1e-3) / 1e9, 1) if traffic else None),
                     "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": res["bytes"]["lm_head"],
                     "avg_launch_ms": round(res["lm_head_ms"], 5),
                     "avg_call_ms": round(res["lm_head_call_ms"], 5)},
        "block16": b16,
        "q4": q4,
        "cpu_baseline": cpu,
        "mean_accepted": res["mean_accepted"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
