"""Per-kernel summary of rocprofv3 runs over bench.py.

Inputs are the CSV outputs of separate rocprofv3 runs of one bench command: a kernel trace
(durations), a FETCH_SIZE pass and a WRITE_SIZE pass (HBM bytes, KiB per dispatch), an SQ pass
(MfmaUtil, VALUBusy, SQ_INSTS_MFMA, SQ_INSTS_VALU), and the FETCH_SIZE / WRITE_SIZE passes
over `bench.py --copy-probe-mib N` (a device copy of known size, which calibrates each
counter: the copy reads and writes N MiB per launch).

Dispatches are split into the bench's legs at each run of weight-repack kernels (every leg
creates its own context), and each GEMM instantiation is named by its role from its
template arguments and launch grid. Algorithmic bytes per launch are the weights the launch
streams (each read once) plus, for attention, the live K/V window of one layer.

Usage:
  python -m block_drafting_dflash_amd.profile_summary --trace T.csv --fetch F.csv --write W.csv \
      --sq S.csv --copy-fetch CF.csv --copy-write CW.csv --copy-mib 1024 --legs b4,b16 [--out X.md]
"""
from __future__ import annotations

import argparse
import collections
import csv
import re
import statistics
from typing import Dict, List, Optional

PEAK_GBS = 8000.0

# Muse-shaped drafter (hidden 2048, 5 layers, 32/4 heads x 128, intermediate 6144, vocab
# 202048, fc 20480 -> 2048): weight elements of each GEMM role
H, I, V, F, QD, KVD = 2048, 6144, 202048, 20480, 32 * 128, 4 * 128
ELEMS = {"lm_head": V * H, "gate/up": 2 * I * H, "QKV or K/V projection": (QD + 2 * KVD) * H, "down": H * I,
         "O": H * QD, "fc": H * F}


def read_csv(path: Optional[str]) -> List[dict]:
    if not path:
        return []
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def gemm_role(name: str, wgs: int = 0) -> Optional[str]:
    """The GEMM's role from its template arguments (wgs: its work-groups, which tell the
    DSpark lm_head's logit store from the projections that share its arguments)."""
    m = re.search(r"gemm_kernel<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (true|false)>", name)
    if not m:
        return None
    wt, rt, nb, epi, xsrc, t, nch, ch, split = m.groups()
    epi, nb, xsrc, nch, ch = int(epi), int(nb), int(xsrc), int(nch), int(ch)
    k_per_wave = nch * ch * 32
    if epi == 3:
        return "lm_head"
    if nb == 2:
        return "gate/up"
    if epi == 1:
        return "down" if k_per_wave * 8 == I else "O"
    if epi == 0 and xsrc in (2, 3, 4, 5):  # normed rows: one staging, a second gain row, two phases
        return "QKV or K/V projection"
    if epi == 0 and xsrc == 0 and k_per_wave * 8 == F:
        return "fc"
    if epi == 0 and xsrc == 0 and wgs >= V // 16:
        return "lm_head"  # every row's logits stored (DSpark)
    if epi == 0 and xsrc == 0:
        return "QKV or K/V projection"  # normed rows streamed from planes (long blocks)
    return None


def short(name: str) -> str:
    name = name.replace("void ", "").replace("dflash::", "")
    return name.split("(")[0].strip()


def split_legs(rows: List[dict]) -> List[List[dict]]:
    """Dispatches in order, cut into legs at each run of repack kernels; each leg keeps only
    its rounds, from its first block embedding on (the repack and the context prefill before
    it are left out)."""
    rows = sorted(rows, key=lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0))
    legs: List[List[dict]] = []
    in_pack = False
    started = False
    for r in rows:
        is_pack = any(k in r["Kernel_Name"] for k in ("pack_kernel", "pack_q4_kernel", "deinterleave_kernel"))
        if is_pack and not in_pack:
            legs.append([])
            started = False
        in_pack = is_pack
        started = started or re.search(r"embed(_batch)?_kernel", r["Kernel_Name"]) is not None
        if legs and started:
            legs[-1].append(r)
    return legs


def by_dispatch(rows: List[dict]) -> Dict[int, Dict[str, float]]:
    out: Dict[int, Dict[str, float]] = collections.defaultdict(dict)
    for r in rows:
        out[int(r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def counter_legs(rows: List[dict]) -> List[Dict[str, Dict[str, List[float]]]]:
    """Per leg: kernel name -> counter -> per-dispatch values (legs split like the trace)."""
    disp = {}
    for r in rows:
        disp.setdefault(int(r["Dispatch_Id"]), r)
    vals = by_dispatch(rows)
    legs = split_legs(list(disp.values()))
    out = []
    for leg in legs:
        d: Dict[str, Dict[str, List[float]]] = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in leg:
            for c, v in vals[int(r["Dispatch_Id"])].items():
                d[r["Kernel_Name"]][c].append(v)
        out.append(d)
    return out


def copy_scale(rows: List[dict], counter: str, mib: int) -> Optional[float]:
    """Bytes per counted KiB: the copy moves mib MiB each way per launch."""
    vals = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()]
    if not vals:
        vals = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter]
    if not vals:
        return None
    kib = statistics.median(vals)
    return (mib << 20) / kib if kib > 0 else None


def lm_head_traffic(args) -> Optional[dict]:
    """Counted HBM bytes per launch of the verify-row lm_head argmax (single operand plane) in
    the first leg, from the FETCH_SIZE and WRITE_SIZE passes and the copy calibration."""
    fs = copy_scale(read_csv(args.copy_fetch), "FETCH_SIZE", args.copy_mib)
    ws = copy_scale(read_csv(args.copy_write), "WRITE_SIZE", args.copy_mib)
    fetch, write = counter_legs(read_csv(args.fetch)), counter_legs(read_csv(args.write))
    if not (fs and ws and fetch and write):
        return None
    for k in fetch[0]:
        if gemm_role(k) == "lm_head" and "false>" in k:
            f = statistics.median(fetch[0][k]["FETCH_SIZE"])
            w = statistics.median(write[0][k]["WRITE_SIZE"])
            return {"kernel": short(k), "fetch_kib": f, "write_kib": w, "fetch_scale": fs, "write_scale": ws,
                    "traffic_bytes": f * fs + w * ws}
    return None


def summarize(args) -> str:
    trace = read_csv(args.trace)
    legs = split_legs(trace)
    names = args.legs.split(",")
    fetch, write, sq = counter_legs(read_csv(args.fetch)), counter_legs(read_csv(args.write)), counter_legs(read_csv(args.sq))
    cf, cw = read_csv(args.copy_fetch), read_csv(args.copy_write)
    fs = copy_scale(cf, "FETCH_SIZE", args.copy_mib)
    ws = copy_scale(cw, "WRITE_SIZE", args.copy_mib)
    lines = []
    lines.append(f"FETCH_SIZE scale {fs:.4f} bytes per counted KiB, WRITE_SIZE scale {ws:.4f} "
                 f"(a {args.copy_mib} MiB device copy, per launch)." if fs and ws else "No copy calibration.")
    lines.append("")
    for li, leg in enumerate(legs):
        if li >= len(names):
            break
        lines.append(f"## {names[li]}")
        lines.append("")
        lines.append("| kernel | role | calls | median us | p90 us | alg MB | GB/s | frac of 8 TB/s | counted MB "
                     "(fetch+write) | counted/alg | MfmaUtil % | VALUBusy % | MFMA inst | VALU inst |")
        lines.append("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
        per: Dict[str, List[float]] = collections.defaultdict(list)
        wgs: Dict[str, int] = {}
        for r in leg:
            per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            try:
                wgs[r["Kernel_Name"]] = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            except (KeyError, ValueError):
                wgs[r["Kernel_Name"]] = 0
        total = sum(sum(v) for v in per.values())
        rows = []
        for k, ds in per.items():
            role = gemm_role(k, wgs.get(k, 0))
            alg = ELEMS[role] * (9 / 16 if short(k).startswith("gemm_kernel<2") else 2) if role else None
            mk = re.search(r"markov_step_kernel<(true|false), (\d+)>", k)
            if mk:  # markov_w2 [V, rank] once plus one f32 logit row
                role, alg = "Markov chain step", V * int(mk.group(2)) * (2 if mk.group(1) == "true" else 4) + V * 4
            if "attn_mfma_batch" in k:
                role, alg = "attention (every sequence of a batch)", None
            elif "attn_mfma" in k:
                kv = [int(x) for x in str(args.kv_rows).split(",")]
                role, alg = "attention (live K/V of one layer)", kv[min(li, len(kv) - 1)] * KVD * 2 * 2
            med = statistics.median(ds)
            p90 = sorted(ds)[int(0.9 * (len(ds) - 1))]
            gbs = alg / (med * 1e-6) / 1e9 if alg else None

            def cv(src, c):
                if li >= len(src) or k not in src[li] or c not in src[li][k]:
                    return None
                return statistics.median(src[li][k][c])
            fk, wk = cv(fetch, "FETCH_SIZE"), cv(write, "WRITE_SIZE")
            counted = (fk * fs + wk * ws) if (fk is not None and wk is not None and fs and ws) else None
            mu, vb, mi, vi = cv(sq, "MfmaUtil"), cv(sq, "VALUBusy"), cv(sq, "SQ_INSTS_MFMA"), cv(sq, "SQ_INSTS_VALU")
            f = lambda x, fmt: (fmt % x) if x is not None else "-"
            rows.append((sum(ds), "| `%s` | %s | %d | %.2f | %.2f | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
                short(k), role or "-", len(ds), med, p90, f(alg / 1e6 if alg else None, "%.1f"), f(gbs, "%.0f"),
                f(gbs / PEAK_GBS if gbs else None, "%.3f"), f(counted / 1e6 if counted else None, "%.1f"),
                f(counted / alg if (counted and alg) else None, "%.3f"), f(mu, "%.2f"), f(vb, "%.2f"),
                f(mi, "%.0f"), f(vi, "%.0f"))))
        for _, line in sorted(rows, key=lambda x: -x[0]):
            lines.append(line)
        lines.append("")
        lines.append(f"{len(leg)} dispatches, {total / 1e3:.2f} ms of kernel time.")
        lines.append("")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--sq")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--legs", default="leg0,leg1,leg2,leg3,leg4,leg5,leg6,leg7")
    ap.add_argument("--kv-rows", default="2048", help="live window rows per leg (comma list) for the attention's bytes")
    ap.add_argument("--out")
    ap.add_argument("--lm-json", help="write the verify-row lm_head's counted traffic here (JSON)")
    ap.add_argument("--kernel-source", help="source file whose SHA-256 goes with the traffic JSON")
    args = ap.parse_args()
    text = summarize(args)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    print(text)
    if args.lm_json:
        import hashlib
        import json
        t = lm_head_traffic(args)
        if t and args.kernel_source:
            t["kernel_source_sha256"] = hashlib.sha256(open(args.kernel_source, "rb").read()).hexdigest()
        with open(args.lm_json, "w") as f:
            json.dump(t, f, indent=1)


if __name__ == "__main__":
    main()
