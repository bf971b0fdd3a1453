"""Summaries of rocprofv3 output for the frame-step kernels.

    python -m rq_transformer_frame_amd.profsum stats <kernel_stats.csv> [bench.json]
    python -m rq_transformer_frame_amd.profsum traffic <fetch counter_collection.csv> <write ...csv> <copy MiB>
    python -m rq_transformer_frame_amd.profsum steps <kernel_trace.csv> <marker kernel> <steps>
    python -m rq_transformer_frame_amd.profsum counters <counter_collection.csv> [marker kernel]

`stats` prints a markdown table of the per-kernel averages (stage names recovered from the kernels'
stage tags; algorithmic GB/s when the bench JSON line of the same run is given).  `traffic` prints
per-kernel HBM bytes per dispatch from a FETCH_SIZE run and a WRITE_SIZE run, each scaled by what
the same counter reads for the first device-to-device copy of `copy MiB` in that run.  `steps`
keeps the dispatches after the last one whose name contains `marker` (e.g. the end of a prefill)
and prints per-stage averages and microseconds per step over `steps` steps.  `counters` prints, per
stage, the mean of every counter of a --pmc run per dispatch (after the last `marker` dispatch when
given) and, where the run holds them, the matrix-core figures: SQ_INSTS_VALU_MFMA_MOPS_BF16 (and _F32)
x 512 flops per dispatch over the dispatch's duration, and the matrix-core busy fraction
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDS x SIMDS): the busy counter sums the cycles of
every SIMD, and GRBM_GUI_ACTIVE sums the active cycles of every XCD (MI355X: 8 XCDs, 256 CUs of 4
SIMDs).
"""
from __future__ import annotations

import collections
import csv
import json
import re
import sys

XCDS, SIMDS = 8, 256 * 4  # MI355X

STAGES = ["embed", "qkv", "attn", "out_proj", "gate_in", "gate_out", "text_head", "dep_in", "dep_qkv",
          "dep_out", "dep_gate_in", "dep_gate_out", "dep_head", "frame_end"]


def stage_of(name: str) -> str:
    """The frame stage a kernel symbol belongs to (from its stage tag template argument)."""
    for key, stage in (("k_qkv_rope", "qkv"), ("k_attn", "attn"), ("k_dep_qkv", "dep_qkv"),
                       ("k_dep_out", "dep_out"), ("k_embed_begin", "embed"), ("k_frame_end", "frame_end"),
                       ("k_frame_persistent", "whole frame (persistent kernel)"),
                       ("k_gemm_reduce", "split-K reduction")):
        if key in name:
            return stage
    # k_gemm_x<weight type, add, stage, activation tiles>: the stage is the third argument
    m = re.search(r"mk::k_gemm_x<[^,>]+,\s*(?:true|false),\s*(\d+),\s*\d+>", name) or \
        re.search(r"mk::k_(?:gemv|gate|head|gemm)<[^>]*?,\s*(\d+)>", name)
    if m and int(m.group(1)) < len(STAGES):
        return STAGES[int(m.group(1))]
    return name.split("(")[0]


def stats(path: str, bench: str | None = None) -> str:
    rows = list(csv.DictReader(open(path)))
    per_stage = {}
    if bench:
        line = json.loads(open(bench).read().strip().splitlines()[-1])
        per_stage = {k: v.get("bytes_per_launch") for k, v in line.get("stages", {}).items()}
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    out = ["| stage (kernel) | calls | avg us | min us | share | algorithmic GB/s (avg) |",
           "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        st = stage_of(r["Name"])
        avg = float(r["AverageNs"]) / 1e3
        b = per_stage.get(st)
        gbs = f"{b / avg / 1e3:.0f}" if b else ""
        out.append(f"| {st} | {r['Calls']} | {avg:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{100 * float(r['TotalDurationNs']) / tot:.1f}% | {gbs} |")
    return "\n".join(out)


def traffic(fetch: str, write: str, copy_mib: float, after: str | None = None) -> str:
    """Per-kernel HBM bytes per dispatch from a FETCH_SIZE and a WRITE_SIZE run, scaled by the
    readings of the first device-to-device copy (copy_mib MiB).  With `after`, only the dispatches
    that follow the last dispatch whose kernel name contains it count (the copy still scales)."""
    def load(p):
        rows = sorted(csv.DictReader(open(p)), key=lambda r: int(r["Dispatch_Id"]))
        last = max((i for i, r in enumerate(rows) if after and after in r["Kernel_Name"]), default=-1)
        d = collections.defaultdict(list)
        first_copy = None
        for i, r in enumerate(rows):
            v = float(r["Counter_Value"])
            if first_copy is None and "copyBuffer" in r["Kernel_Name"]:
                first_copy = v
            if i > last:
                d[r["Kernel_Name"]].append(v)
        return d, first_copy

    f, fc = load(fetch)
    w, wc = load(write)
    kib = copy_mib * 1024.0
    ff, fw = kib / fc, kib / wc  # the copy reads and writes copy_mib MiB
    out = [f"Scale factors from the {copy_mib:g} MiB copy: FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {fw:.3f}.", "",
           "| stage (kernel) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per dispatch (scaled) |",
           "|---|---|---|---|---|"]
    for name in sorted(f, key=lambda n: -sum(f[n]) / len(f[n])):
        if "rocclr" in name:
            continue
        fv = sum(f[name]) / len(f[name])
        wv = sum(w.get(name, [0.0])) / max(len(w.get(name, [])), 1)
        out.append(f"| {stage_of(name)} | {len(f[name])} | {fv:.1f} | {wv:.1f} | "
                   f"{(fv * ff + wv * fw) * 1024:.0f} |")
    return "\n".join(out)


def steps(path: str, marker: str, nsteps: int) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = max((i for i, r in enumerate(rows) if marker in r["Kernel_Name"]), default=-1)
    agg = collections.defaultdict(lambda: [0, 0.0])
    for r in rows[last + 1:]:
        st = stage_of(r["Kernel_Name"])
        agg[st][0] += 1
        agg[st][1] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    tot = sum(v[1] for v in agg.values())
    out = [f"{len(rows) - last - 1} dispatches after the last `{marker}`, {tot / nsteps:.1f} us of kernel time per step.",
           "", "| stage (kernel) | dispatches | avg us | us per step | share |", "|---|---|---|---|---|"]
    for st, (n, t) in sorted(agg.items(), key=lambda x: -x[1][1]):
        out.append(f"| {st} | {n} | {t / n:.2f} | {t / nsteps:.1f} | {100 * t / tot:.1f}% |")
    return "\n".join(out)


def counters(path: str, after: str | None = None) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    last = max((int(r["Dispatch_Id"]) for r in rows if after and after in r["Kernel_Name"]), default=-1)
    # one row per (dispatch, counter)
    disp = collections.defaultdict(dict)
    meta = {}
    for r in rows:
        i = int(r["Dispatch_Id"])
        if i <= last or "rocclr" in r["Kernel_Name"]:
            continue
        disp[i][r["Counter_Name"]] = float(r["Counter_Value"])
        meta[i] = (stage_of(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3,
                   int(r["Grid_Size"]))
    names = sorted({c for d in disp.values() for c in d})
    agg = collections.defaultdict(list)
    for i, d in disp.items():
        agg[meta[i][0]].append((d, meta[i][1]))
    head = "| stage (kernel) | dispatches | avg us | " + " | ".join(names)
    mops = [c for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32") if c in names]
    bz = "SQ_VALU_MFMA_BUSY_CYCLES" in names and "GRBM_GUI_ACTIVE" in names
    for c in mops:
        head += f" | {c[-4:].lstrip('_').lower()} MFMA TFLOP/s (MOPS x 512 / duration)"
    if bz:
        head += " | MFMA busy"
    out = [head + " |", "|" + "---|" * (head.count("|") )]
    tot = lambda v, c: sum(d.get(c, 0.0) for d, _ in v)
    for st, v in sorted(agg.items(), key=lambda x: -sum(t for _, t in x[1])):
        us = sum(t for _, t in v) / len(v)
        cells = [f"{tot(v, c) / len(v):.4g}" for c in names]
        for c in mops:
            cells.append(f"{512.0 * tot(v, c) / (sum(t for _, t in v) * 1e6):.1f}")
        if bz:
            a = tot(v, "GRBM_GUI_ACTIVE")
            cells.append(f"{tot(v, 'SQ_VALU_MFMA_BUSY_CYCLES') / (a / XCDS * SIMDS):.3f}" if a else "")
        out.append(f"| {st} | {len(v)} | {us:.2f} | " + " | ".join(cells) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        print(stats(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else None))
    elif len(sys.argv) in (5, 6) and sys.argv[1] == "traffic":
        print(traffic(sys.argv[2], sys.argv[3], float(sys.argv[4]), sys.argv[5] if len(sys.argv) == 6 else None))
    elif len(sys.argv) in (3, 4) and sys.argv[1] == "counters":
        print(counters(sys.argv[2], sys.argv[3] if len(sys.argv) == 4 else None))
    elif len(sys.argv) == 5 and sys.argv[1] == "steps":
        print(steps(sys.argv[2], sys.argv[3], int(sys.argv[4])))
    else:
        print(__doc__)
        sys.exit(2)
