"""Summaries of rocprofv3 output for one benchmark step of the layer shard.

The benchmark's step issues its kernels in a fixed order (forward of the MLP and
attention sublayers, then their backward), so the dispatch sequence of a
rocprofv3 run of ``bench.py`` can be cut into steps and each dispatch assigned to
its hook step (``tpshard.STEPS``).  Two summaries are produced from the CSV files
rocprofv3 writes with ``--output-format csv``:

* kernel durations per step, from ``*_kernel_trace.csv`` (``--kernel-trace``);
* HBM traffic per step launch, from ``*_counter_collection.csv`` of one
  ``--pmc FETCH_SIZE`` run and one ``--pmc WRITE_SIZE`` run, each scaled by what
  the same counter reads for a plain device copy of known size
  (``bench.py --copy-calibration``).

The traffic table records a hash of the kernel sources; ``bench.py`` reports the
traffic of its dominant kernel only while that hash still matches.

Usage:
  python -m tensor_transformer_layer_02_amd.profiling traffic FETCH_DIR WRITE_DIR CFETCH_DIR CWRITE_DIR OUT
  python -m tensor_transformer_layer_02_amd.profiling durations TRACE_DIR OUT
  python -m tensor_transformer_layer_02_amd.profiling counters OUT PMC_DIR [PMC_DIR ...]
  python -m tensor_transformer_layer_02_amd.profiling stats TRACE_DIR OUT TITLE COMMAND NOTE
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

# (step, kernel-name patterns in the order the steps are enqueued, either
# stream); "gather*" is the forward's Q|K|V weight-staging copy where it makes one, "add*"
# any number of reduction launches (the second half of a
# K-split GEMM added into its outputs).
STEP_ORDER = [
    ("MLP_UP", ["gemm"]), ("MLP_DOWN", ["gemm"]), ("QKV", ["gather*", "gemm"]), ("ATTN_CORE", ["attn_fwd"]),
    ("ATTN_OUT", ["gemm"]), ("MLP_DU", ["gemm"]), ("MLP_DB1", ["colsum_partial", "colsum_final"]),
    ("MLP_DW", ["gemm", "add*"]), ("MLP_DX", ["gemm"]), ("ATTN_DO", ["gemm"]),
    ("ATTN_CORE_BWD", ["attn_rowdot*", "attn_bwd_dkdv", "attn_bwd_dq*"]),  # 16-bit: D from the dO GEMM, dK/dV + dQ one launch
    ("ATTN_DW", ["gemm", "add*"]), ("ATTN_DBIAS", ["colsum_partial", "colsum_final"]), ("ATTN_DX", ["gemm"]),
]
KEYS = {"gemm": ("gemm_bf16_kernel", "gemm_f32_kernel"), "attn_fwd": ("attn_fwd",), "add": ("add_f32_2d",),
        "gather": ("gather3",),
        "colsum_partial": ("colsum_partial",), "colsum_final": ("colsum_final",), "attn_rowdot": ("attn_rowdot",),
        "attn_bwd_dkdv": ("attn_bwd_dkdv",), "attn_bwd_dq": ("attn_bwd_dq",)}


def _code_only(text: str) -> str:
    """Source text without comments and blank space (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash() -> str:
    """sha256 over the kernel sources, comments and spacing ignored (any code change
    makes stored counters stale)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        if p.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(p).encode())
            with open(p, encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _is(name: str, key: str) -> bool:
    return any(k in name for k in KEYS[key])


def _ours(name: str) -> bool:
    return any(_is(name, k) for k in KEYS)


def split_steps(dispatches):
    """dispatches: [(name, record)] in dispatch order, library kernels only.
    Returns a list of steps, each {step_name: [records]}; incomplete tails are dropped."""
    steps, i, n = [], 0, len(dispatches)
    while i < n:
        cur, j, ok = {}, i, True
        for step, pats in STEP_ORDER:
            recs = []
            for pat in pats:
                if pat.endswith("*"):
                    while j < n and _is(dispatches[j][0], pat[:-1]):
                        recs.append(dispatches[j][1]); j += 1
                elif j < n and _is(dispatches[j][0], pat):
                    recs.append(dispatches[j][1]); j += 1
                else:
                    ok = False
                    break
            if not ok:
                break
            if step.endswith("+"):
                cur[step[:-1]] = cur.get(step[:-1], []) + recs
            else:
                cur[step] = recs
        if ok:
            steps.append(cur)
            i = j
        else:
            i += 1  # resynchronise on the next dispatch
    return steps


def _read(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _one(d, suffix):
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def counter_steps(d, counter):
    """Per-step lists of per-launch counter sums (KiB) from one --pmc run."""
    rows = _read(_one(d, "_counter_collection.csv"))
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        did = int(r["Dispatch_Id"])
        e = per.setdefault(did, [r["Kernel_Name"], 0.0])
        e[1] += float(r["Counter_Value"])
    seq = [(v[0], v[1]) for k, v in sorted(per.items()) if _ours(v[0])]
    return split_steps(seq)


def copy_factor(d, counter, nbytes=256 << 20):
    rows = _read(_one(d, "_counter_collection.csv"))
    vals = {}
    for r in rows:
        if "copy" in r["Kernel_Name"].lower() and r["Counter_Name"] == counter:
            vals[int(r["Dispatch_Id"])] = vals.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no copy kernel in {d}")
    kib = sum(vals.values()) / len(vals)
    return (nbytes / 1024.0) / kib


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, out):
    ff, fw = copy_factor(cfetch_dir, "FETCH_SIZE"), copy_factor(cwrite_dir, "WRITE_SIZE")
    fs, ws = counter_steps(fetch_dir, "FETCH_SIZE"), counter_steps(write_dir, "WRITE_SIZE")
    lines = [
        "# HBM traffic per step launch, layer shard gpt8b (8.3B shape, t = 8, shard 0), bf16 fwd+bwd",
        "# commands (from the repository root, on the GPU host):",
        "#   rocprofv3 --pmc FETCH_SIZE --kernel-trace -d F -o f --output-format csv -- "
        "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-others --no-kernel-timing",
        "#   rocprofv3 --pmc WRITE_SIZE --kernel-trace -d W -o w --output-format csv -- "
        "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-others --no-kernel-timing",
        "#   rocprofv3 --pmc FETCH_SIZE --kernel-trace -d CF -o f --output-format csv -- python3 bench.py --copy-calibration",
        "#   rocprofv3 --pmc WRITE_SIZE --kernel-trace -d CW -o w --output-format csv -- python3 bench.py --copy-calibration",
        "#   python -m tensor_transformer_layer_02_amd.profiling traffic F W CF CW <this file>",
        f"# copy calibration (256 MiB read + 256 MiB written): FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f}",
        f"# steps averaged: fetch {len(fs)}, write {len(ws)}; values are bytes per step launch (all its kernels)",
        f"source_sha256_16 {source_hash()}",
        "# step fetch_bytes write_bytes kernels",
    ]
    for step, _ in STEP_ORDER:
        if step.endswith("+"):
            continue
        fv = [sum(s[step]) for s in fs if step in s]
        wv = [sum(s[step]) for s in ws if step in s]
        nk = [len(s[step]) for s in fs if step in s]
        if not fv or not wv:
            continue
        fb = sum(fv) / len(fv) * 1024 * ff
        wb = sum(wv) / len(wv) * 1024 * fw
        lines.append(f"{step} {fb:.0f} {wb:.0f} {max(nk)}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def durations(trace_dir, out):
    rows = _read(_one(trace_dir, "_kernel_trace.csv"))
    seq = []
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        if _ours(r["Kernel_Name"]):
            seq.append((r["Kernel_Name"], (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))))
    steps = split_steps(seq)
    lines = [
        "# kernel durations per step, layer shard gpt8b (8.3B shape, t = 8, shard 0), bf16 fwd+bwd",
        "# command (from the repository root, on the GPU host):",
        "#   rocprofv3 --kernel-trace --stats -d T -o kt --output-format csv -- "
        "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-others",
        "#   python -m tensor_transformer_layer_02_amd.profiling durations T <this file>",
        f"# steps found in the trace: {len(steps)} (warm-up, timed and hooked passes)",
        f"source_sha256_16 {source_hash()}",
        "# step  avg_us_per_step_launch  kernels: avg_us each",
    ]
    tot = 0.0
    for step, _ in STEP_ORDER:
        if step.endswith("+"):
            continue
        per = [s[step] for s in steps if step in s]
        if not per:
            continue
        k = max(len(p) for p in per)
        avg = sum(sum(d for _, d in p) for p in per) / len(per) / 1e3
        tot += avg
        parts = []
        for i in range(k):
            ds = [p[i][1] for p in per if len(p) > i]
            nm = per[0][i][0] if len(per[0]) > i else "?"
            short = nm.replace("void ", "").replace("tp::(anonymous namespace)::", "").split("(")[0]
            parts.append(f"{short} {sum(ds) / len(ds) / 1e3:.2f}")
        lines.append(f"{step:<14} {avg:9.2f}   " + "; ".join(parts))
    lines.append(f"# sum of kernel time per step: {tot:.2f} us")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_traffic(path):
    """{step: (fetch_bytes, write_bytes)} and the recorded source hash, or ({}, None)."""
    if not os.path.exists(path):
        return {}, None
    tab, h = {}, None
    with open(path) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "source_sha256_16":
                h = t[1]
            elif len(t) >= 3:
                tab[t[0]] = (float(t[1]), float(t[2]))
    return tab, h


def counters(out, *dirs):
    """Per-step averages of every counter of one or more --pmc runs (one run per counter
    group), with the kernel time of the step in that run and, where a run holds
    SQ_VALU_MFMA_BUSY_CYCLES and SQ_BUSY_CU_CYCLES, the matrix-core utilisation
    MFMA-busy / (4 SIMDs x CU-busy cycles) of the busy CUs and cu_busy_GHz = CU-busy /
    (256 CUs x time), which is the clock times the fraction of CUs that are busy (lower than
    the clock where a launch leaves CUs idle).  GRBM_GUI_ACTIVE is listed raw: it counts the
    GPU-busy cycles of the whole counter window around a dispatch (summed over the XCDs), which
    is longer than the kernel, so it gives no clock per kernel."""
    lines = ["# hardware counters per step launch, layer shard gpt8b (8.3B shape, t = 8, shard 0), bf16 fwd+bwd",
             "# commands (from the repository root, on the GPU host), one per counter group:"]
    body = []
    for d in dirs:
        rows = _read(_one(d, "_counter_collection.csv"))
        per = {}
        for r in rows:
            e = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "us": (
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        names = sorted({k for e in per.values() for k in e if k not in ("name", "us")})
        lines.append(f"#   rocprofv3 --pmc {' '.join(names)} --kernel-trace -d DIR -o c --output-format csv "
                     "-- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-others --no-kernel-timing")
        steps = split_steps([(e["name"], e) for k, e in sorted(per.items()) if _ours(e["name"])])
        mf, cu = "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES"
        derived = mf in names and cu in names
        body.append("# step  kernel_us  " + ("mfma_util  cu_busy_GHz  " if derived else "") + "  ".join(names))
        for step, _ in STEP_ORDER:
            launches = [st[step] for st in steps if step in st]
            if not launches:
                continue
            avg = lambda f: sum(sum(f(r) for r in recs) for recs in launches) / len(launches)
            us = avg(lambda r: r["us"])
            vals = {n: avg(lambda r, n=n: r.get(n, 0.0)) for n in names}
            txt = f"{step:<14} {us:9.2f}  "
            if derived:
                txt += f"{vals[mf] / (4 * vals[cu]) if vals[cu] else 0.0:9.3f}  {vals[cu] / 256 / us / 1e3:9.2f}  "
            body.append(txt + "  ".join(f"{vals[n]:.4g}" for n in names))
        body.append("")
    lines.append("#   python -m tensor_transformer_layer_02_amd.profiling counters <this file> DIR [DIR ...]")
    lines.append(f"source_sha256_16 {source_hash()}")
    with open(out, "w") as f:
        f.write("\n".join(lines + body))


def _short(name: str) -> str:
    """Kernel name without namespaces and the parameter list's struct qualifiers."""
    for q in ("tp::(anonymous namespace)::", "tp::"):
        name = name.replace(q, "")
    return name[5:] if name.startswith("void ") else name


def stats(trace_dir, out, title, command, note):
    """Markdown table of rocprofv3's --stats kernel summary (every kernel of the run)."""
    rows = _read(_one(trace_dir, "_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel statistics: {title}", "", "Command (from the repository root, on one MI355X):",
             "", f"    {command}", "", note, "", f"source_sha256_16 {source_hash()}", "",
             "| calls | avg us | min us | max us | % time | kernel |", "|---:|---:|---:|---:|---:|---|"]
    for r in rows:
        lines.append(f"| {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} | `{_short(r['Name'])}` |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if len(sys.argv) == 7 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:7])
    elif len(sys.argv) == 4 and sys.argv[1] == "durations":
        durations(*sys.argv[2:4])
    elif len(sys.argv) >= 4 and sys.argv[1] == "counters":
        counters(sys.argv[2], *sys.argv[3:])
    elif len(sys.argv) == 7 and sys.argv[1] == "stats":
        stats(*sys.argv[2:7])
    else:
        raise SystemExit(__doc__)
