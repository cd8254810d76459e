"""Summaries of rocprofv3 counter runs (the benchmark's HBM and stall figures).

    python -m long_context_sparse_idx_amd.counters hbm WORKLOAD FETCH_DB WRITE_DB
        -> adds this workload's entries to profiles/hbm_counters.json and
           writes profiles/<workload>_hbm_counters.md
    python -m long_context_sparse_idx_amd.counters table OUT_MD TITLE COMMAND DB [DB ...]
        -> per-kernel average of every counter in the runs, as a markdown table
    python -m long_context_sparse_idx_amd.counters trace OUT_MD TITLE COMMAND DB
        -> per-kernel calls, total and average duration of a --kernel-trace run
    python -m long_context_sparse_idx_amd.counters mfma OUT_MD TITLE COMMAND DB
        -> MFMA instructions, flops and busy cycles per kernel, with the clock
           and busy fraction they imply

Each database is the output of one ``rocprofv3 --pmc ... -- python3 bench.py
... --calibrate-copy`` run.  HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per
dispatch) are scaled by what they read for two dispatches of known size that
``--calibrate-copy`` runs first: a 1 GiB device copy (1 GiB read, 1 GiB
written) and a 1 GiB read-only reduction (1 GiB read).  An entry records the
SHA-256 of the kernel sources it was measured on; bench.py uses an entry only
while those sources are unchanged.
"""
from __future__ import annotations

import datetime
import hashlib
import json
import os
import re
import sqlite3
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROFILES = os.path.join(ROOT, "profiles")
HBM_JSON = os.path.join(PROFILES, "hbm_counters.json")
GIB_KIB = 1 << 20

# kernel name prefix -> the sources its code comes from
KERNEL_SOURCES = {
    "score_prefill_kernel": ("score.hip",),
    "score_splitkey_kernel": ("score.hip",),
    "select_": ("select.hip",),
    "attn_kernel": ("attn.hip",),
    "attn_merge_kernel": ("attn.hip",),
    "zero_i32_kernel": ("score.hip",),
}


def short_name(name: str) -> str:
    n = re.sub(r"\(lcsi::.*", "", name)
    n = n.replace("void lcsi::(anonymous namespace)::", "").replace("lcsi::(anonymous namespace)::", "")
    return n.strip()


def per_dispatch(db_path: str):
    """{kernel: {counter: [value per dispatch]}} from one rocpd database."""
    db = sqlite3.connect(db_path)
    out = defaultdict(lambda: defaultdict(list))
    for name, counter, value in db.execute(
            "select kernel_name, counter_name, value from counters_collection order by dispatch_id"):
        out[name][counter].append(float(value))
    return out


def _sha(src: str) -> str:
    with open(os.path.join(CSRC, src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _calibration(fetch, write):
    """Scale factors (bytes per KiB counted) from the 1 GiB copy and the
    1 GiB read-only reduction of --calibrate-copy."""
    copy = [k for k in fetch if "copyBuffer" in k]
    red = [k for k in fetch if "reduce_kernel" in k]
    if not copy:
        raise SystemExit("no copy dispatch in the FETCH_SIZE run (use bench.py --calibrate-copy)")
    copy_fetch = max(fetch[copy[0]]["FETCH_SIZE"])
    copy_write = max(write[copy[0]]["WRITE_SIZE"]) if copy[0] in write else None
    cal = {"copy_1GiB_FETCH_SIZE_KiB": copy_fetch, "copy_1GiB_WRITE_SIZE_KiB": copy_write,
           "fetch_factor": GIB_KIB / copy_fetch, "write_factor": GIB_KIB / copy_write if copy_write else 1.0}
    if red:
        red_fetch = max(max(fetch[k]["FETCH_SIZE"]) for k in red)
        cal["read_1GiB_FETCH_SIZE_KiB"] = red_fetch
        cal["read_fetch_factor"] = GIB_KIB / red_fetch
    return cal


def hbm(workload: str, fetch_db: str, write_db: str):
    fetch, write = per_dispatch(fetch_db), per_dispatch(write_db)
    cal = _calibration(fetch, write)
    ff, wf = cal["fetch_factor"], cal["write_factor"]
    entries = []
    for name in fetch:
        sn = short_name(name)
        srcs = next((v for k, v in KERNEL_SOURCES.items() if sn.startswith(k)), None)
        if srcs is None or name not in write:
            continue
        f = fetch[name]["FETCH_SIZE"]
        w = write[name]["WRITE_SIZE"]
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        entries.append({"workload": workload, "kernel": sn, "dispatches": len(f),
                        "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                        "bytes_per_launch": int(round((fk * ff + wk * wf) * 1024)),
                        "sources": {s: _sha(s) for s in srcs}})
    try:
        with open(HBM_JSON) as fh:
            doc = json.load(fh)
    except OSError:
        doc = {"entries": []}
    doc["entries"] = [e for e in doc.get("entries", []) if e["workload"] != workload] + entries
    doc.setdefault("calibration", {})[workload] = cal
    doc["note"] = ("HBM bytes per dispatch = FETCH_SIZE x fetch_factor + WRITE_SIZE x write_factor "
                   "(KiB -> bytes); factors from a 1 GiB copy run in the same process")
    with open(HBM_JSON, "w") as fh:
        json.dump(doc, fh, indent=1)
    md = os.path.join(PROFILES, f"{workload}_hbm_counters.md")
    with open(md, "w") as fh:
        fh.write(f"# HBM traffic counters: {workload} workload\n\n")
        fh.write("Commands (one counter per run, from the repository root):\n\n```\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            fh.write(f"rocprofv3 --pmc {c} -d gpurun_out/pmc_{c} -o pmc -- python3 bench.py --workload "
                     f"{workload} --steps 1 --warmup 0 --no-cpu --no-allf --no-ceilings --no-secondary "
                     f"--calibrate-copy\n")
        fh.write("```\n\n")
        fh.write(f"Calibration: the 1 GiB copy reads back as FETCH_SIZE = {cal['copy_1GiB_FETCH_SIZE_KiB']:.0f} KiB "
                 f"and WRITE_SIZE = {cal['copy_1GiB_WRITE_SIZE_KiB']:.0f} KiB")
        if "read_1GiB_FETCH_SIZE_KiB" in cal:
            fh.write(f"; the 1 GiB read-only reduction as FETCH_SIZE = {cal['read_1GiB_FETCH_SIZE_KiB']:.0f} KiB")
        fh.write(f" (1 GiB = {GIB_KIB} KiB).  Factors: FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {wf:.3f}.  "
                 f"Counts cover L2-to-memory traffic (Infinity Cache hits included).\n\n")
        fh.write("| kernel | dispatches | FETCH_SIZE KiB (avg) | WRITE_SIZE KiB (avg) | HBM bytes per dispatch |\n")
        fh.write("|---|---:|---:|---:|---:|\n")
        for e in sorted(entries, key=lambda e: -e["bytes_per_launch"]):
            fh.write(f"| `{e['kernel']}` | {e['dispatches']} | {e['fetch_kib']:.0f} | {e['write_kib']:.0f} | "
                     f"{e['bytes_per_launch'] / 1e9:.4f} GB |\n")
        fh.write(f"\nWritten by `python -m long_context_sparse_idx_amd.counters hbm` on "
                 f"{datetime.date.today().isoformat()}; sources: "
                 + ", ".join(sorted({s for e in entries for s in e['sources']})) + ".\n")
    print(f"wrote {len(entries)} entries for {workload} to {HBM_JSON} and {md}")


def table(out_md: str, title: str, command: str, dbs):
    rows = defaultdict(dict)
    for db in dbs:
        for name, cs in per_dispatch(db).items():
            sn = short_name(name)
            if not any(sn.startswith(k) for k in KERNEL_SOURCES):
                continue
            for c, v in cs.items():
                rows[sn][c] = sum(v) / len(v)
                rows[sn]["dispatches"] = len(v)
    counters = sorted({c for r in rows.values() for c in r if c != "dispatches"})
    with open(out_md, "w") as fh:
        fh.write(f"# {title}\n\nCommand(s), from the repository root:\n\n```\n{command}\n```\n\n")
        fh.write("Per-dispatch averages.\n\n| kernel | dispatches | " + " | ".join(counters) + " |\n")
        fh.write("|---|---:|" + "---:|" * len(counters) + "\n")
        for k in sorted(rows):
            fh.write(f"| `{k}` | {rows[k].get('dispatches', 0)} | "
                     + " | ".join(f"{rows[k][c]:.4g}" if c in rows[k] else "" for c in counters) + " |\n")
    print(f"wrote {out_md}")


def trace(out_md: str, title: str, command: str, db_path: str):
    db = sqlite3.connect(db_path)
    agg = defaultdict(list)
    for name, start, end in db.execute("select name, start, end from kernels"):
        agg[short_name(name)].append((end - start) / 1e6)
    with open(out_md, "w") as fh:
        fh.write(f"# {title}\n\nCommand, from the repository root:\n\n```\n{command}\n```\n\n")
        fh.write("| kernel | calls | total ms | avg ms |\n|---|---:|---:|---:|\n")
        other = [0, 0.0]
        for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            if any(k.startswith(p) for p in KERNEL_SOURCES) or "zero_i32" in k or "merge" in k:
                fh.write(f"| `{k}` | {len(v)} | {sum(v):.3f} | {sum(v) / len(v):.4f} |\n")
            else:
                other[0] += len(v)
                other[1] += sum(v)
        fh.write(f"| (other kernels: input generation and copies, outside the timed region) | {other[0]} | "
                 f"{other[1]:.1f} | |\n")
    print(f"wrote {out_md}")


def mfma(out_md: str, title: str, command: str, db_path: str, n_simd: int = 1024, n_xcd: int = 8):
    """One counter pass of SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_VALU_MFMA_BF16,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE: the SQ
    counters are summed over all SIMDs, GRBM_GUI_ACTIVE over the XCDs, MOPS
    count 512 flops each.  The clock is one XCD's active cycles over the
    dispatch's duration in the same run (kernels run slower under counter
    collection)."""
    pd = per_dispatch(db_path)
    db = sqlite3.connect(db_path)
    dur = defaultdict(list)
    try:
        for name, start, end in db.execute("select name, start, end from kernels"):
            dur[short_name(name)].append((end - start) / 1e6)
    except sqlite3.Error:
        pass
    mean = lambda v: sum(v) / len(v) if v else 0.0
    with open(out_md, "w") as fh:
        fh.write(f"# {title}\n\nCommand, from the repository root:\n\n```\n{command}\n```\n\n")
        fh.write(f"Per-dispatch averages over {n_simd} SIMDs and {n_xcd} XCDs.\n\n"
                 "| kernel | dispatches | avg ms | MFMA instructions | MFMA flops (MOPS x 512) | "
                 "MFMA busy cycles / SIMD | active cycles / XCD | clock (GHz) | MFMA busy |\n"
                 "|---|---:|---:|---:|---:|---:|---:|---:|---:|\n")
        for name, cs in sorted(pd.items(), key=lambda kv: -mean(dur.get(short_name(kv[0]), []))):
            sn = short_name(name)
            if not any(sn.startswith(k) for k in KERNEL_SOURCES):
                continue
            n = max(len(v) for v in cs.values())
            ms = mean(dur.get(sn, []))
            ins = mean(cs.get("SQ_INSTS_VALU_MFMA_BF16", []))
            flops = mean(cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])) * 512
            busy = mean(cs.get("SQ_VALU_MFMA_BUSY_CYCLES", [])) / n_simd
            act = mean(cs.get("GRBM_GUI_ACTIVE", [])) / n_xcd
            # (no clock for dispatches too short for their duration to mean much)
            clock = f"{act / (ms * 1e-3) / 1e9:.2f}" if ms >= 0.01 and act > 0 and busy > 0 else "--"
            frac = f"{100 * busy / act:.0f} %" if act > 0 and busy > 0 else ("0 %" if act > 0 else "--")
            fh.write(f"| `{sn}` | {n} | {ms:.3f} | {ins:.4g} | {flops:.4g} | {busy:.4g} | {act:.4g} | {clock} | {frac} |\n")
    print(f"wrote {out_md}")


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "hbm":
        hbm(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 6 and sys.argv[1] == "table":
        table(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    elif len(sys.argv) == 6 and sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif len(sys.argv) == 6 and sys.argv[1] == "mfma":
        mfma(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    else:
        print(__doc__)
        sys.exit(2)
