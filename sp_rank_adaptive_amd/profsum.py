"""Text summaries of rocprofv3 CSV output (``--output-format csv``).

    python -m sp_rank_adaptive_amd.profsum stats DIR OUT.md --cmd "..."
        per-kernel call count and durations from ``*_kernel_stats.csv``
    python -m sp_rank_adaptive_amd.profsum traffic FETCH_DIR WRITE_DIR OUT.json OUT.md --cmd "..."
        HBM bytes per GEMM launch from a FETCH_SIZE run and a WRITE_SIZE run of
        ``bench.py --copy-calibration``, each counter scaled by what it reads
        for the plain copy of known size that run ends with
    python -m sp_rank_adaptive_amd.profsum counters DIR OUT.md --cmd "..."
        MFMA busy fraction, bf16/fp16 MFMA flops, LDS bank-conflict rate and
        VALU instructions per wave per GEMM launch from an SQ/GRBM counter run

    traffic and counters take --kernel SUBSTR --label NAME to summarise
    every dispatch whose kernel name holds SUBSTR instead of the bench
    step's GEMMs; traffic then needs --algo-bytes N (algorithmic bytes per
    launch) and --source FILE (the csrc file whose hash is recorded).

In a ``bench.py`` step the GEMM launches come in the order fo_ag_gemm,
fo_gemm_rs; the summaries name them by that order.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(HERE, "csrc", "fo_gemm.hip")
LAUNCHES = ("ag_gemm", "gemm_rs")
COPY_BYTES = 1 << 29          # bench.py's calibration copy: 512 MiB read + 512 MiB written
# algorithmic bytes of one launch of each GEMM on the TP=8 MLP share:
# X and W read once (bf16), Y written once (fp32)
ALGO_BYTES = {
    "ag_gemm": 4096 * 4096 * 2 + 1792 * 4096 * 2 + 4096 * 1792 * 4,
    "gemm_rs": 4096 * 1792 * 2 + 4096 * 1792 * 2 + 4096 * 4096 * 4,
}


def _one(dirpath, suffix):
    hits = sorted(glob.glob(os.path.join(dirpath, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {dirpath}")
    return hits[0]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def source_hash(path=GEMM_SRC):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _per_dispatch(rows):
    """[(kernel name, {counter: summed value, "_ns": duration})] in dispatch order."""
    out = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        name, vals = out.setdefault(d, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        vals["_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return [out[d] for d in sorted(out)]


def _gemm_launches(disp, select=None):
    """Counter dicts of the profiled dispatches, grouped by launch name: by
    default the GEMM dispatches of bench steps (fo_ag_gemm, fo_gemm_rs in
    turn); with select = (kernel-name substring, label), every dispatch whose
    name holds the substring, under that label."""
    if select is not None:
        sub, label = select
        hits = [(n, v) for n, v in disp if sub in n]
        names = list(dict.fromkeys(n for n, _ in hits))
        if len(names) <= 1:
            return {label: [v for _, v in hits]}, {label: hits[0][0] if hits else None}
        # several kernels hold the substring: one launch per kernel, in the
        # order they first ran, labelled label_1, label_2, ...
        res = {f"{label}_{j + 1}": [v for n, v in hits if n == nm] for j, nm in enumerate(names)}
        return res, {f"{label}_{j + 1}": nm for j, nm in enumerate(names)}
    g = [v for n, v in disp if "gemm_kernel" in n]
    names = [n for n, _ in disp if "gemm_kernel" in n]
    res = {k: [] for k in LAUNCHES}
    kern = {}
    for i, v in enumerate(g):
        k = LAUNCHES[i % 2]
        res[k].append(v)
        kern[k] = names[i]
    return res, kern


def cmd_stats(d, out_md, cmd):
    rows = _rows(_one(d, "_kernel_stats.csv"))
    med = {}
    hits = sorted(glob.glob(os.path.join(d, "**", "*_kernel_trace.csv"), recursive=True))
    if hits:
        per = {}
        for r in _rows(hits[0]):
            per.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        med = {k: statistics.median(v) for k, v in per.items()}
    lines = ["# Kernel durations (rocprofv3 --kernel-trace --stats)", "", "Command:", "",
             "```", cmd, "```", "",
             "| kernel | calls | average us | median us | min us | max us | share % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        m = med.get(r["Name"])
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{(m / 1e3) if m is not None else float('nan'):.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    _write(out_md, "\n".join(lines) + "\n")


def cmd_traffic(fetch_dir, write_dir, out_json, out_md, cmd, select=None, algo=None, src=GEMM_SRC):
    res = {}
    scale = {}
    for key, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = _per_dispatch(_rows(_one(d, "_counter_collection.csv")))
        copies = [v[key] for n, v in disp if "copyBuffer" in n or "copy" in n.lower() and "gemm" not in n]
        if not copies:
            raise SystemExit(f"{key}: no calibration copy in {d}")
        kib = statistics.median(copies)
        scale[key] = COPY_BYTES / (kib * 1024.0)
        launches, kern = _gemm_launches(disp, select)
        for k, vals in launches.items():
            res.setdefault(k, {"kernel": kern.get(k)})
            res[k][key + "_KiB_median"] = statistics.median(v[key] for v in vals)
            res[k]["dispatches"] = len(vals)
    algo_bytes = dict(ALGO_BYTES)
    if select is not None:
        algo_bytes[select[1]] = algo
    out = {"kernel_source": os.path.basename(src), "kernel_source_sha256_16": source_hash(src), "copy_bytes": COPY_BYTES,
           "scale": {k: round(v, 5) for k, v in scale.items()}, "launches": {}}
    for k, r in res.items():
        fb = r["FETCH_SIZE_KiB_median"] * 1024 * scale["FETCH_SIZE"]
        wb = r["WRITE_SIZE_KiB_median"] * 1024 * scale["WRITE_SIZE"]
        out["launches"][k] = {"kernel": r["kernel"], "dispatches": r["dispatches"],
                              "fetch_bytes": int(fb), "write_bytes": int(wb),
                              "bytes_per_launch": int(fb + wb),
                              "algorithmic_bytes": algo_bytes[k],
                              "over_algorithmic": round((fb + wb) / algo_bytes[k], 3)}
    out["command"] = cmd
    _write(out_json, json.dumps(out, indent=1) + "\n")
    lines = ["# HBM traffic per launch (FETCH_SIZE, WRITE_SIZE)", "", "Command:", "",
             "```", cmd, "```", "",
             f"Calibration: a {COPY_BYTES >> 20} MiB device copy reads as "
             f"{COPY_BYTES / scale['FETCH_SIZE'] / 1024:.0f} KiB FETCH_SIZE and "
             f"{COPY_BYTES / scale['WRITE_SIZE'] / 1024:.0f} KiB WRITE_SIZE, so the counters are "
             f"scaled by {scale['FETCH_SIZE']:.4f} and {scale['WRITE_SIZE']:.4f}.", "",
             f"{out['kernel_source']} sha256[:16] = `{out['kernel_source_sha256_16']}`", "",
             "| launch | kernel | fetch MiB | write MiB | total MiB | algorithmic MiB | ratio |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for k, r in out["launches"].items():
        lines.append(f"| {k} | `{r['kernel']}` | {r['fetch_bytes'] / 2**20:.1f} | "
                     f"{r['write_bytes'] / 2**20:.1f} | {r['bytes_per_launch'] / 2**20:.1f} | "
                     f"{r['algorithmic_bytes'] / 2**20:.1f} | {r['over_algorithmic']:.2f} |")
    _write(out_md, "\n".join(lines) + "\n")


def cmd_counters(d, out_md, cmd, simds=1024, clock_hz=2.4e9, select=None):
    disp = _per_dispatch(_rows(_one(d, "_counter_collection.csv")))
    launches, kern = _gemm_launches(disp, select)
    lines = ["# MFMA and LDS counters (MFMA busy, bf16/fp16 MFMA flops, LDS bank conflicts, VALU)", "", "Command:", "",
             "```", cmd, "```", "",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x 2.4 GHz x dispatch duration in "
             "this counter run); bf16 flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; LDS conflict = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.  Each 16x16x32 bf16 MFMA counts 16 busy "
             "cycles, so the busy fraction equals the fraction of dense bf16 peak reached during "
             "the dispatch.", "",
             "| launch | kernel | dispatch us | MFMA busy % | bf16 GFLOP | fp16 GFLOP | LDS conflict % | "
             "VALU instr / wave | dispatches |",
             "|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for k, vals in launches.items():
        if not vals:
            continue
        med = lambda f: statistics.median(f(v) for v in vals)
        dur = med(lambda v: v["_ns"])
        busy = med(lambda v: v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (simds * clock_hz * v["_ns"] * 1e-9))
        fl = med(lambda v: v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) * 512 / 1e9)
        fl16 = med(lambda v: v.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0) * 512 / 1e9)
        conf = med(lambda v: v.get("SQ_LDS_BANK_CONFLICT", 0) / max(v.get("SQ_LDS_IDX_ACTIVE", 1), 1))
        valu = med(lambda v: v.get("SQ_INSTS_VALU", 0) / max(v.get("SQ_WAVES", 1), 1))
        lines.append(f"| {k} | `{kern[k]}` | {dur / 1e3:.1f} | {100 * busy:.1f} | {fl:.2f} | {fl16:.2f} | "
                     f"{100 * conf:.2f} | {valu:.0f} | {len(vals)} |")
    _write(out_md, "\n".join(lines) + "\n")


def _write(path, text):
    with open(path, "w") as f:
        f.write(text)
    print(f"wrote {path}")


def _opt(argv, name):
    if name in argv:
        i = argv.index(name)
        return argv[i + 1], argv[:i] + argv[i + 2:]
    return None, argv


def main(argv):
    cmd, argv = _opt(argv, "--cmd")
    kernel, argv = _opt(argv, "--kernel")
    label, argv = _opt(argv, "--label")
    algo, argv = _opt(argv, "--algo-bytes")
    src, argv = _opt(argv, "--source")
    cmd = cmd or ""
    select = (kernel, label or kernel) if kernel else None
    if not argv:
        raise SystemExit(__doc__)
    if argv[0] == "stats" and len(argv) == 3:
        cmd_stats(argv[1], argv[2], cmd)
    elif argv[0] == "traffic" and len(argv) == 5:
        cmd_traffic(argv[1], argv[2], argv[3], argv[4], cmd, select, int(algo) if algo else None,
                    os.path.join(HERE, "csrc", src) if src else GEMM_SRC)
    elif argv[0] == "counters" and len(argv) == 3:
        cmd_counters(argv[1], argv[2], cmd, select=select)
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
