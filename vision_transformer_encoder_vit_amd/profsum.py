"""Summaries of rocprofv3 CSV output as markdown tables (measurement tooling).

  python -m vision_transformer_encoder_vit_amd.profsum stats DIR
      kernel statistics (calls, mean/min/max duration, share of GPU time)
      from every *kernel_stats.csv under DIR
  python -m vision_transformer_encoder_vit_amd.profsum counters DIR [DIR ...]
      per kernel: the mean of each hardware counter over its dispatches
      (from every *counter_collection.csv under the DIRs), the mean dispatch
      duration (from *kernel_trace.csv in the same DIRs) and the derived
      rates below

Derived rates (MI355X: 256 CUs = 1024 SIMDs in 8 XCDs):
  MFMA busy      sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024)
  bf16 MFMA FLOP SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
  clock MHz      GRBM_GUI_ACTIVE per XCD / dispatch duration in us
  VALU busy      sum SQ_ACTIVE_INST_VALU x 4 / (GRBM_GUI_ACTIVE per XCD x 256)
                 (the SQ counts VALU issue in quad-cycles per CU)
  LDS busy       sum SQ_LDS_IDX_ACTIVE x 4 / (GRBM_GUI_ACTIVE per XCD x 256)
GRBM_GUI_ACTIVE is reported summed over the XCDs; it is divided by 8.
"""
import csv
import glob
import os
import sys
from collections import defaultdict

N_XCD, N_CU, N_SIMD = 8, 256, 1024


def _rows(dirs, suffix):
    out = []
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
            with open(f, newline="") as fh:
                out.extend(csv.DictReader(fh))
    return out


def short(name, n=70):
    name = name.replace("void ", "")
    return name if len(name) <= n else name[:n]


def stats(d):
    rows = _rows([d], "kernel_stats.csv")
    print("| kernel | calls | avg us | min us | max us | total % |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            short(r["Name"], 110), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))


def counters(dirs):
    vals = defaultdict(lambda: defaultdict(list))  # kernel -> counter -> per-dispatch values
    per_dispatch = defaultdict(lambda: defaultdict(float))
    for r in _rows(dirs, "counter_collection.csv"):
        key = (r.get("Dispatch_Id"), r["Kernel_Name"], r.get("Process_Id"))
        per_dispatch[key][r["Counter_Name"]] += float(r["Counter_Value"])
    for (_, k, _), cs in per_dispatch.items():
        for c, v in cs.items():
            vals[k][c].append(v)
    dur = defaultdict(list)
    for r in _rows(dirs, "kernel_trace.csv"):
        dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    names = sorted(vals, key=lambda k: -(sum(dur[k]) / len(dur[k]) if dur[k] else 0))
    cols = sorted({c for k in names for c in vals[k]})
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    print("| kernel | dispatches | mean us | " + " | ".join(cols) + " |")
    print("|---|---:|---:|" + "---:|" * len(cols))
    for k in names:
        print("| `%s` | %d | %.2f | %s |" % (short(k), max(len(v) for v in vals[k].values()), mean(dur[k]),
                                            " | ".join("%.4g" % mean(vals[k][c]) if c in vals[k] else ""
                                                       for c in cols)))
    print()
    print("| kernel | mean us | clock MHz | MFMA busy | bf16 MFMA TFLOP/s | VALU busy | LDS busy |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for k in names:
        v = {c: mean(x) for c, x in vals[k].items()}
        us = mean(dur[k])
        gui = v.get("GRBM_GUI_ACTIVE", float("nan")) / N_XCD
        f = lambda x: "%.3f" % x if x == x else "-"
        mfma = v.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (gui * N_SIMD)
        tf = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", float("nan")) * 512 / (us * 1e-6) / 1e12
        valu = v.get("SQ_ACTIVE_INST_VALU", float("nan")) * 4 / (gui * N_CU)
        lds = v.get("SQ_LDS_IDX_ACTIVE", float("nan")) * 4 / (gui * N_CU)
        print("| `%s` | %.2f | %s | %s | %s | %s | %s |" % (short(k), us, "%.0f" % (gui / us) if gui == gui else "-",
                                                         f(mfma), "%.0f" % tf if tf == tf else "-", f(valu), f(lds)))


if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in ("stats", "counters"):
        print(__doc__)
        sys.exit(2)
    if sys.argv[1] == "stats":
        stats(sys.argv[2])
    else:
        counters(sys.argv[2:])
