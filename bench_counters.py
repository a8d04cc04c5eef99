"""Hardware-counter summaries of bench.py's kernels (rocprofv3 --pmc).

Three counter passes over one bench.py step of a workload, each within the
per-block limits of one rocprofv3 run (at most 8 SQ, 4 TCC, 2 TA, 2 TD and
2 GRBM counters):

  sq:   SQ_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES
        SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_LDS_IDX_ACTIVE
        GRBM_GUI_ACTIVE
  wait: SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VMEM
        SQ_INSTS_VALU_MFMA_MOPS_BF16 TA_TA_BUSY_sum TD_TD_BUSY_sum GRBM_GUI_ACTIVE
  l2:   TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE

On a machine with the GPU, from the repo root (OUT is any output folder, W the workload):
  rocprofv3 --pmc <sq counters>   --output-format csv -d OUT/counters/W/sq   -o c -- python bench.py --workload W --steps 1 --warmup 1 --no-cpu-baseline --no-breakdown --no-next --no-configs
  rocprofv3 --pmc <wait counters> --output-format csv -d OUT/counters/W/wait -o c -- python bench.py (same arguments)
  rocprofv3 --pmc <l2 counters>   --output-format csv -d OUT/counters/W/l2   -o c -- python bench.py (same arguments)
  rocprofv3 --kernel-trace --stats --output-format csv -d OUT/counters/W/trace -o c -- python bench.py (same arguments)
Then, anywhere:
  python bench_counters.py --summarize OUT/counters/W --workload W

which writes profiles/counters_W.md. Derived figures, per dispatch of a kernel,
averaged over its dispatches:
  * MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES): the
    fraction of SIMD cycles the matrix cores work, while the CUs are busy;
  * MFMA/VALU co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES;
  * VALU and LDS activity = SQ_ACTIVE_INST_VALU, SQ_LDS_IDX_ACTIVE per CU-cycle;
  * waits = SQ_WAIT_ANY (on s_waitcnt), SQ_WAIT_INST_ANY (for an instruction to
    issue) per wave-cycle (SQ_WAVE_CYCLES);
  * TA / TD busy per CU-cycle (texture address / data units, the vector-memory
    path); L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS);
  * clock = GRBM_GUI_ACTIVE / 8 XCDs / the kernel's average duration from the
    kernel-trace pass (meaningless for kernels of a few microseconds, whose
    GRBM count includes the dispatch around them).
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))

# Substrings of the mangled kernel names that identify the kernels of interest.
KERNELS = {
    "ctx_proj": "AStacked", "ctx_kv": "EpCtxKV", "qkv": "BQKV", "gate_up": "EpSwiGLU",
    "o_proj/down": "EpResidual", "attention (main)": "block_attn_kernelIDF16bLi128ELi64ELb0",
    "attention (redo)": "block_attn_kernelIDF16bLi128ELi64ELb1", "attn_combine": "attn_combine_kernel",
}


def _rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter csv under {d}")
    for f in files:
        yield from csv.DictReader(open(f))


def _per_kernel(d):
    """{kernel: {counter: mean per dispatch}} for one pass."""
    acc = {}
    for r in _rows(d):
        for k, key in KERNELS.items():
            if key in r["Kernel_Name"]:
                disp = acc.setdefault(k, {}).setdefault(r["Counter_Name"], {})
                disp[r["Dispatch_Id"]] = disp.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def _durations(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    out = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            for k, key in KERNELS.items():
                if key in r["Name"]:
                    out[k] = float(r["AverageNs"]) / 1e3
    return out


def summarize(root, workload):
    sq, wait, l2 = (_per_kernel(os.path.join(root, p)) for p in ("sq", "wait", "l2"))
    dur = _durations(os.path.join(root, "trace")) if os.path.isdir(os.path.join(root, "trace")) else {}
    lines = [f"# Hardware counters: {workload}", "",
             "Made by `bench_counters.py` (its docstring lists the four rocprofv3 commands: three "
             f"`--pmc` passes and one `--kernel-trace --stats` pass of `python bench.py --workload {workload} "
             "--steps 1 --warmup 1 --no-cpu-baseline --no-breakdown --no-next --no-configs`), then "
             f"`python bench_counters.py --summarize OUT/counters/{workload} --workload {workload}`.", "",
             "Per dispatch, averaged over the kernel's dispatches in the run. MFMA busy is per SIMD-cycle "
             "while the CUs are busy; VALU, LDS, TA and TD activity per CU-cycle; waits per wave-cycle.", "",
             "| kernel | avg us | clock GHz | MFMA busy | MFMA+VALU co-issue | VALU active | LDS active | "
             "wait s_waitcnt | wait issue | TA busy | TD busy | L2 hit |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in KERNELS:
        if k not in sq:
            continue
        s, w, c = sq[k], wait.get(k, {}), l2.get(k, {})
        cu = s.get("SQ_BUSY_CU_CYCLES", 0.0) or 1.0
        wave = s.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        mf = s.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        pct = lambda x: f"{100.0 * x:.1f}%"
        us = dur.get(k)
        clk = (s.get("GRBM_GUI_ACTIVE", 0.0) / 8.0 / (us * 1e-6) / 1e9) if us else None
        hit = c.get("TCC_HIT_sum")
        miss = c.get("TCC_MISS_sum")
        l2h = pct(hit / (hit + miss)) if hit is not None and miss is not None and hit + miss > 0 else "-"
        wcu = w.get("SQ_BUSY_CU_CYCLES", cu) or cu
        cells = [k, f"{us:.1f}" if us else "-", f"{clk:.2f}" if clk else "-",
                 pct(mf / (4.0 * cu)),
                 pct(s.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / mf) if mf else "-",
                 pct(s.get("SQ_ACTIVE_INST_VALU", 0.0) / cu),
                 pct(s.get("SQ_LDS_IDX_ACTIVE", 0.0) / cu),
                 pct(w.get("SQ_WAIT_ANY", 0.0) / wave),
                 pct(w.get("SQ_WAIT_INST_ANY", 0.0) / wave),
                 pct(w.get("TA_TA_BUSY_sum", 0.0) / wcu),
                 pct(w.get("TD_TD_BUSY_sum", 0.0) / wcu),
                 l2h]
        lines.append("| " + " | ".join(cells) + " |")
    lines += ["", "Raw means per dispatch:", ""]
    for k in KERNELS:
        if k not in sq:
            continue
        allc = {**sq.get(k, {}), **wait.get(k, {}), **l2.get(k, {})}
        lines.append(f"- **{k}**: " + ", ".join(f"{c} {v:.4g}" for c, v in sorted(allc.items())))
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize", required=True)
    ap.add_argument("--workload", default="c3")
    a = ap.parse_args()
    summarize(a.summarize, a.workload)


if __name__ == "__main__":
    sys.exit(main())
