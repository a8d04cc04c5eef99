"""HBM traffic of bench.py's dominant kernel, from rocprofv3 counters.

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are collected in two separate
rocprofv3 --pmc runs of the bench command; each is scaled by the factor that
makes the same counter read the known byte count of a plain device-to-device
copy (1 GiB read + 1 GiB written, run with `python bench_traffic.py --copy`
under the same counter). The result is written to
profiles/traffic_<workload>_<kernel>.json together with a hash of the forward
kernels' sources, so bench.py reports it only while those kernels are
unchanged. A kernel made of several launches per call (attention: the main
pass and the redo pass) is counted per call: the bytes
of all its dispatches divided by the number of calls.

On a machine with the GPU, from the repo root (OUT is any output folder):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/traffic/fetch -o b -- python bench.py --workload c3 --steps 2 --warmup 1 --no-cpu-baseline --no-breakdown --no-next
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/traffic/write -o b -- python bench.py --workload c3 --steps 2 --warmup 1 --no-cpu-baseline --no-breakdown --no-next
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/traffic/copy_fetch -o c -- python bench_traffic.py --copy
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/traffic/copy_write -o c -- python bench_traffic.py --copy
Then, anywhere:
  python bench_traffic.py --summarize OUT/traffic --workload c3 --kernel ctx_proj
  python bench_traffic.py --summarize OUT/traffic --workload c4 --kernel attention
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30

# Substrings of the mangled kernel names that identify each dflash_kernel.
KERNEL_MATCH = {
    "ctx_proj": "AStacked", "ctx_kv": "EpCtxKV", "qkv": "BQKV", "gate_up": "EpSwiGLU",
    "attention": "block_attn_kernel", "attn_combine": "attn_combine_kernel", "rmsnorm": "rmsnorm_kernel",
}
# Launches per call of the library's kernel (every call makes all of them).
DISPATCHES_PER_CALL = {"attention": 2}


def _strip_comments(text: str) -> str:
    """The code without comments or whitespace: editing a comment or the layout
    leaves the hash unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "".join(text.split())


def source_hash() -> str:
    """Hash of the sources the measured forward kernels are built from, with
    comments and whitespace removed: the translation unit that instantiates them (dflash.hip),
    every header, and the public header. The other translation units (plan,
    verification, backward, profiling hook) cannot change these kernels' code."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_draft_model_build_amd", "csrc")
    files = [os.path.join(csrc, "dflash.hip")] + glob.glob(os.path.join(csrc, "*.h")) + \
        [os.path.join(ROOT, "include", "dflash.h")]
    for p in sorted(files):
        with open(p) as f:
            h.update(os.path.basename(p).encode())
            h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def copy_main():
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    a.fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def _per_dispatch(csv_dir, counter, match):
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter csv under {csv_dir}")
    vals = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
                continue
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for the kernel in {csv_dir}")
    return sum(vals.values()) / len(vals), len(vals)


def summarize(root, workload, kernel):
    key = KERNEL_MATCH[kernel]
    fetch, nf = _per_dispatch(os.path.join(root, "fetch"), "FETCH_SIZE", lambda n: key in n)
    write, nw = _per_dispatch(os.path.join(root, "write"), "WRITE_SIZE", lambda n: key in n)
    is_copy = lambda n: "copy" in n.lower() and "dflash" not in n
    cf, _ = _per_dispatch(os.path.join(root, "copy_fetch"), "FETCH_SIZE", is_copy)
    cw, _ = _per_dispatch(os.path.join(root, "copy_write"), "WRITE_SIZE", is_copy)
    f_fetch = COPY_BYTES / (cf * 1024.0)
    f_write = COPY_BYTES / (cw * 1024.0)
    per_call = DISPATCHES_PER_CALL.get(kernel, 1)
    out = {
        "workload": workload, "kernel": kernel,
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write, "dispatches": [nf, nw],
        "dispatches_per_call": per_call,
        "copy_factor_fetch": f_fetch, "copy_factor_write": f_write,
        "bytes_per_launch": per_call * (fetch * 1024.0 * f_fetch + write * 1024.0 * f_write),
        "source_hash": source_hash(),
        "command": "see bench_traffic.py docstring (FETCH_SIZE and WRITE_SIZE runs of bench.py --workload "
                   f"{workload} --steps 2 --warmup 1 --no-cpu-baseline --no-breakdown --no-next, plus the copy calibration)",
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{kernel}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def load(workload, kernel):
    """Traffic per launch in bytes for bench.py, or None when absent or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{kernel}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel or t.get("source_hash") != source_hash():
        return None
    return t["bytes_per_launch"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--copy", action="store_true")
    ap.add_argument("--summarize")
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--kernel", default="ctx_proj")
    a = ap.parse_args()
    if a.copy:
        copy_main()
    elif a.summarize:
        summarize(a.summarize, a.workload, a.kernel)
    else:
        ap.print_help()
        sys.exit(1)


if __name__ == "__main__":
    main()
