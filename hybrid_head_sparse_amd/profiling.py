"""rocprofv3 helpers for the attention kernel's roofline figures.

    # a plain copy of known size, profiled with the same counters, calibrates them
    python3 -m hybrid_head_sparse_amd.profiling copy [--mib 1024]

    # turn rocprofv3 CSV output into the committed summaries
    python3 -m hybrid_head_sparse_amd.profiling summarize --workload llama3_128k \\
        --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --commands FILE

`summarize` reads the kernel statistics of a `--kernel-trace --stats` run and
the per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of two `--pmc` runs of the same
benchmark, scales each counter by what it reads for the copy (bytes moved /
counter bytes), and writes profiles/attend_<workload>_kernel_stats.md,
profiles/attend_<workload>_counters.md and the JSON the benchmark reads.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")
ATTEND_SRC = os.path.join(HERE, "csrc", "attend.hip")
KERNEL_SOURCES = (ATTEND_SRC, os.path.join(HERE, "csrc", "common.hpp"))
HYBRID_KERNEL = "attend_kernel<lychee::(anonymous namespace)::BF16, 128, 4, true, false, false>"
DENSE_KERNEL = "attend_kernel<lychee::(anonymous namespace)::BF16, 128, 4, false, false, false>"


def kernel_code_digest(texts=None) -> str:
    """sha256 of the kernel's sources (attend.hip, common.hpp) with comments
    and runs of blank space removed: editing a comment leaves it unchanged,
    editing code changes it."""
    if texts is None:
        texts = [open(f).read() for f in KERNEL_SOURCES]
    h = hashlib.sha256()
    for src in texts:
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(re.sub(r"\s+", " ", src).strip().encode())
        h.update(b"\0")
    return h.hexdigest()


def run_copy(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    x = torch.arange(n, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    assert torch.equal(x[-16:], y[-16:])
    print(f"copied {mib} MiB three times", flush=True)


def _one_csv(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[-1]


def _counter_per_dispatch(d: str, counter: str, name_pred) -> list[float]:
    """Per-dispatch values (summed over the rows of a dispatch) of `counter`
    for kernels whose name satisfies name_pred."""
    per = {}
    with open(_one_csv(d, "counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter or not name_pred(row.get("Kernel_Name", "")):
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    return list(per.values())


def _kernel_stats(d: str) -> list[dict]:
    with open(_one_csv(d, "kernel_stats.csv")) as f:
        return list(csv.DictReader(f))


def write_stats(trace: str, wl: str, cmds: str) -> None:
    """profiles/attend_<wl>_kernel_stats.md from a --kernel-trace --stats run."""
    rows = []
    for r in _kernel_stats(trace):
        name = r.get("Name") or r.get("KERNEL_NAME") or ""
        if not any(k in name for k in ("attend_kernel", "rule", "correction", "merge")):
            continue
        rows.append((name, int(r["Calls"]), float(r["TotalDurationNs"]), float(r["AverageNs"]),
                     float(r["MinNs"]), float(r["MaxNs"])))
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"attend_{wl}_kernel_stats.md"), "w") as f:
        f.write(f"# rocprofv3 kernel statistics: attention kernels, {wl}\n\n")
        f.write("Commands (from the repository root on one MI355X):\n\n```\n" + cmds + "\n```\n\n")
        f.write("| kernel | calls | total ms | average us | min us | max us |\n|---|---|---|---|---|---|\n")
        for name, calls, tot, avg, mn, mx in rows:
            f.write(f"| `{name}` | {calls} | {tot / 1e6:.3f} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} |\n")
        f.write("\nThe hybrid kernel's token top-k build (`..., true, false, false>`) runs every layer of the step\n"
                "(layer 0 all retrieval, the others mixed) in the eager, graph and event-timed passes of the\n"
                "benchmark; the dense build (`..., false, false, false>`) is the all-retrieval comparison (the\n"
                "block and Top-p rules have builds of their own).  The hybrid average over a step's layers is\n"
                "what the benchmark reports as `roofline.avg_launch_us` (its step time over the layers).\n")


def summarize(a) -> None:
    is_copy = lambda name: ("copy" in name.lower() or "elementwise" in name.lower()) and "attend" not in name
    is_hyb = lambda name: HYBRID_KERNEL in name
    copy_bytes = 3 * a.copy_mib * (1 << 20)             # per direction, three copies
    cf = _counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", is_copy)
    cw = _counter_per_dispatch(a.copy_write, "WRITE_SIZE", is_copy)
    big = lambda v: sorted(v)[-3:]                          # the three 1 GiB copies
    f_scale = copy_bytes / (sum(big(cf)) * 1024.0)
    w_scale = copy_bytes / (sum(big(cw)) * 1024.0)
    fetch = _counter_per_dispatch(a.fetch, "FETCH_SIZE", is_hyb)
    write = _counter_per_dispatch(a.write, "WRITE_SIZE", is_hyb)
    fetch_b = statistics.mean(fetch) * 1024.0 * f_scale
    write_b = statistics.mean(write) * 1024.0 * w_scale
    cmds = open(a.commands).read().strip()
    sha = kernel_code_digest()
    wl = a.workload
    write_stats(a.trace, wl, cmds)
    res = {
        "workload": wl,
        "kernel": HYBRID_KERNEL,
        "kernel_code_sha256": sha,
        "dispatches": {"fetch": len(fetch), "write": len(write)},
        "fetch_kib_per_dispatch_raw": statistics.mean(fetch),
        "write_kib_per_dispatch_raw": statistics.mean(write),
        "copy_calibration": {"bytes_per_direction": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale},
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "traffic_bytes_per_launch": fetch_b + write_b,
    }
    with open(os.path.join(PROFILES, f"attend_{wl}_counters.json"), "w") as f:
        json.dump(res, f, indent=1)
    with open(os.path.join(PROFILES, f"attend_{wl}_counters.md"), "w") as f:
        f.write(f"# HBM traffic of the hybrid attention kernel, {wl}\n\n")
        f.write("Commands (from the repository root on one MI355X):\n\n```\n" + cmds + "\n```\n\n")
        f.write(f"- kernel: `{HYBRID_KERNEL}`, {len(fetch)} dispatches with FETCH_SIZE, {len(write)} with WRITE_SIZE\n")
        f.write(f"- raw mean per dispatch: FETCH_SIZE {res['fetch_kib_per_dispatch_raw']:.1f} KiB, "
                f"WRITE_SIZE {res['write_kib_per_dispatch_raw']:.1f} KiB\n")
        f.write(f"- copy calibration: 3 x {a.copy_mib} MiB copies read as {sum(big(cf)):.0f} KiB fetched and "
                f"{sum(big(cw)):.0f} KiB written -> scale {f_scale:.4f} (fetch), {w_scale:.4f} (write)\n")
        f.write(f"- traffic per launch: {fetch_b / 1e6:.2f} MB fetched + {write_b / 1e6:.2f} MB written = "
                f"{(fetch_b + write_b) / 1e6:.2f} MB\n")
        f.write(f"- kernel code digest at measurement (attend.hip + common.hpp, comments removed): `{sha}`\n")
    print(json.dumps(res, indent=1))


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    s = sub.add_parser("summarize")
    s.add_argument("--workload", default="llama3_128k")
    for k in ("trace", "fetch", "write", "copy_fetch", "copy_write", "commands"):
        s.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    t = sub.add_parser("stats")
    t.add_argument("--workload", required=True)
    t.add_argument("--trace", required=True)
    t.add_argument("--commands", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        run_copy(a.mib)
    elif a.cmd == "stats":
        write_stats(a.trace, a.workload, open(a.commands).read().strip())
    else:
        summarize(a)


if __name__ == "__main__":
    main(sys.argv[1:])
