"""Where a layer's time goes: phase timestamps of the attention kernel.

    python -m hybrid_head_sparse_amd.build --trace
    LYCHEE_LIB=hybrid_head_sparse_amd/liblychee_trace.so \
        python3 -m hybrid_head_sparse_amd.timeline --workload llama3_128k \
        [--reps 3] [--out profiles/timeline_llama3_128k.md]

Runs the workload's decode step eagerly (every layer chained through S, the
inputs resident on the device) --reps times with the trace build of the
library, which stamps s_memrealtime (100 MHz) at each phase of each
workgroup.  For the last repetition it prints, per layer, times measured from
the layer's first workgroup entry:
  prologue    median workgroup time from entry to ranges ready
  first load  median time from entry to its first head's start
  stream      last workgroup done streaming / gathering
  sel-arrive  last selection arrival (retrieval heads: bound, candidate
              append and the arrival counted)
  record      last partial record complete
  merged      last merge done (the layer's outputs written)
  resolved    last top-k resolve done
  exit        last workgroup exit (= the kernel's span)
and the gap from the previous layer's last exit to this layer's first
entry.  The stamps perturb the kernel a little (one scalar stamp per phase
per workgroup); the spans agree with the untraced kernel's to a few percent.
"""
from __future__ import annotations

import argparse
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SLOTS = 32
(ENTRY, PROLOGUE, HEAD, STREAM, SELARR, RECORD, ARRIVE, MERGED, RSTART, REND, EXIT, FLAGS, HEADS) = range(13)
RES0 = 16               # resolver phase stamps: RES0 + 0..10
RES_PHASES = ("hist+words", "crossing", "recount", "staged+group", "cut", "offsets", "emitted", "padded",
              "staged", "compacted", "gathered")
PRO0 = 28               # prologue phase stamps: PRO0 + 0..3
SSTAGED = 27            # a sparse head's S entries staged
PRO_PHASES = ("contexts", "cost prefix", "boundaries", "loop entry")
TICK_US = 0.01          # s_memrealtime: 100 MHz


def analyse(tr, grid: int, layer_roles):
    """tr: uint64 array [launches, grid, SLOTS]; returns one dict per launch."""
    import numpy as np
    rows = []
    prev_exit = None
    for li in range(tr.shape[0]):
        t = tr[li].astype(np.int64)
        live = t[:, ENTRY] > 0
        t0 = int(t[live, ENTRY].min())

        def last(slot):
            v = t[live, slot]
            v = v[v > 0]
            return (int(v.max()) - t0) * TICK_US if v.size else float("nan")

        def med(slot):
            v = t[live, slot]
            ok = v > 0
            return statistics.median(((v[ok] - t[live, ENTRY][ok]) * TICK_US).tolist()) if ok.any() else float("nan")

        r = {"layer": li, "retrieval": int(layer_roles[li]), "wgs": int(live.sum()),
             "prologue": med(PROLOGUE), "first_load": med(HEAD), "stream": last(STREAM), "sel_arrive": last(SELARR),
             "record": last(RECORD), "merged": last(MERGED), "resolved": last(REND), "exit": last(EXIT),
             "gap": (t0 - prev_exit) * TICK_US if prev_exit is not None else float("nan")}
        prev_exit = int(t[live, EXIT].max())
        rows.append(r)
    return rows


def resolver_table(tr, kinds) -> str:
    """Median time (us from the resolver's start) at which each phase of the
    last-arrival candidate resolver ends, per layer kind; n = resolves seen."""
    import numpy as np
    lines = ["| retrieval heads | n | " + " | ".join(RES_PHASES) + " | full scans |",
             "|---|---|" + "---|" * len(RES_PHASES) + "---|"]
    for R in sorted(kinds):
        per = [[] for _ in RES_PHASES]
        n = fb = 0
        for r in kinds[R]:
            t = tr[r["layer"]].astype(np.int64)
            for wg in np.nonzero(t[:, RSTART] > 0)[0]:
                n += 1
                fb += int(t[wg, FLAGS]) >> 5 & 1
                for j in range(len(RES_PHASES)):
                    if t[wg, RES0 + j] > 0:
                        per[j].append((t[wg, RES0 + j] - t[wg, RSTART]) * TICK_US)
        if n:
            lines.append(f"| {R} | {n} | " + " | ".join(f"{statistics.median(v):.1f}" if v else "-" for v in per) +
                         f" | {fb} |")
    return "\n".join(lines) + "\n"


def report(tr, grid: int, roles, spans):
    import numpy as np
    rows = analyse(tr, grid, roles.sum(axis=1))
    cols = ["layer", "retrieval", "wgs", "gap", "prologue", "first_load", "stream", "sel_arrive", "record",
            "merged", "resolved", "exit"]
    lines = ["| " + " | ".join(cols) + " |", "|" + "---|" * len(cols)]
    for r in rows:
        lines.append("| " + " | ".join(f"{r[c]:.1f}" if isinstance(r[c], float) else str(r[c]) for c in cols) + " |")
    kinds = {}
    for r in rows[1:]:
        kinds.setdefault(r["retrieval"], []).append(r)
    summ = ["| retrieval heads | layers | mean gap | prologue | first load | stream | sel-arrive | record | "
            "merged | resolved | exit |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for R in sorted(kinds):
        rs = kinds[R]

        def mean(c):
            v = [x[c] for x in rs if x[c] == x[c]]
            return statistics.mean(v) if v else float("nan")
        summ.append(f"| {R} | {len(rs)} | " + " | ".join(f"{mean(c):.1f}" for c in
                    ("gap", "prologue", "first_load", "stream", "sel_arrive", "record", "merged", "resolved",
                     "exit")) + " |")
    # streaming end by workgroup kind (retrieval rows only, gathered rows only, both)
    kind_lines = ["| retrieval heads | WG kind | WGs | stream end median | stream end max |", "|---|---|---|---|---|"]
    for R in sorted(kinds):
        for fl, name in ((1, "retrieval rows"), (2, "gathered rows"), (3, "both")):
            ends = []
            for r in kinds[R]:
                t = tr[r["layer"]].astype(np.int64)
                live = t[:, ENTRY] > 0
                t0 = t[live, ENTRY].min()
                sel = live & ((t[:, FLAGS] & 3) == fl) & (t[:, STREAM] > 0)
                ends += ((t[sel, STREAM] - t0) * TICK_US).tolist()
            if ends:
                kind_lines.append(f"| {R} | {name} | {len(ends) / len(kinds[R]):.0f} | {statistics.median(ends):.1f} | "
                                  f"{max(ends):.1f} |")
    text = "\n".join(lines) + "\n\nPer layer kind (layers 1..L-1), mean us:\n\n" + "\n".join(summ) + "\n"
    text += "\nStreaming end by workgroup kind (us from the layer's first entry; WGs per layer):\n\n" + \
        "\n".join(kind_lines) + "\n"
    text += "\nCandidate resolver phases (median us from its start to the end of each phase):\n\n" + \
        resolver_table(tr, kinds)
    sp = ["| retrieval heads | head start | S staged | stream end |", "|---|---|---|---|"]
    for R in sorted(kinds):
        hs, st, se = [], [], []
        for r in kinds[R]:
            t = tr[r["layer"]].astype(np.int64)
            ok = (t[:, ENTRY] > 0) & (t[:, SSTAGED] > 0) & ((t[:, FLAGS] & 3) == 2)
            hs += ((t[ok, HEAD] - t[ok, ENTRY]) * TICK_US).tolist()
            st += ((t[ok, SSTAGED] - t[ok, ENTRY]) * TICK_US).tolist()
            se += ((t[ok, STREAM] - t[ok, ENTRY]) * TICK_US).tolist()
        if st:
            sp.append(f"| {R} | {statistics.median(hs):.2f} | {statistics.median(st):.2f} | {statistics.median(se):.2f} |")
    text += "\nGathered-rows workgroups (median us from entry):\n\n" + "\n".join(sp) + "\n"
    pro = ["| " + " | ".join(PRO_PHASES) + " | prologue done |", "|" + "---|" * (len(PRO_PHASES) + 1)]
    vals = [[] for _ in range(len(PRO_PHASES) + 1)]
    for r in rows:
        t = tr[r["layer"]].astype(np.int64)
        live = t[:, ENTRY] > 0
        for j, slot in enumerate([PRO0 + i for i in range(len(PRO_PHASES))] + [PROLOGUE]):
            ok = live & (t[:, slot] > 0)
            vals[j] += ((t[ok, slot] - t[ok, ENTRY]) * TICK_US).tolist()
    pro.append("| " + " | ".join(f"{statistics.median(v):.2f}" if v else "-" for v in vals) + " |")
    text += "\nPrologue phases (median us from each workgroup's entry, all layers):\n\n" + "\n".join(pro) + "\n"
    text += f"\nSum of layer spans {sum(r['exit'] for r in rows):.1f} us"
    if spans:
        text += f"; eager steps {', '.join(f'{s:.1f}' for s in spans)} us"
    return text + ".\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama3_128k")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--out", default=None)
    ap.add_argument("--raw", default=None, help="also save the raw stamps of the last repetition (.npy)")
    ap.add_argument("--from-raw", default=None, help="report on saved stamps (.npy) instead of running")
    ap.add_argument("--rule", default="topk", choices=["topk", "ratio", "threshold", "topp", "block"],
                    help="selection rule of the retrieval heads (as bench.py --rule)")
    ap.add_argument("--param", type=float, default=0.0, help="the rule's parameter (as bench.py --param)")
    a = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import numpy as np

    import synth
    if a.from_raw:
        w = synth.WORKLOADS[a.workload]
        tr = np.load(a.from_raw)
        print(report(tr, tr.shape[1], synth.roles(w), []), flush=True)
        return 0
    import torch

    import hybrid_head_sparse_amd as hhs

    if not hasattr(hhs.load(), "lychee_set_trace"):
        raise SystemExit("load the trace build: LYCHEE_LIB=hybrid_head_sparse_amd/liblychee_trace.so")
    w = synth.WORKLOADS[a.workload]
    roles = synth.roles(w)
    lens = synth.n_ctx(w)
    dev = []
    for l in range(w.layers):
        x = synth.layer_inputs(w, l, threads=min(16, os.cpu_count() or 1))
        conv = (lambda v: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()) if w.dtype == "bf16" \
            else (lambda v: torch.from_numpy(v).cuda())
        dev.append({key: conv(x[key]) for key in ("q", "k", "v")})
        print(f"[timeline] layer {l} resident", flush=True)
    B, Hq, Hkv, d, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k
    h = hhs.Handle(B, Hq, Hkv, d, w.max_ctx, k, w.dtype)
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    n_ctx = torch.from_numpy(lens).cuda()
    S = [torch.full((B, Hkv, k), -1, dtype=torch.int32, device="cuda") for _ in range(w.layers)]
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device="cuda") for _ in range(w.layers)]
    buf = torch.zeros(w.layers * grid * SLOTS, dtype=torch.int64, device="cuda")
    spans = []
    for rep in range(a.reps):
        buf.zero_()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for l in range(w.layers):
            h.set_trace(buf, l)
            x = dev[l]
            h.decode_layer(x["q"], x["k"], x["v"], roles[l], S[l - 1] if l else None, S[l], outs[l], n_ctx, k,
                           rule=a.rule, param=a.param)
        ev1.record()
        torch.cuda.synchronize()
        spans.append(ev0.elapsed_time(ev1) * 1e3)
        print(f"[timeline] rep {rep}: eager step {spans[-1]:.1f} us", flush=True)
    h.set_trace(None, 0)
    h.check_device_errors()
    tr = buf.cpu().numpy().view(np.uint64).reshape(w.layers, grid, SLOTS)
    if a.raw:
        np.save(a.raw, tr)
    text = report(tr, grid, roles, spans)
    print(text, flush=True)
    if a.out:
        cmd = "LYCHEE_LIB=hybrid_head_sparse_amd/liblychee_trace.so python3 -m hybrid_head_sparse_amd.timeline " + \
              " ".join(argv if argv is not None else sys.argv[1:])
        with open(a.out, "w") as f:
            f.write(f"# Phase timeline of the attention kernel, {w.name}\n\n")
            f.write(f"Command (repository root, one MI355X, after `python -m hybrid_head_sparse_amd.build --trace`):\n"
                    f"`{cmd.strip()}`\n\n")
            f.write("Times in us from each layer's first workgroup entry (s_memrealtime stamps of the trace build; "
                    "`gap` from the previous layer's last exit).  Columns: see the module docstring of "
                    "`hybrid_head_sparse_amd/timeline.py`.\n\n")
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
