"""Benchmark of the hybrid-head decode-attention step on one MI355X.

One step = every layer of the workload's decode step (layer 0 all retrieval,
S chained layer to layer through the C ABI), on seeded synthetic inputs
resident in HBM, captured once into a HIP graph and replayed.  Reported next
to the dense all-heads decode step on the same GPU and the CPU oracle.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload llama3_128k]
                    [--rule topk|ratio|threshold|topp|block --param P]

Prints one JSON line.  Algorithmic bytes per step (what the method must move;
workspace traffic excluded):
    sum_l [ R_l sum_b 2 n_b d s + (Hkv - R_l) sum_b (2 k_eff d s + 4 k_eff)
            + R_l sum_b 4 k_eff + B Hq d (s + 4) ]
with R_l retrieval KV heads in layer l, s bytes per cache element, k_eff =
min(k, n_b) (S_out aliases nothing extra: sparse rows are read once, written
once by the copy and counted as the 4 k_eff read).  Under the ratio and
threshold rules a sparse head gathers only the valid (not -1) entries of its
row, so its 2 k_eff d s term counts those instead.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

import synth

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
METRICS = {
    "llama3_128k": "decode-attn us/step + achieved HBM GB/s, Llama3-8B shape, 128K ctx, k=4096",
    "llama3_32k": "decode-attn us/step + achieved HBM GB/s, Llama3-8B shape, 32K ctx, k=4096",
    "llama3_ragged_b8": "decode-attn us/step + achieved HBM GB/s, Llama3-8B shape, batch 8, ragged 32K-64K ctx, k=2048",
    "qwen3_128k_k1024": "decode-attn us/step + achieved HBM GB/s, Qwen3-8B shape, 128K ctx, k=1024, tie groups",
    "qwen3_128k_k4096": "decode-attn us/step + achieved HBM GB/s, Qwen3-8B shape, 128K ctx, k=4096, tie groups",
}


def algorithmic_bytes(w: synth.Workload, roles: np.ndarray, lens: np.ndarray, valid=None):
    """Per-layer algorithmic bytes of the hybrid step and of the dense step.
    ``valid[l][b][g]``: valid entries of the S row a sparse head of layer l
    attends to (default k_eff)."""
    s = 2 if w.dtype == "bf16" else 4
    d = w.head_dim
    hyb, dense = [], []
    qo = w.batch * w.n_q_heads * d * (s + 4)
    for l in range(w.layers):
        R = int(roles[l].sum())
        tot = qo
        for b in range(w.batch):
            n = int(lens[b])
            ke = min(w.k, n)
            tot += R * (2 * n * d * s + 4 * ke)
            for g in range(w.n_kv_heads):
                if not roles[l][g]:
                    nv = ke if valid is None else int(valid[l][b][g])
                    tot += 2 * nv * d * s + 4 * ke
        hyb.append(tot)
        dense.append(qo + w.n_kv_heads * sum(2 * int(n) * d * s for n in lens))
    return hyb, dense


def load_inputs(w, roles, lens, threads: int):
    """Generate every layer on the host and move it to the GPU."""
    import torch
    dev = []
    for l in range(w.layers):
        x = synth.layer_inputs(w, l, threads=threads)
        if w.dtype == "bf16":
            conv = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            conv = lambda a: torch.from_numpy(a).cuda()
        dev.append({key: conv(x[key]) for key in ("q", "k", "v")})
        print(f"[bench] layer {l} resident", file=sys.stderr, flush=True)
    return dev


def host_info():
    """Logical CPUs the OS reports and the CPU model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline(w, roles, lens, dev, threads: int, reps: int = 3, rule="topk", param=0.0):
    """Time the oracle (as it stands) over the whole step: every layer, S
    chained, on `threads` host threads; each layer's inputs are copied back
    from the GPU untimed and the oracle runs `reps` times on them.  The step
    time of repetition r is the sum over layers of the r-th run; the median
    over repetitions is reported."""
    import oracle
    per = np.zeros((reps, w.layers))
    S = None
    for l in range(w.layers):
        x = {key: (t.view(torch_int16()).cpu().numpy().view(np.uint16) if w.dtype == "bf16" else t.cpu().numpy())
             for key, t in dev[l].items()}
        for r in range(reps):
            t0 = time.perf_counter()
            _, S_new, _ = oracle.layer(x["q"], x["k"], x["v"], roles[l], S, lens, w.k, threads=threads, rule=rule,
                                       param=param)
            per[r, l] = time.perf_counter() - t0
        S = S_new
        del x
        print(f"[bench] oracle layer {l}: {per[:, l].min() * 1e3:.1f} ms", file=sys.stderr, flush=True)
    steps = per.sum(axis=1)
    nproc, model = host_info()
    return {"value": float(np.median(steps)) * 1e6, "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": f"the whole {w.layers}-layer step (S chained), median of {reps} repetitions per layer "
                      f"summed per repetition (step times {', '.join(f'{v:.3f}' for v in steps)} s); inputs "
                      f"copied back from the GPU outside the timing",
            "nproc": nproc, "cpu_model": model,
            "threads_note": "the oracle's OpenMP threads: the host CPU share of one GPU (16), or every CPU if fewer"}


def torch_int16():
    import torch
    return torch.int16


def counters_traffic(workload: str):
    """HBM traffic of the attention kernel from the committed rocprofv3 counter
    summary of this workload, if it was taken on the current kernel source
    (else None)."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    from hybrid_head_sparse_amd.profiling import kernel_code_digest
    if c.get("kernel_code_sha256") != kernel_code_digest():
        return None
    return c.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_128k", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--cpu-reps", type=int, default=3, help="oracle repetitions per layer for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--rule", default="topk", choices=["topk", "ratio", "threshold", "topp", "block"],
                    help="selection rule of the retrieval heads (default: top-k, the headline)")
    ap.add_argument("--param", type=float, default=0.0, help="theta of the ratio rule, tau of the threshold rule, p of the Top-p rule, the block size of the block rule")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); the sharding plan is described in DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_head_sparse_amd as hhs

    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    roles = synth.roles(w)
    lens = synth.n_ctx(w)
    threads = min(16, os.cpu_count() or 1)
    dev = load_inputs(w, roles, lens, threads)
    B, Hq, Hkv, d, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k
    n_ctx = torch.from_numpy(lens).cuda()
    S = [torch.full((B, Hkv, k), -1, dtype=torch.int32, device="cuda") for _ in range(w.layers)]
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device="cuda") for _ in range(w.layers)]
    dense_outs = [torch.empty((B, Hq, d), dtype=torch.float32, device="cuda") for _ in range(w.layers)]
    h = hhs.Handle(B, Hq, Hkv, d, w.max_ctx, k, w.dtype)

    def step():
        for l in range(w.layers):
            x = dev[l]
            h.decode_layer(x["q"], x["k"], x["v"], roles[l], S[l - 1] if l else None, S[l], outs[l], n_ctx, k,
                           rule=args.rule, param=args.param)

    def dense_step():
        for l in range(w.layers):
            x = dev[l]
            h.dense_decode_layer(x["q"], x["k"], x["v"], dense_outs[l], n_ctx)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                               # warm the kernels on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            h.set_stream(torch.cuda.current_stream())
            fn()
        h.set_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return g

    def timed(g, steps, warmup):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        total_ms = t0.elapsed_time(t1)
        # per-replay distribution in a second pass
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) for a, b in evs)
        return total_ms / steps, per

    # eager reference run, then the graph; every replay must reproduce it bitwise
    step()
    torch.cuda.synchronize()
    h.check_device_errors()
    ref_out = [o.clone() for o in outs]
    ref_S = [s_.clone() for s_ in S]
    g_step = capture(step)
    ms_per_step, per = timed(g_step, args.steps, args.warmup)
    for l in range(w.layers):
        assert torch.equal(outs[l], ref_out[l]) and torch.equal(S[l], ref_S[l]), f"graph replay differs at layer {l}"

    # attention-kernel launch durations (HIP events on the handle's stream, eager steps)
    att_ms = [[] for _ in range(w.layers)]
    ev_pairs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(w.layers)] for _ in range(args.steps)]
    for rep in ev_pairs:
        for a, b in rep:
            a.record()
            b.record()
    torch.cuda.synchronize()
    for rep in ev_pairs:
        for l in range(w.layers):
            a, b = rep[l]
            h.set_profile_events(a, b)
            x = dev[l]
            h.decode_layer(x["q"], x["k"], x["v"], roles[l], S[l - 1] if l else None, S[l], outs[l], n_ctx, k,
                           rule=args.rule, param=args.param)
    h.set_profile_events(None, None)
    torch.cuda.synchronize()
    for rep in ev_pairs:
        for l in range(w.layers):
            a, b = rep[l]
            att_ms[l].append(a.elapsed_time(b))

    valid = None
    kept = [int((ref_S[l][:, g] != -1).sum()) for l in range(w.layers) for g in range(Hkv) if roles[l][g]]
    if args.rule != "topk":
        valid = [np.zeros((B, Hkv), np.int64)] + [(ref_S[l - 1] != -1).sum(dim=2).cpu().numpy()
                                                  for l in range(1, w.layers)]
    hyb_bytes, dense_bytes = algorithmic_bytes(w, roles, lens, valid)
    step_bytes = sum(hyb_bytes)
    att_mean = [statistics.mean(v) for v in att_ms]
    # The roofline's launch time: the graph-timed step (HIP events on the
    # replay stream) over its launches -- one attention kernel per layer.  The
    # per-launch event times of eager calls add the launch overhead of an
    # eager call and are reported beside it.
    att_all_bytes = sum(hyb_bytes)                    # per step, over all attention launches
    avg_launch_ms = ms_per_step / w.layers
    achieved = att_all_bytes / (ms_per_step * 1e-3) / 1e9
    l0_ms = att_mean[0]
    l0_achieved = hyb_bytes[0] / (l0_ms * 1e-3) / 1e9

    dense_res = None
    dense_l0 = None
    if not args.no_dense:
        dense_step()
        torch.cuda.synchronize()
        g_dense = capture(dense_step)
        dense_ms, dense_per = timed(g_dense, args.steps, args.warmup)
        dense_res = {"us_per_step": dense_ms * 1e3, "p10_us": dense_per[len(dense_per) // 10] * 1e3,
                     "p90_us": dense_per[(9 * len(dense_per)) // 10] * 1e3,
                     "algorithmic_bytes": sum(dense_bytes),
                     "achieved_GBps": sum(dense_bytes) / (dense_ms * 1e-3) / 1e9}
        # the same kernel without selection on layer 0's inputs (HIP events on the handle's stream)
        d0_ms = []
        d0_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a_, b_ in d0_ev:
            a_.record()
            b_.record()
        torch.cuda.synchronize()
        for a_, b_ in d0_ev:
            h.set_profile_events(a_, b_)
            x = dev[0]
            h.dense_decode_layer(x["q"], x["k"], x["v"], dense_outs[0], n_ctx)
        h.set_profile_events(None, None)
        torch.cuda.synchronize()
        d0_ms = statistics.mean(a_.elapsed_time(b_) for a_, b_ in d0_ev)
        dense_l0 = {"kernel": "attend_kernel (dense: the retrieval path without selection), layer 0 inputs",
                    "achieved": dense_bytes[0] / (d0_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": dense_bytes[0] / (d0_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "bytes_per_launch": dense_bytes[0],
                    "avg_launch_us": d0_ms * 1e3}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, roles, lens, dev, threads, args.cpu_reps, args.rule, args.param)

    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    n_retr = int(roles.sum())
    result = {
        "metric": METRICS.get(w.name, f"decode-attn us/step + achieved HBM GB/s, {w.name}"),
        "value": ms_per_step * 1e3,
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "layers": w.layers, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": d, "n_ctx": [int(v) for v in lens] if B > 1 else int(lens[0]), "k": k,
                   "kv_cache": w.dtype, "retrieval_kv_head_instances": n_retr,
                   "sparse_kv_head_instances": w.layers * Hkv - n_retr,
                   "selection_rule": args.rule if args.rule == "topk" else f"{args.rule}({args.param:g})"},
        "mean_selected_per_retrieval_head": statistics.mean(kept) / B,
        "achieved_GBps": step_gbps,
        "frac_of_hbm_peak": step_gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "p10_us": per[len(per) // 10] * 1e3,
        "p50_us": per[len(per) // 2] * 1e3,
        "p90_us": per[(9 * len(per)) // 10] * 1e3,
        "dense_baseline": dense_res,
        "speedup_vs_dense": (dense_res["us_per_step"] / (ms_per_step * 1e3)) if dense_res else None,
        "roofline": {"kernel": "attend_kernel (hybrid, all launches of the step)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counters_traffic(w.name) if args.rule == "topk" else None,
                     "bytes_per_launch": att_all_bytes / w.layers, "avg_launch_us": avg_launch_ms * 1e3,
                     "avg_launch_source": "graph-timed step / launches per step",
                     "eager_event_launch_us": statistics.mean(att_mean) * 1e3},
        "roofline_all_retrieval_layer": {"kernel": "attend_kernel (hybrid), layer 0: every KV head retrieval",
                                         "achieved": l0_achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                         "frac": l0_achieved / HBM_PEAK_GBPS, "bytes_per_launch": hyb_bytes[0],
                                         "avg_launch_us": l0_ms * 1e3},
        "roofline_all_retrieval_layer_without_selection": dense_l0,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
