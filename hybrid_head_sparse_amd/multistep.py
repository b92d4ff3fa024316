"""Measurement of the multi-step loop's kernels on one GPU.

The loop around the hybrid step (Algorithm 1 of the LycheeDecode digest,
section 3.4; Cache Correction, section 4.2.2): every decoded token appends its
K and V rows to each layer's cache, and every 32 tokens a dense causal
attention over the last 32 positions refreshes them.  This times, on the
Llama3-8B attention shape (32 query / 8 KV heads, d = 128, bf16 cache) at one
context length:

  * the correction attention (T = 32 positions, all query heads) against its
    roofline: algorithmic bytes = every cache row of K and V once (2 n d 2
    bytes per KV head) plus q and out; flops = 4 d per (query row, visible
    key) pair, i.e. 4 d sum_t (n - T + t + 1) per query head;
  * the cache append (one token, every KV head);
  * the hybrid layer at the same length, for the per-token cost of the loop:
    hybrid + append + correction / 32.

Each is captured --reps times back to back in a HIP graph and the replay is
timed with events (median of 3).

    python3 -m hybrid_head_sparse_amd.multistep [--ctx 131072] [--reps 10]
        [--out profiles/correction_llama3_128k.md]
"""
from __future__ import annotations

import argparse
import math
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HQ, HKV, D, T = 32, 8, 128, 32
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def correction_cost(n: int, B: int = 1):
    """(algorithmic bytes, flops) of one correction launch."""
    kv = B * HKV * 2 * n * D * 2
    qo = B * T * HQ * D * (2 + 4)
    visible = sum(n - T + t + 1 for t in range(T))
    flops = B * HQ * 4 * D * visible
    return kv + qo, flops


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--ctx", type=int, default=131072)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--k", type=int, default=4096)
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    sys.path.insert(0, ROOT)
    import torch
    import hybrid_head_sparse_amd as hhs

    n = a.ctx
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    inv = 1.0 / math.sqrt(D)
    kc = (torch.randn(1, HKV, n, D, generator=gen, device="cuda") * inv).to(torch.bfloat16)
    vc = torch.randn(1, HKV, n, D, generator=gen, device="cuda").to(torch.bfloat16)
    qc = (torch.randn(1, T, HQ, D, generator=gen, device="cuda") * inv).to(torch.bfloat16)
    q1 = (torch.randn(1, HQ, D, generator=gen, device="cuda") * inv).to(torch.bfloat16)
    kn = (torch.randn(1, HKV, D, generator=gen, device="cuda") * inv).to(torch.bfloat16)
    vn = torch.randn(1, HKV, D, generator=gen, device="cuda").to(torch.bfloat16)
    h = hhs.Handle(1, HQ, HKV, D, n, a.k, "bf16")
    n_full = torch.full((1,), n, dtype=torch.int32, device="cuda")
    n_app = torch.full((1,), n - a.reps - 1, dtype=torch.int32, device="cuda")
    out_c = torch.empty((1, T, HQ, D), dtype=torch.float32, device="cuda")
    out_1 = torch.empty((1, HQ, D), dtype=torch.float32, device="cuda")
    S = torch.empty((1, HKV, a.k), dtype=torch.int32, device="cuda")

    def timed(fn, reset=None):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            h.set_stream(torch.cuda.current_stream())
            for _ in range(a.reps):
                fn()
        h.set_stream(torch.cuda.current_stream())
        t = []
        for _ in range(3):
            if reset:
                reset()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) / a.reps * 1e3)
        return statistics.median(t)

    us_corr = timed(lambda: h.correction_attention(qc, kc, vc, n_full, out_c))
    us_app = timed(lambda: h.kv_append(kn, vn, kc, vc, n_app), reset=lambda: n_app.fill_(n - a.reps - 1))
    us_layer = timed(lambda: h.decode_layer(q1, kc, vc, [1] * HKV, None, S, out_1, n_full, a.k))
    h.check_device_errors()
    bytes_c, flops_c = correction_cost(n)
    gbps = bytes_c / (us_corr * 1e-6) / 1e9
    tflops = flops_c / (us_corr * 1e-6) / 1e12
    per_token = us_layer + us_app + us_corr / 32.0
    lines = [
        f"correction attention (T = {T}, {HQ}/{HKV} heads, n = {n}): {us_corr:.1f} us, "
        f"{gbps:.0f} GB/s of {bytes_c / 1e6:.1f} MB ({gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s), "
        f"{tflops:.0f} TFLOP/s of {flops_c / 1e9:.1f} GFLOP ({tflops / MFMA_BF16_PEAK_TFLOPS:.1%} of 2.5 PFLOP/s)",
        f"cache append (one token, {HKV} KV heads): {us_app:.2f} us",
        f"hybrid layer, all retrieval, k = {a.k}: {us_layer:.1f} us",
        f"per token and layer of the loop (hybrid + append + correction / 32): {per_token:.1f} us",
    ]
    for line in lines:
        print("[multistep] " + line, flush=True)
    if a.out:
        cmd = "python3 -m hybrid_head_sparse_amd.multistep " + " ".join(argv if argv is not None else sys.argv[1:])
        with open(a.out, "w") as f:
            f.write("# The multi-step loop's kernels, Llama3-8B attention shape\n\n")
            f.write(f"Command (repository root, one MI355X): `{cmd.strip()}`\n\n")
            f.write("Random bf16 cache (q, K ~ N(0,1)/sqrt(d), V ~ N(0,1)); each kernel captured "
                    f"{a.reps} times back to back in a HIP graph, replay timed with events (median of 3).\n\n")
            for line in lines:
                f.write(f"- {line}\n")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
