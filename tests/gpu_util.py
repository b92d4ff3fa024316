"""Helpers for the GPU tests: move seeded inputs to the device, run layers
through the C ABI binding, and plant boundary tie groups (via the oracle)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def make_handle(w: synth.Workload):
    import hybrid_head_sparse_amd as hhs
    return hhs.Handle(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_ctx, w.k, w.dtype)


def run_layer(handle, x, role, S_in_dev, n_ctx_dev, k, *, S_out_dev=None, rule="topk", param=0.0):
    """Returns (out_host, S_out_host, S_out_dev)."""
    import torch
    d = handle.dims
    dtype = "bf16" if d.dtype == 1 else "f32"
    q = to_device(x["q"], dtype)
    kc = to_device(x["k"], dtype)
    vc = to_device(x["v"], dtype)
    if S_out_dev is None:
        S_out_dev = torch.full((d.batch, d.n_kv_heads, k), -7, dtype=torch.int32, device="cuda")
    out = torch.full((d.batch, d.n_q_heads, d.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    handle.decode_layer(q, kc, vc, role, S_in_dev, S_out_dev, out, n_ctx_dev, k, rule=rule, param=param)
    torch.cuda.synchronize()
    res = out.cpu().numpy(), S_out_dev.cpu().numpy().copy(), S_out_dev
    del q, kc, vc
    return res


def plant_boundary_groups(w: synth.Workload, x: dict, k: int, ties: dict, heads=None, layer: int = 0):
    """Copy the oracle k-th-ranked K row of each KV head in ``heads`` (default:
    all) into 7 lower-ranked positions, some below and some above its index,
    so an exact tie group straddles the top-k boundary.  Mutates x["k"] and
    appends the groups to ``ties``."""
    lens = synth.n_ctx(w)
    heads = list(range(w.n_kv_heads)) if heads is None else [int(g) for g in heads]
    if not heads:
        return x
    G = w.group
    hq = [g * G + i for g in heads for i in range(G)]
    ones = np.ones(len(heads), np.uint8)
    _, S, scores = oracle.layer(np.ascontiguousarray(x["q"][:, hq]), np.ascontiguousarray(x["k"][:, heads]),
                                np.ascontiguousarray(x["v"][:, heads]), ones, None, lens, k, want_scores=True)
    rng = np.random.default_rng([w.seed, 4242, layer])
    for b in range(w.batch):
        n = int(lens[b])
        ke = min(k, n)
        if ke >= n:
            continue
        for gi, g in enumerate(heads):
            O = S[b, gi, :ke]
            s = scores[b, gi, :n]
            order = sorted(O.tolist(), key=lambda j: (-s[j], j))
            jk = order[-1]
            busy = np.zeros(n, bool)
            busy[O] = True
            for grp in ties.get((b, g), []):
                busy[np.asarray(grp)] = True
            low = np.nonzero(~busy[:jk] & (s[:jk] < s[jk]))[0]
            high = jk + 1 + np.nonzero(~busy[jk + 1:] & (s[jk + 1:] < s[jk]))[0]
            pick = np.concatenate([rng.choice(low, size=min(3, low.size), replace=False),
                                   rng.choice(high, size=min(7 - min(3, low.size), high.size), replace=False)])
            x["k"][b, g, pick] = x["k"][b, g, jk]
            ties[(b, g)] = list(ties.get((b, g), [])) + [np.sort(np.concatenate([[jk], pick]))]
    return x
